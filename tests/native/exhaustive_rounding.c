/*
 * Exhaustive pins for the oracle's rounding primitives (test code, CPU only).
 *
 * Loads an oracle library with dlopen and compares, over every input:
 *
 *   mode "round": oracle_round_bf16((double)f) for all 2^32 binary32 bit
 *                 patterns f, against rounding by definition on the bit
 *                 pattern (truncate to the upper 16 bits, then step up if the
 *                 dropped half exceeds one half, or equals it and the kept
 *                 pattern is odd).
 *   mode "add":   oracle_bf16_add(a, b) for all 2^32 pairs of bf16 patterns,
 *                 against the exact sum formed in integers (both operands
 *                 scaled to a common power of two) rounded once to the nearest
 *                 bf16, ties to even, with gradual underflow.  This is the
 *                 value two bf16 tensor additions must produce when they are
 *                 correctly rounded (page "Kimi K3: fold the MoE-tail
 *                 additions into the next attention-residual", section Op).
 *
 * Usage: exhaustive_rounding <liboracle.so> round|add <threads> [max_report]
 * Prints "mismatches <count>" and exits 0 when the count is zero.
 */
#include <dlfcn.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef uint16_t (*round_fn)(double);
typedef uint16_t (*add_fn)(uint16_t, uint16_t);

static round_fn g_round;
static add_fn g_add;
static int g_mode; /* 0 round, 1 add */
static int g_threads;
static long g_max_report = 8;
static pthread_mutex_t g_lock = PTHREAD_MUTEX_INITIALIZER;
static long g_reported;

static int is_nan16(uint16_t b) { return ((b >> 7) & 0xFF) == 0xFF && (b & 0x7F); }

/* rounding by definition on the binary32 pattern */
static uint16_t round_bits(uint32_t u)
{
    uint32_t keep = u >> 16, drop = u & 0xFFFFu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u; /* carries into the exponent field; 0x7F7F+1 = Inf */
    return (uint16_t)keep;
}

/* exact bf16 + bf16, rounded once; returns 0xFFFF for "any NaN" */
static uint16_t exact_add(uint16_t a, uint16_t b)
{
    int sa = a >> 15, sb = b >> 15;
    int ea = (a >> 7) & 0xFF, eb = (b >> 7) & 0xFF;
    int fa = a & 0x7F, fb = b & 0x7F;
    if (is_nan16(a) || is_nan16(b))
        return 0xFFFF;
    if (ea == 0xFF || eb == 0xFF) {
        if (ea == 0xFF && eb == 0xFF && sa != sb)
            return 0xFFFF;
        return ea == 0xFF ? a : b;
    }
    /* value = (-1)^s * mant * 2^exp */
    int64_t ma = ea ? 128 + fa : fa, mb = eb ? 128 + fb : fb;
    int xa = ea ? ea - 134 : -133, xb = eb ? eb - 134 : -133;
    if (ma == 0 && mb == 0)
        return (sa && sb) ? 0x8000 : 0x0000;
    int E = xa < xb ? xa : xb;
    int da = xa - E, db = xb - E;
    if (da > 60 && mb != 0 && ma != 0)
        return a; /* |b| is far below a quarter ulp of a */
    if (db > 60 && ma != 0 && mb != 0)
        return b;
    if (da > 60 || db > 60)
        return ma ? a : b;
    __int128 A = (__int128)(sa ? -ma : ma) << da;
    __int128 B = (__int128)(sb ? -mb : mb) << db;
    __int128 S = A + B;
    if (S == 0)
        return 0x0000; /* exact cancellation rounds to +0 */
    int neg = S < 0;
    unsigned __int128 mag = (unsigned __int128)(neg ? -S : S);
    int L = 0;
    for (unsigned __int128 t = mag; t; t >>= 1)
        ++L;
    int p = E + L - 1;                  /* value in [2^p, 2^(p+1)) */
    int Q = p >= -126 ? p - 7 : -133;   /* exponent of the bf16 quantum */
    int shift = Q - E;
    unsigned __int128 q;
    if (shift <= 0) {
        q = mag << (-shift);
    } else {
        q = mag >> shift;
        unsigned __int128 rem = mag - (q << shift);
        unsigned __int128 half = (unsigned __int128)1 << (shift - 1);
        if (rem > half || (rem == half && (q & 1)))
            q += 1;
    }
    while (q >= 256) {
        q >>= 1;
        Q += 1;
    }
    uint16_t bits;
    if (q < 128) {
        bits = (uint16_t)q; /* subnormal (Q == -133) */
    } else {
        int e = Q + 134;
        if (e >= 255)
            bits = 0x7F80;
        else
            bits = (uint16_t)((e << 7) | (int)(q - 128));
    }
    return (uint16_t)(bits | (neg ? 0x8000 : 0));
}

typedef struct {
    uint64_t lo, hi, bad;
} job_t;

static void report(uint64_t i, uint16_t want, uint16_t got)
{
    pthread_mutex_lock(&g_lock);
    if (g_reported < g_max_report) {
        if (g_mode == 0)
            printf("round f32=0x%08x want=0x%04x got=0x%04x\n", (unsigned)i, want, got);
        else
            printf("add a=0x%04x b=0x%04x want=0x%04x got=0x%04x\n",
                   (unsigned)(i >> 16), (unsigned)(i & 0xFFFF), want, got);
        ++g_reported;
    }
    pthread_mutex_unlock(&g_lock);
}

static void* worker(void* arg)
{
    job_t* j = (job_t*)arg;
    for (uint64_t i = j->lo; i < j->hi; ++i) {
        uint16_t want, got;
        if (g_mode == 0) {
            uint32_t u = (uint32_t)i;
            float f;
            memcpy(&f, &u, 4);
            if (((u >> 23) & 0xFF) == 0xFF && (u & 0x7FFFFF)) {
                got = g_round((double)f);
                if (!is_nan16(got)) {
                    ++j->bad;
                    report(i, 0x7FC0, got);
                }
                continue;
            }
            want = round_bits(u);
            got = g_round((double)f);
        } else {
            uint16_t a = (uint16_t)(i >> 16), b = (uint16_t)(i & 0xFFFF);
            want = exact_add(a, b);
            got = g_add(a, b);
            if (want == 0xFFFF) {
                if (!is_nan16(got)) {
                    ++j->bad;
                    report(i, want, got);
                }
                continue;
            }
        }
        if (want != got) {
            ++j->bad;
            report(i, want, got);
            if (j->bad > 1000000)
                break;
        }
    }
    return NULL;
}

int main(int argc, char** argv)
{
    if (argc < 4) {
        fprintf(stderr, "usage: %s lib round|add threads [max_report]\n", argv[0]);
        return 2;
    }
    void* h = dlopen(argv[1], RTLD_NOW | RTLD_LOCAL);
    if (!h) {
        fprintf(stderr, "dlopen: %s\n", dlerror());
        return 2;
    }
    g_round = (round_fn)dlsym(h, "oracle_round_bf16");
    g_add = (add_fn)dlsym(h, "oracle_bf16_add");
    if (!g_round || !g_add) {
        fprintf(stderr, "missing symbols\n");
        return 2;
    }
    g_mode = strcmp(argv[2], "add") == 0 ? 1 : 0;
    g_threads = atoi(argv[3]);
    if (g_threads < 1)
        g_threads = 1;
    if (argc > 4)
        g_max_report = atol(argv[4]);
    uint64_t total = (uint64_t)1 << 32;
    pthread_t* th = (pthread_t*)calloc((size_t)g_threads, sizeof(pthread_t));
    job_t* jobs = (job_t*)calloc((size_t)g_threads, sizeof(job_t));
    for (int t = 0; t < g_threads; ++t) {
        jobs[t].lo = total * (uint64_t)t / (uint64_t)g_threads;
        jobs[t].hi = total * (uint64_t)(t + 1) / (uint64_t)g_threads;
        pthread_create(&th[t], NULL, worker, &jobs[t]);
    }
    uint64_t bad = 0;
    for (int t = 0; t < g_threads; ++t) {
        pthread_join(th[t], NULL);
        bad += jobs[t].bad;
    }
    printf("mismatches %llu\n", (unsigned long long)bad);
    return bad ? 1 : 0;
}
