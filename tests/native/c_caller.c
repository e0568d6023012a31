/*
 * A plain C99 caller of libattnres, for the tests: it includes attnres.h as C,
 * links against libattnres.so and uses only the C ABI and the HIP runtime's C
 * API.
 *
 *   c_caller abi            no GPU needed: version, status strings, and calls
 *                           that must be rejected before any HIP call
 *   c_caller run IN OUT     one fused call on the current device: IN holds
 *                           the int64 header {M, H, N, has_add2}, eps as a
 *                           float, then the bf16 words of prefix, add, [add2],
 *                           N snapshots ([M,H] each), query and gamma ([H]);
 *                           OUT receives out_prefix and out_norm ([M,H] each)
 */
#include "attnres.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CHECK(cond, ...)                                                                                   \
    do {                                                                                                   \
        if (!(cond)) {                                                                                     \
            fprintf(stderr, __VA_ARGS__);                                                                  \
            fprintf(stderr, "\n");                                                                         \
            return 1;                                                                                      \
        }                                                                                                  \
    } while (0)

static int abi_checks(void)
{
    printf("version %d\n", attnres_version());
    CHECK(attnres_version() > 0, "bad version");
    CHECK(strlen(attnres_status_string(ATTNRES_EALIAS)) > 0, "empty status string");
    CHECK(strstr(attnres_status_string(ATTNRES_ENOINIT), "attnres_init") != NULL, "ENOINIT status string");
    CHECK(strstr(attnres_status_string(ATTNRES_EUNSUPPORTED), "64") != NULL, "EUNSUPPORTED status string");
    /* rejected before any HIP call: no GPU is touched */
    CHECK(attnres_add_rmsnorm_fwd(NULL, NULL, NULL, NULL, 65, NULL, NULL, 1e-6f, 1, 7168, NULL, NULL, 0) ==
              ATTNRES_EUNSUPPORTED,
          "65 snapshots must be unsupported");
    CHECK(attnres_add_rmsnorm_fwd(NULL, NULL, NULL, NULL, 1, NULL, NULL, 1e-6f, 1, 7168, NULL, NULL, 0) ==
              ATTNRES_EINVAL,
          "null pointers must be invalid");
    CHECK(attnres_add_rmsnorm_fwd(NULL, NULL, NULL, NULL, 0, NULL, NULL, -1.f, 0, 7168, NULL, NULL, 0) ==
              ATTNRES_EINVAL,
          "negative eps must be invalid");
    CHECK(attnres_add_rmsnorm_fwd(NULL, NULL, NULL, NULL, 0, NULL, NULL, 1e-6f, 0, 7168, NULL, NULL, 0) ==
              ATTNRES_OK,
          "an empty batch must succeed");
    int v = 0, c = 0, t = 0;
    CHECK(attnres_plan(256, 12, 7168, &v, &c, &t) == ATTNRES_OK && v == 1, "plan at M=256 must be one workgroup per token");
    printf("abi ok\n");
    return 0;
}

static int read_exact(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

static int run(const char* in_path, const char* out_path)
{
    FILE* f = fopen(in_path, "rb");
    CHECK(f, "cannot open %s", in_path);
    int64_t hdr[4];
    float eps;
    CHECK(read_exact(f, hdr, sizeof hdr) && read_exact(f, &eps, sizeof eps), "short header");
    const int64_t M = hdr[0], H = hdr[1];
    const int N = (int)hdr[2], has_add2 = (int)hdr[3];
    CHECK(M > 0 && H > 0 && N >= 0 && N <= ATTNRES_MAX_SNAPSHOTS, "bad header");
    const size_t row = (size_t)M * (size_t)H * 2u, vec = (size_t)H * 2u;
    const int nrows = 2 + has_add2 + N; /* prefix, add, [add2], snapshots */
    void* host = malloc(row * (size_t)nrows + 2 * vec);
    CHECK(host, "out of host memory");
    CHECK(read_exact(f, host, row * (size_t)nrows + 2 * vec), "short input");
    fclose(f);

    void* dev_rows[2 + 1 + ATTNRES_MAX_SNAPSHOTS];
    void *dq, *dg, *dop, *don;
    for (int i = 0; i < nrows; ++i) {
        CHECK(hipMalloc(&dev_rows[i], row) == hipSuccess, "hipMalloc");
        CHECK(hipMemcpy(dev_rows[i], (char*)host + row * (size_t)i, row, hipMemcpyHostToDevice) == hipSuccess,
              "hipMemcpy");
    }
    CHECK(hipMalloc(&dq, vec) == hipSuccess && hipMalloc(&dg, vec) == hipSuccess, "hipMalloc");
    CHECK(hipMemcpy(dq, (char*)host + row * (size_t)nrows, vec, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(dg, (char*)host + row * (size_t)nrows + vec, vec, hipMemcpyHostToDevice) == hipSuccess,
          "hipMemcpy");
    CHECK(hipMalloc(&dop, row) == hipSuccess && hipMalloc(&don, row) == hipSuccess, "hipMalloc");

    const void* snaps[ATTNRES_MAX_SNAPSHOTS + 1];
    for (int s = 0; s < N; ++s)
        snaps[s] = dev_rows[2 + has_add2 + s];
    /* before attnres_init the call launches nothing and says why */
    int rc = attnres_add_rmsnorm_fwd(dev_rows[0], dev_rows[1], has_add2 ? dev_rows[2] : NULL, N ? snaps : NULL, N,
                                     dq, dg, eps, M, H, dop, don, 0);
    CHECK(rc == ATTNRES_ENOINIT, "call before attnres_init -> %d (%s)", rc, attnres_status_string(rc));
    CHECK(attnres_init() == ATTNRES_OK && attnres_init() == ATTNRES_OK, "attnres_init");
    rc = attnres_add_rmsnorm_fwd(dev_rows[0], dev_rows[1], has_add2 ? dev_rows[2] : NULL, N ? snaps : NULL, N, dq,
                                 dg, eps, M, H, dop, don, 0);
    CHECK(rc == ATTNRES_OK, "attnres_add_rmsnorm_fwd -> %d (%s)", rc, attnres_status_string(rc));
    CHECK(hipDeviceSynchronize() == hipSuccess, "hipDeviceSynchronize");

    void* out = malloc(2 * row);
    CHECK(out, "out of host memory");
    CHECK(hipMemcpy(out, dop, row, hipMemcpyDeviceToHost) == hipSuccess &&
              hipMemcpy((char*)out + row, don, row, hipMemcpyDeviceToHost) == hipSuccess,
          "hipMemcpy");
    FILE* o = fopen(out_path, "wb");
    CHECK(o && fwrite(out, 1, 2 * row, o) == 2 * row, "cannot write %s", out_path);
    fclose(o);
    for (int i = 0; i < nrows; ++i)
        (void)hipFree(dev_rows[i]);
    (void)hipFree(dq);
    (void)hipFree(dg);
    (void)hipFree(dop);
    (void)hipFree(don);
    free(host);
    free(out);
    printf("run ok: M=%lld H=%lld N=%d add2=%d\n", (long long)M, (long long)H, N, has_add2);
    return 0;
}

int main(int argc, char** argv)
{
    if (argc == 2 && strcmp(argv[1], "abi") == 0)
        return abi_checks();
    if (argc == 4 && strcmp(argv[1], "run") == 0)
        return run(argv[2], argv[3]);
    fprintf(stderr, "usage: c_caller abi | c_caller run IN OUT\n");
    return 2;
}
