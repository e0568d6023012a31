#!/usr/bin/env python3
"""Benchmark of the fused AttnRes combine + RMSNorm decode step on one MI355X.

Workload (the bandwidth configuration): the 25-layer decoder chain of the fused
op, 256 tokens, H = 7168, bf16, the snapshot bank growing by one entry every
two layers up to 12 sources (N = 1,1,2,2,...,11,11,12,12,12), each layer's
MoE tail (routed, shared) folded into the call.  A step is one pass of the
whole chain.  To measure HBM and not the 256 MB Infinity Cache, the step runs
16 independent 256-token chains interleaved layer by layer (16 micro-batches,
about 6 GB of distinct buffers): between two calls of one chain, more than
256 MB of other data streams through the caches.

value = algorithmic bytes of the step / step time (GB/s, HIP-graph replay,
inputs resident in HBM).  Algorithmic bytes of one call with N sources:
14336 * M * (5 + N) + 28672 (reads prefix, add, add2, N snapshots; writes
out_prefix, out_norm; plus query and gamma).

Also reported on the same JSON line:
  roofline      the fused kernel's achieved GB/s: algorithmic bytes per launch
                / average launch duration, the latter from the HIP events that
                bracket the timed region (graph replays holding only the fused
                launches); per-layer times from events around each layer's
                group of launches (queue pre-filled by a sleep kernel, so the
                events bracket back-to-back kernels); against 8 TB/s; traffic
                from the committed rocprofv3 PMC summary when it was taken on
                the current kernel source
  cpu_baseline  the CPU oracle on the same chain (all 256 tokens, one
                micro-batch), parallel over token blocks
  cpu_latency   the CPU oracle on each small named call (median of 5), one
                thread and token-parallel
  latency_us    per-call time of the small named calls with inputs cold in
                HBM (>= 1.1 GB of distinct buffer sets): graph replay, and
                eager back-to-back launches; plus a warm figure (16 sets,
                resident in the Infinity Cache)
  fold          the pages' comparison: fused call with add2 vs the unfused
                route (standalone add, then the fused call without add2)
  fold_per_config  the same comparison per small named call and per kernel
                variant: fused with add2, fused with the pre-summed addend,
                standalone add
  tap           cost of the optional pre-norm mixture output (the capture tap)
                at M = 256 and at one token, N = 12
  prefill       prefill-sized calls (M = 1,024 and 4,096, N = 12): µs per call
                and the fraction of 8 TB/s

parity_after_timing: after the timed replays, every micro-batch instance's
outputs on sampled token rows of every layer against the oracle chain, and
the instances against each other bit for bit.

--mode grid prints µs per call and GB/s over a grid of token and source counts
at H = 7168 ("grid") and at one tensor-parallel rank's 896 columns of it
("tp8_share").  Every timing follows a parity check against the CPU oracle.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of ~8 TB/s) at M tokens × N sources, H=7168"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attnres_fwd_chain_m256_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "attention_residual_rmsnorm_amd", "csrc", n)
                  for n in ("attnres.hip", "attnres_device.hpp", "attnres_host.cpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_only(text: str) -> str:
    """C++ source with comments removed and runs of whitespace collapsed to one
    space (string and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """First 16 hex digits of the sha256 of the kernel sources' code (comments
    and layout do not count): identifies the kernels a stored profile was
    taken on."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def call_bytes(M, H, N, add2=True):
    return 2 * H * (M * (4 + int(add2) + N) + 2)


def dev(bits):
    """numpy bf16 bit patterns -> bfloat16 device tensor."""
    import numpy as np
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def host(t):
    import numpy as np
    import torch

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def norm_ok(got, want):
    """out_norm within 2 bf16 ulps (monotone integer distance) or 1e-2 absolute, no NaN."""
    import numpy as np

    from attention_residual_rmsnorm_amd.workloads import bf16_bits_to_f32

    def ordv(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    ulps = np.abs(ordv(got) - ordv(want))
    diff = np.abs(bf16_bits_to_f32(got).astype(np.float64) - bf16_bits_to_f32(want))
    return bool(np.all(((ulps <= 2) | (diff <= 1e-2)) & ~nan(got) & ~nan(want)))


# --------------------------------------------------------------------------
# raw launches (precomputed ctypes arguments keep host overhead low)

class Launcher:
    def __init__(self):
        import attention_residual_rmsnorm_amd as ar

        self.ar = ar
        self.lib = ar.library()
        self.fwd = self.lib.attnres_add_rmsnorm_fwd
        self.fwd_mix = self.lib.attnres_add_rmsnorm_mix_fwd
        self.add = self.lib.attnres_bf16_add
        self._keep = []

    def fused_args(self, prefix, add, add2, snaps, query, gamma, eps, out_prefix, out_norm):
        vp = ctypes.c_void_p
        n = len(snaps)
        arr = (vp * max(n, 1))(*[s.data_ptr() for s in snaps])
        self._keep.append(arr)
        M, H = prefix.shape
        return (prefix.data_ptr(), add.data_ptr(), None if add2 is None else add2.data_ptr(),
                arr if n else None, n, query.data_ptr(), gamma.data_ptr(), ctypes.c_float(eps), M, H,
                out_prefix.data_ptr(), out_norm.data_ptr())

    def run_fused(self, args, stream):
        rc = self.fwd(*args, stream)
        if rc != 0:
            raise RuntimeError("attnres_add_rmsnorm_fwd -> %d" % rc)

    def run_mix(self, args, out_mix, stream):
        rc = self.fwd_mix(*args, out_mix, stream)
        if rc != 0:
            raise RuntimeError("attnres_add_rmsnorm_mix_fwd -> %d" % rc)

    def run_add(self, a, b, out, stream):
        rc = self.add(a.data_ptr(), b.data_ptr(), out.data_ptr(), a.numel(), stream)
        if rc != 0:
            raise RuntimeError("attnres_bf16_add -> %d" % rc)


# --------------------------------------------------------------------------
# the chain, R micro-batches on the device

class DeviceChains:
    """R copies of one 256-token chain, each with its own buffers."""

    def __init__(self, chain, R, launcher):
        import torch

        self.chain, self.R, self.L = chain, R, launcher
        self.layers = chain.layers
        q = [dev(l.query) for l in chain.layers]
        g = [dev(l.gamma) for l in chain.layers]
        routed0 = [dev(l.routed) for l in chain.layers]
        shared0 = [dev(l.shared) for l in chain.layers]
        emb0, p00 = dev(chain.embedding), dev(chain.prefix0)
        M, H = chain.M, chain.H
        self.inst = []
        for i in range(R):
            c = dict(
                emb=emb0.clone(), p0=p00.clone(), zero=torch.zeros_like(p00),
                routed=[t.clone() for t in routed0], shared=[t.clone() for t in shared0],
                tail=[torch.empty_like(p00) for _ in chain.layers],
                out_prefix=[torch.empty((M, H), dtype=torch.bfloat16, device="cuda") for _ in chain.layers],
                out_norm=[torch.empty((M, H), dtype=torch.bfloat16, device="cuda") for _ in chain.layers])
            self.inst.append(c)
        self.q, self.g = q, g
        # static hand-off plan per (instance, layer): prefix and bank tensors
        self.fused = []      # [layer][instance] ctypes args, both addends
        self.unfused = []    # [layer][instance] ctypes args, pre-summed addend
        for l, layer in enumerate(chain.layers):
            row_f, row_u = [], []
            for c in self.inst:
                bank = [c["emb"]] + [c["out_prefix"][k] for k in range(l) if self.layers[k].push_after]
                if l == 0:
                    prefix = c["p0"]
                elif self.layers[l - 1].push_after:
                    prefix = c["zero"]
                else:
                    prefix = c["out_prefix"][l - 1]
                assert len(bank) == layer.n_sources
                row_f.append(launcher.fused_args(prefix, c["routed"][l], c["shared"][l], bank, q[l], g[l],
                                                 chain.eps, c["out_prefix"][l], c["out_norm"][l]))
                row_u.append(launcher.fused_args(prefix, c["tail"][l], None, bank, q[l], g[l],
                                                 chain.eps, c["out_prefix"][l], c["out_norm"][l]))
            self.fused.append(row_f)
            self.unfused.append(row_u)

    def step(self, stream, fused=True):
        L = self.L
        for l in range(len(self.layers)):
            for i, c in enumerate(self.inst):
                if fused:
                    L.run_fused(self.fused[l][i], stream)
                else:
                    L.run_add(c["routed"][l], c["shared"][l], c["tail"][l], stream)
                    L.run_fused(self.unfused[l][i], stream)

    def launches_per_step(self):
        return len(self.layers) * self.R

    def bytes_per_step(self):
        c = self.chain
        return self.R * sum(call_bytes(c.M, c.H, l.n_sources) for l in self.layers)


# --------------------------------------------------------------------------

def graph_time(fn, steps, warmup):
    """Capture fn(stream) into a HIP graph; replay `warmup` then `steps` times.
    Returns seconds per replay (events bracketed by synchronisation)."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps, g


def event_group_times(groups, sleep_cycles=200_000_000):
    """GPU time of each group of back-to-back launches (seconds).  A sleep
    kernel holds the queue while the host enqueues every group, with one HIP
    event between groups, so the events bracket kernels that run back to back
    (not host launch gaps).  `groups` is a list of lists of fn(stream_handle)."""
    import torch

    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(groups) + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles)
    evs[0].record(stream)
    for i, grp in enumerate(groups):
        for fn in grp:
            fn(h)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(len(groups))]


# --------------------------------------------------------------------------

def parity_gate(chain, launcher, orc):
    """Run one chain on the GPU (fresh buffers) and compare sampled token rows
    with the CPU oracle chain: bit-exact prefixes, out_norm within 2 ulps."""
    import numpy as np
    import torch

    from attention_residual_rmsnorm_amd import workloads as W
    ar = launcher.ar
    d = [(dev(l.query), dev(l.gamma), dev(l.routed), dev(l.shared)) for l in chain.layers]
    step = lambda l, p, b, L: ar.attnres_add_rmsnorm_fwd(p, d[l][2], d[l][3], b, d[l][0], d[l][1], chain.eps)
    zero = lambda: torch.zeros((chain.M, chain.H), dtype=torch.bfloat16, device="cuda")
    outs, _ = W.run_chain(chain, step, zero, embedding=dev(chain.embedding), prefix0=dev(chain.prefix0))
    torch.cuda.synchronize()
    idx = np.array([0, 1, 63, 128, 200, 255])
    sub = chain.rows(idx)
    ref, _ = W.run_chain(sub, lambda l, p, b, L: orc.fwd(p, L.routed, L.shared, b, L.query, L.gamma, sub.eps),
                         lambda: np.zeros((sub.M, sub.H), np.uint16))
    for l, ((gp, gn), (rp, rn)) in enumerate(zip(outs, ref)):
        gp, gn = host(gp)[idx], host(gn)[idx]
        if not np.array_equal(gp, rp):
            raise SystemExit("parity gate: layer %d out_prefix differs from the oracle" % l)
        if not norm_ok(gn, rn):
            raise SystemExit("parity gate: layer %d out_norm outside 2 ulps of the oracle" % l)
    log("parity gate: 25 layers, %d sampled tokens: ok" % len(idx))
    return idx, ref


def verify_instances(dc, idx, ref):
    """After the timed graph replays: every micro-batch instance's outputs, on
    the sampled token rows of every layer, against the oracle chain (bit-exact
    prefixes, out_norm within 2 ulps), and the instances against each other
    bit for bit (same inputs, same dispatch)."""
    import numpy as np
    import torch

    torch.cuda.synchronize()
    first = None
    for i, c in enumerate(dc.inst):
        got = [(host(c["out_prefix"][l])[idx], host(c["out_norm"][l])[idx]) for l in range(len(dc.layers))]
        for l, ((gp, gn), (rp, rn)) in enumerate(zip(got, ref)):
            if not np.array_equal(gp, rp):
                raise SystemExit("after timing: instance %d layer %d out_prefix differs from the oracle" % (i, l))
            if not norm_ok(gn, rn):
                raise SystemExit("after timing: instance %d layer %d out_norm outside 2 ulps of the oracle" % (i, l))
        if first is None:
            first = got
        elif not all(np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) for a, b in zip(got, first)):
            raise SystemExit("after timing: instance %d differs from instance 0" % i)
    return {"instances": len(dc.inst), "layers": len(dc.layers), "tokens_sampled": int(len(idx)), "ok": True}


def cpu_baseline(chain, threads, min_cpu_seconds=12.0, max_passes=8):
    """The CPU oracle (as it stands) on the chain: all 256 tokens, token blocks
    on `threads` threads (ctypes releases the GIL), repeated until about
    `min_cpu_seconds` of CPU work (threads x wall) is done."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from attention_residual_rmsnorm_amd import workloads as W

    orc = oracle.get()
    blocks = np.array_split(np.arange(chain.M), threads)
    subs = [chain.rows(idx) for idx in blocks]

    def run_block(sub):
        W.run_chain(sub, lambda l, p, b, L: orc.fwd(p, L.routed, L.shared, b, L.query, L.gamma, sub.eps),
                    lambda: np.zeros((sub.M, sub.H), np.uint16))

    passes, wall = 0, 0.0
    with ThreadPoolExecutor(threads) as ex:
        while passes < max_passes and (passes == 0 or wall * threads < min_cpu_seconds):
            t0 = time.perf_counter()
            list(ex.map(run_block, subs))
            wall += time.perf_counter() - t0
            passes += 1
    nbytes = passes * sum(call_bytes(chain.M, chain.H, l.n_sources) for l in chain.layers)
    return {"value": round(nbytes / wall / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the full 25-layer chain (256 tokens, H=7168, N=1..12, add2) %d times, oracle in "
                      "binary64, token blocks over %d threads; %.2f s wall; host: %s, %d logical CPUs"
                      % (passes, threads, wall, cpu_model(), os.cpu_count() or 0)}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_latency(threads, repeats=5):
    """The CPU oracle (as it stands) on each small named call: median wall time
    of `repeats` runs on one thread, and with the tokens split over `threads`
    threads (the single-token calls cannot use more than one)."""
    import statistics
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from attention_residual_rmsnorm_amd import workloads as W

    orc = oracle.get()
    out = {}
    with ThreadPoolExecutor(threads) as ex:
        for name in ("cfg1", "cfg2", "cfg3", "cfg4", "cfg4b"):
            case = W.config_case(name)
            run = lambda c: orc.fwd(c.prefix, c.add, c.add2, c.snapshots, c.query, c.gamma, c.eps)

            def median(fn):
                ts = []
                for _ in range(repeats):
                    t0 = time.perf_counter()
                    fn()
                    ts.append(time.perf_counter() - t0)
                return statistics.median(ts)

            one = median(lambda: run(case))
            subs = [case.rows(idx) for idx in np.array_split(np.arange(case.M), min(threads, case.M))]
            many = median(lambda: list(ex.map(run, subs)))
            out[name] = {"M": case.M, "N": case.N, "ms_1_thread": round(one * 1e3, 3),
                         "ms_threads": round(many * 1e3, 3), "threads": len(subs)}
    return out


def read_traffic(src_hash):
    """HBM bytes per fused launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pool_sets(launcher, case, nsets, tail=False):
    """`nsets` distinct buffer sets of one call shape, carved out of one device
    pool (inputs copied from the case, outputs uninitialised).  Returns the
    pool (keep it alive) and a dict of per-set ctypes argument tuples:
    "fused" for the fused call; with `tail` also "add" (the standalone add of
    the two addends into a tail row of the set, run here once) and
    "presummed" (the fused call given that tail and no second addend)."""
    import torch

    M, H, N = case.M, case.H, case.N
    has2 = case.add2 is not None
    rows = [case.prefix, case.add] + ([case.add2] if has2 else []) + list(case.snapshots)
    nr, row_elems, vec_elems = len(rows), M * H, H
    per_set = (nr + 2 + int(tail)) * row_elems + 2 * vec_elems  # rows, outputs, [tail], query, gamma
    pool = torch.empty((nsets, per_set), dtype=torch.bfloat16, device="cuda")
    # layout per set: rows [0, nr), out_prefix nr, out_norm nr+1, [tail nr+2], query, gamma
    q_off = (nr + 2 + int(tail)) * row_elems
    places = [(r, i * row_elems, row_elems) for i, r in enumerate(rows)]
    places += [(case.query, q_off, vec_elems), (case.gamma, q_off + vec_elems, vec_elems)]
    for src, off, n in places:
        pool[:, off:off + n].copy_(dev(src).reshape(1, n).expand(nsets, n))
    base, esz = pool.data_ptr(), pool.element_size()
    vp = ctypes.c_void_p
    out = {"fused": [], "presummed": [], "add": []}
    stream = torch.cuda.current_stream().cuda_stream
    first_snap = 3 if has2 else 2
    for k in range(nsets):
        a = base + k * per_set * esz
        ptr = lambda i: a + i * row_elems * esz
        snaps = (vp * max(N, 1))(*[ptr(first_snap + j) for j in range(N)])
        launcher._keep.append(snaps)
        q = a + q_off * esz
        g = q + vec_elems * esz
        out["fused"].append((ptr(0), ptr(1), ptr(2) if has2 else None, snaps if N else None, N, q, g,
                             ctypes.c_float(case.eps), M, H, ptr(nr), ptr(nr + 1)))
        if tail:
            out["add"].append((ptr(1), ptr(2), ptr(nr + 2), row_elems))
            rc = launcher.add(*out["add"][-1], stream)
            if rc != 0:
                raise RuntimeError("attnres_bf16_add -> %d" % rc)
            out["presummed"].append((ptr(0), ptr(nr + 2), None, snaps if N else None, N, q, g,
                                     ctypes.c_float(case.eps), M, H, ptr(nr), ptr(nr + 1)))
    torch.cuda.synchronize()
    return pool, out


def latency_suite(launcher, calls=96, warm_sets=16, cold_bytes=1.1e9):
    """µs per call of the small named workloads.  Cold: graph replay of one
    launch per distinct buffer set, with at least `cold_bytes` of sets, so
    every call's inputs come from HBM (the 256 MB Infinity Cache has been
    cycled since they were last touched); eager back-to-back launches over the
    sets touched longest ago.  Warm: graph replay of `calls` launches over
    `warm_sets` sets (a few MB, resident in the Infinity Cache)."""
    import torch

    from attention_residual_rmsnorm_amd import workloads as W

    out = {}
    for name in ("cfg1", "cfg2", "cfg3", "cfg4", "cfg4b"):
        case = W.config_case(name)
        nbytes = call_bytes(case.M, case.H, case.N, case.add2 is not None)
        nsets = max(calls * 3, int(cold_bytes // nbytes) + 1)
        pool, sets = pool_sets(launcher, case, nsets)
        args = sets["fused"]

        def cold(stream):
            for a in args:
                launcher.run_fused(a, stream)

        per_cold, _ = graph_time(cold, steps=3, warmup=1)
        grp = event_group_times([[lambda h, a=args[g * calls + k]: launcher.run_fused(a, h) for k in range(calls)]
                                 for g in range(3)], sleep_cycles=50_000_000)
        per_warm, _ = graph_time(lambda s: [launcher.run_fused(args[k % warm_sets], s) for k in range(calls)],
                                 steps=20, warmup=3)
        out[name] = {"M": case.M, "N": case.N, "graph_us_per_call": round(per_cold / nsets * 1e6, 3),
                     "eager_us_per_call": round(min(grp) / calls * 1e6, 3),
                     "GBps_graph": round(nbytes / (per_cold / nsets) / 1e9, 1),
                     "warm_graph_us_per_call": round(per_warm / calls * 1e6, 3),
                     "cold_sets": nsets, "variant": launcher.ar.attnres_plan(case.M, case.N, case.H)[0]}
        log("latency %s: %s" % (name, out[name]))
        del pool, sets, args
        torch.cuda.empty_cache()
    return out


def fold_suite(launcher, cold_bytes=1.1e9):
    """The pages' own comparison of the fold, per small named workload and per
    kernel variant (W: one workgroup per token; S: split hidden): µs per call
    of the fused call with both addends, of the fused call given the pre-summed
    addend (add2 = NULL), and of the standalone bf16 add that the pre-summed
    route needs first.  Graph replay of one launch per distinct buffer set,
    with at least `cold_bytes` of sets (inputs cold in HBM)."""
    import torch

    from attention_residual_rmsnorm_amd import workloads as W

    ar = launcher.ar
    out = {}
    for name in ("cfg2", "cfg3", "cfg4", "cfg4b"):
        case = W.config_case(name)
        nbytes = call_bytes(case.M, case.H, case.N, True)
        nsets = int(cold_bytes // nbytes) + 1
        pool, sets = pool_sets(launcher, case, nsets, tail=True)

        def timed(kind, fn):
            sec, _ = graph_time(lambda s: [fn(a, s) for a in sets[kind]], 3, 1)
            return sec / nsets * 1e6

        def add(a, s):
            rc = launcher.add(*a, s)
            if rc != 0:
                raise RuntimeError("attnres_bf16_add -> %d" % rc)

        t_add = timed("add", add)
        row = {"M": case.M, "N": case.N, "standalone_add_us": round(t_add, 3)}
        for vname, var in (("W", (1, 0)), ("S", (2, 0))):
            ar.attnres_set_variant(*var)
            try:
                f_us = timed("fused", launcher.run_fused)
                p_us = timed("presummed", launcher.run_fused)
            finally:
                ar.attnres_set_variant(0, 0)
            row[vname] = {"fused_us": round(f_us, 3), "presummed_us": round(p_us, 3),
                          "fold_cost_us": round(f_us - p_us, 3), "unfused_us": round(p_us + t_add, 3)}
        row["auto_variant"] = "W" if ar.attnres_plan(case.M, case.N, case.H)[0] == 1 else "S"
        out[name] = row
        log("fold %s: %s" % (name, row))
        del pool, sets
        torch.cuda.empty_cache()
    return out


def grid_suite(launcher, Ms=(1, 2, 4, 8, 16, 32, 48, 64, 96, 128, 256, 288, 320, 384, 448, 512, 1024),
               Ns=(0, 1, 2, 4, 8, 12),
               H=7168, cold_bytes=1.1e9, max_sets=20000):
    """The metric over a grid of token and source counts (add2, automatic
    dispatch): µs per call with inputs cold in HBM (graph replay of one launch
    per distinct buffer set over >= 1.1 GB of sets, or over max_sets sets for
    the smallest calls, still more than the 256 MB Infinity Cache holds) and
    the achieved GB/s of the algorithmic bytes."""
    import torch

    from attention_residual_rmsnorm_amd import workloads as W

    out = []
    for N in Ns:
        for M in Ms:
            case = W.make_case(cfg=93, M=M, N=N, add2=True, H=H)
            nbytes = call_bytes(M, case.H, N, True)
            nsets = min(max_sets, max(64, int(cold_bytes // nbytes) + 1))
            pool, sets = pool_sets(launcher, case, nsets)
            args = sets["fused"]
            sec, _ = graph_time(lambda s: [launcher.run_fused(a, s) for a in args], 3, 1)
            us = sec / nsets * 1e6
            plan = launcher.ar.attnres_plan(M, N, case.H)
            row = {"M": M, "N": N, "H": H, "us_per_call": round(us, 3),
                   "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                   "frac": round(nbytes / (us * 1e-6) / 8e12, 4),
                   "kernel": {1: "W", 3: "hybrid"}.get(plan[0], "S%dw" % (plan[2] // 64))}
            log("grid %s" % row)
            out.append(row)
            del pool, sets, args
            torch.cuda.empty_cache()
    return out


def tap_suite(launcher, calls=64):
    """Cost of the pre-norm mixture output (the capture tap): µs per call of the
    fused call with and without out_mix, graph replay over >= 1 GB of rotating
    buffer sets, at the bandwidth shape (M=256, N=12) and the single-token one."""
    import torch

    from attention_residual_rmsnorm_amd import workloads as W

    out = {}
    for name, M, N in (("m256_n12", 256, 12), ("cfg4b", 1, 12)):
        case = W.make_case(cfg=90, M=M, N=N, add2=True)
        nbytes = call_bytes(M, case.H, N, True)
        rotate = min(32, max(4, int(1.1e9 // (nbytes + M * case.H * 2)) + 1))
        sets = []
        for r in range(rotate):
            t = [dev(x) for x in [case.prefix, case.add, case.add2] + case.snapshots + [case.query, case.gamma]]
            op, on, om = (torch.empty_like(t[0]) for _ in range(3))
            sets.append((launcher.fused_args(t[0], t[1], t[2], t[3:3 + N], t[-2], t[-1], case.eps, op, on),
                         om.data_ptr(), t, op, on, om))
        plain, _ = graph_time(lambda s: [launcher.run_fused(sets[k % rotate][0], s) for k in range(calls)], 12, 2)
        mix, _ = graph_time(lambda s: [launcher.run_mix(sets[k % rotate][0], sets[k % rotate][1], s)
                                       for k in range(calls)], 12, 2)
        p_us, m_us = plain / calls * 1e6, mix / calls * 1e6
        out[name] = {"M": M, "N": N, "plain_us_per_call": round(p_us, 3), "mix_us_per_call": round(m_us, 3),
                     "extra_us": round(m_us - p_us, 3),
                     "mix_GBps": round((nbytes + M * case.H * 2) / (m_us * 1e-6) / 1e9, 1)}
        log("tap %s: %s" % (name, out[name]))
        del sets
        torch.cuda.empty_cache()
    return out


def prefill_suite(launcher, calls=8):
    """Prefill-sized calls (M beyond the decode window, one launch): µs per call
    and GB/s at N = 12, graph replay over >= 1 GB of rotating buffer sets."""
    import torch

    from attention_residual_rmsnorm_amd import workloads as W

    out = {}
    for M in (1024, 4096):
        N = 12
        case = W.make_case(cfg=91, M=M, N=N, add2=True)
        nbytes = call_bytes(M, case.H, N, True)
        rotate = max(2, int(1.1e9 // nbytes) + 1)
        sets = []
        for r in range(rotate):
            t = [dev(x) for x in [case.prefix, case.add, case.add2] + case.snapshots + [case.query, case.gamma]]
            op, on = torch.empty_like(t[0]), torch.empty_like(t[0])
            sets.append((launcher.fused_args(t[0], t[1], t[2], t[3:3 + N], t[-2], t[-1], case.eps, op, on),
                         t, op, on))
        sec, _ = graph_time(lambda s: [launcher.run_fused(sets[k % rotate][0], s) for k in range(calls)], 6, 2)
        us = sec / calls * 1e6
        out["m%d_n%d" % (M, N)] = {"M": M, "N": N, "us_per_call": round(us, 2),
                                   "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                                   "frac": round(nbytes / (us * 1e-6) / 8e12, 4)}
        log("prefill %s" % out["m%d_n%d" % (M, N)])
        del sets
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--micro-batches", type=int, default=16)
    ap.add_argument("--mode", choices=["full", "chain", "eager", "copy", "latency", "grid", "single"], default="full",
                    help="full: everything; chain: the timed chain only (for kernel-trace "
                         "profiling); eager: --steps eager steps of the chain, no graph and no "
                         "timing (for counter collection); copy: a plain 1 GiB device copy, the "
                         "calibration kernel for the HBM byte counters; latency: the parity gate, "
                         "then only the small named calls and the per-config fold comparison "
                         "(for kernel-trace profiling of the latency workloads); grid: the parity "
                         "gate, then µs per call and GB/s over a grid of token and source counts, "
                         "at H=7168 and at one tensor-parallel rank's share of it (H=896); single: "
                         "the parity gate, then µs per call of one token at N = 1..12 (H=7168)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the step is one "
              "GPU's share; see the design notes for how it would shard). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.mode == "copy":
        n = 1 << 29  # 2^29 bf16 = 1 GiB
        a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_copy": 2 * n, "bytes_written_per_copy": 2 * n,
                          "copies": 5}))
        return

    from attention_residual_rmsnorm_amd import workloads as W

    launcher = Launcher()
    launcher.ar.attnres_init()
    chain = W.make_chain()
    log("chain inputs ready: M=%d H=%d layers=%d" % (chain.M, chain.H, len(chain.layers)))

    import oracle

    gate_idx, gate_ref = parity_gate(chain, launcher, oracle.get())

    if args.mode == "grid":
        # the full hidden size, then one tensor-parallel rank's share of it (7168 / 8 columns)
        res = {"mode": "grid", "grid": grid_suite(launcher),
               "tp8_share": grid_suite(launcher, Ms=(1, 8, 16, 32, 256), Ns=(4, 12), H=896)}
        assert launcher.ar.attnres_debug_timeouts() == 0
        print(json.dumps(res))
        return

    if args.mode == "single":
        res = {"mode": "single", "single_token": grid_suite(launcher, Ms=(1,), Ns=tuple(range(1, 13)))}
        assert launcher.ar.attnres_debug_timeouts() == 0
        print(json.dumps(res))
        return

    if args.mode == "latency":
        res = {"mode": "latency", "latency_us": latency_suite(launcher), "fold_per_config": fold_suite(launcher)}
        assert launcher.ar.attnres_debug_timeouts() == 0
        print(json.dumps(res))
        return

    dc = DeviceChains(chain, args.micro_batches, launcher)
    log("device buffers: %.2f GB" % (torch.cuda.memory_allocated() / 1e9))
    if args.mode == "eager":
        for k in range(args.steps):
            dc.step(torch.cuda.current_stream().cuda_stream, fused=True)
            torch.cuda.synchronize()
            log("eager step %d done" % k)
        print(json.dumps({"mode": "eager", "steps": args.steps, "launches": dc.launches_per_step() * args.steps,
                          "algorithmic_bytes_per_launch": dc.bytes_per_step() / dc.launches_per_step()}))
        return

    # timed region: whole steps as HIP-graph replays
    sec, _ = graph_time(lambda s: dc.step(s, fused=True), args.steps, args.warmup)
    nbytes = dc.bytes_per_step()
    value = nbytes / sec / 1e9
    log("step: %.3f ms, %.1f GB/s" % (sec * 1e3, value))
    # what the timed replays left in every instance's outputs
    after_timing = verify_instances(dc, gate_idx, gate_ref)
    log("after timing: %s" % after_timing)

    # the fused kernel's average launch duration over the timed region: HIP
    # events around the replays on the launch stream, divided by the launches
    # (the replayed graph holds nothing but the step's fused launches, back to
    # back, so this is wall time per launch, gaps between launches included;
    # rocprofv3's kernel trace of the same command gives the per-dispatch
    # durations it is checked against)
    launches = dc.launches_per_step()
    per_launch_bytes = nbytes / launches
    avg_kernel = sec / launches
    achieved = per_launch_bytes / avg_kernel / 1e9
    # per layer: events around each layer's group of micro-batch launches
    groups = [[(lambda h, a=dc.fused[l][i]: launcher.run_fused(a, h)) for i in range(dc.R)]
              for l in range(len(dc.layers))]
    gt = event_group_times(groups)
    per_layer = {}
    for l, layer in enumerate(dc.layers):
        per_layer.setdefault(layer.n_sources, []).append(gt[l] / dc.R)
    t12 = sum(per_layer[12]) / len(per_layer[12])
    b12 = call_bytes(chain.M, chain.H, 12)
    t1 = sum(per_layer[1]) / len(per_layer[1])
    b1 = call_bytes(chain.M, chain.H, 1)
    src_hash = kernel_source_hash()
    traffic = read_traffic(src_hash)
    plan = launcher.ar.attnres_plan(chain.M, 12, chain.H)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "attnres fused fwd, variant %s (%d threads/workgroup)" % (
                    "W" if plan[0] == 1 else "S", plan[2]),
                "wall_us_per_launch": round(avg_kernel * 1e6, 3),
                "algorithmic_bytes_per_launch": round(per_launch_bytes),
                "n12_layer": {"kernel_us": round(t12 * 1e6, 3), "GBps": round(b12 / t12 / 1e9, 1),
                              "frac": round(b12 / t12 / 1e9 / HBM_PEAK_GBS, 4)},
                "n1_layer": {"kernel_us": round(t1 * 1e6, 3), "GBps": round(b1 / t1 / 1e9, 1),
                             "frac": round(b1 / t1 / 1e9 / HBM_PEAK_GBS, 4)},
                "layer_us_by_snapshots": {str(n): round(sum(v) / len(v) * 1e6, 3) for n, v in sorted(per_layer.items())},
                "kernel_source_sha256_16": src_hash}
    log("roofline: %s" % roofline)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "25-layer AttnRes+RMSNorm decode chain, M=256 tokens, H=7168, bf16, "
                               "N=1..12 snapshot sources, MoE tail folded (add2); %d independent "
                               "micro-batches interleaved per layer (HBM-cold)" % args.micro_batches,
                   "tokens": chain.M, "hidden": chain.H, "layers": len(chain.layers),
                   "micro_batches": args.micro_batches, "calls_per_step": launches,
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": roofline,
        "parity_after_timing": after_timing,
    }

    if args.mode == "full":
        # the pages' comparison: fold vs standalone add + unfused call
        sec_u, _ = graph_time(lambda s: dc.step(s, fused=False), max(5, args.steps // 2), args.warmup)
        result["fold"] = {"fused_ms_per_step": round(sec * 1e3, 4), "unfused_ms_per_step": round(sec_u * 1e3, 4),
                          "saving_us_per_call": round((sec_u - sec) / launches * 1e6, 3)}
        log("fold: %s" % result["fold"])
        result["latency_us"] = latency_suite(launcher)
        result["fold_per_config"] = fold_suite(launcher)
        result["tap"] = tap_suite(launcher)
        result["prefill"] = prefill_suite(launcher)
        if not args.no_cpu_baseline:
            threads = args.cpu_threads or max(1, min(16, os.cpu_count() or 1))
            result["cpu_baseline"] = cpu_baseline(chain, threads)
            log("cpu baseline: %s" % result["cpu_baseline"])
            result["cpu_latency"] = cpu_latency(threads)
            log("cpu latency: %s" % result["cpu_latency"])
    assert launcher.ar.attnres_debug_timeouts() == 0
    print(json.dumps(result))


if __name__ == "__main__":
    main()
