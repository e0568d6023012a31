"""CPU tests of the C-ABI boundary: the library loads, exports every symbol the
header declares, and rejects invalid calls with the documented status codes
before any HIP call (so these run without a GPU and launch nothing)."""
import ctypes
import os
import re

import pytest

import attention_residual_rmsnorm_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ar.library_path), reason="libattnres.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attnres_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attnres_add_rmsnorm_fwd", "attnres_add_rmsnorm_mix_fwd", "attnres_bf16_add",
              "attnres_init", "attnres_plan",
              "attnres_set_variant", "attnres_status_string", "attnres_version", "attnres_debug_timeouts",
              "attnres_selftest_rounding"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ar.library_path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = dict(re.findall(r"#define (ATTNRES_E?\w+)\s+\(?(-?\d+)\)?", text))
    assert int(codes["ATTNRES_OK"]) == ar.ATTNRES_OK
    assert int(codes["ATTNRES_EINVAL"]) == ar.ATTNRES_EINVAL
    assert int(codes["ATTNRES_EUNSUPPORTED"]) == ar.ATTNRES_EUNSUPPORTED
    assert int(codes["ATTNRES_EALIAS"]) == ar.ATTNRES_EALIAS
    assert int(codes["ATTNRES_EHIP"]) == ar.ATTNRES_EHIP
    assert int(codes["ATTNRES_ENOINIT"]) == ar.ATTNRES_ENOINIT
    assert int(codes["ATTNRES_MAX_SNAPSHOTS"]) == ar.ATTNRES_MAX_SNAPSHOTS
    assert int(codes["ATTNRES_MAX_HIDDEN"]) == ar.ATTNRES_MAX_HIDDEN
    assert ar.attnres_version() >= 100
    assert "overlap" in ar.attnres_status_string(ar.ATTNRES_EALIAS)
    assert "attnres_init" in ar.attnres_status_string(ar.ATTNRES_ENOINIT)
    assert "64" in ar.attnres_status_string(ar.ATTNRES_EUNSUPPORTED)


# Validation: fake but plausible 16-byte-aligned addresses.  Every call below
# is invalid, so the library returns before touching HIP.
A = 1 << 40
ROW = 7168 * 2 * 4  # bytes of an [M=4, H=7168] tensor


def base_args(**kw):
    d = dict(prefix=A, add=A + 1 * ROW, add2=A + 2 * ROW, snaps=[A + 3 * ROW, A + 4 * ROW],
             query=A + 5 * ROW, gamma=A + 5 * ROW + 65536, eps=1e-6, M=4, H=7168,
             out_prefix=A + 7 * ROW, out_norm=A + 8 * ROW)
    d.update(kw)
    return d


def call(d, n=None):
    lib = ar.library()
    snaps = d["snaps"]
    n = len(snaps) if n is None else n
    arr = (ctypes.c_void_p * max(len(snaps), 1))(*snaps) if snaps is not None else None
    return lib.attnres_add_rmsnorm_fwd(d["prefix"], d["add"], d["add2"], arr, n, d["query"], d["gamma"],
                                       ctypes.c_float(d["eps"]), d["M"], d["H"], d["out_prefix"],
                                       d["out_norm"], None)


@pytest.mark.parametrize("field", ["prefix", "add", "query", "gamma", "out_prefix", "out_norm"])
def test_null_required_pointer(field):
    assert call(base_args(**{field: None})) == ar.ATTNRES_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), ar.ATTNRES_EINVAL),
    (dict(M=1 << 31), ar.ATTNRES_EINVAL),
    (dict(H=0), ar.ATTNRES_EINVAL),
    (dict(H=7164), ar.ATTNRES_EINVAL),
    (dict(H=4), ar.ATTNRES_EINVAL),
    (dict(H=ar.ATTNRES_MAX_HIDDEN + 8), ar.ATTNRES_EINVAL),
    (dict(eps=-1e-6), ar.ATTNRES_EINVAL),
    (dict(eps=float("nan")), ar.ATTNRES_EINVAL),
    (dict(eps=float("inf")), ar.ATTNRES_EINVAL),
    (dict(prefix=A + 8), ar.ATTNRES_EINVAL),
    (dict(add2=A + 2 * ROW + 2), ar.ATTNRES_EINVAL),
    (dict(out_norm=A + 8 * ROW + 4), ar.ATTNRES_EINVAL),
    (dict(snaps=[A + 3 * ROW, A + 4 * ROW + 2]), ar.ATTNRES_EINVAL),
    (dict(snaps=[A + 3 * ROW, None]), ar.ATTNRES_EINVAL),
])
def test_invalid_sizes_and_alignment(kw, code):
    assert call(base_args(**kw)) == code


def test_snapshot_count():
    assert ar.ATTNRES_MAX_SNAPSHOTS == 64
    assert call(base_args(), n=-1) == ar.ATTNRES_EINVAL
    many = [A + (10 + i) * ROW for i in range(65)]
    assert call(base_args(snaps=many)) == ar.ATTNRES_EUNSUPPORTED
    # more than one pass of snapshots is accepted; a bad pointer among them is still caught
    bad = [A + (10 + i) * ROW for i in range(30)]
    bad[20] += 2
    assert call(base_args(snaps=bad)) == ar.ATTNRES_EINVAL
    alias = [A + (10 + i) * ROW for i in range(30)]
    assert call(base_args(snaps=alias, out_norm=alias[25])) == ar.ATTNRES_EALIAS
    assert call(base_args(snaps=None), n=2) == ar.ATTNRES_EINVAL


@pytest.mark.parametrize("kw", [
    dict(out_prefix=A + 16),                       # partial overlap with prefix
    dict(out_prefix=A + 1 * ROW),                  # == add
    dict(out_prefix=A + 2 * ROW + 4096),           # inside add2
    dict(out_prefix=A + 4 * ROW),                  # == a snapshot
    dict(out_norm=A),                              # == prefix
    dict(out_norm=A + 7 * ROW),                    # == out_prefix
    dict(out_norm=A + 5 * ROW),                    # == query
    dict(out_norm=A + 5 * ROW + 65536 - 16),       # overlaps gamma
    dict(out_norm=A + 7 * ROW + 16),               # partial overlap with out_prefix
])
def test_aliasing(kw):
    assert call(base_args(**kw)) == ar.ATTNRES_EALIAS


def call_mix(d, out_mix):
    lib = ar.library()
    snaps = d["snaps"]
    arr = (ctypes.c_void_p * len(snaps))(*snaps)
    return lib.attnres_add_rmsnorm_mix_fwd(d["prefix"], d["add"], d["add2"], arr, len(snaps), d["query"],
                                           d["gamma"], ctypes.c_float(d["eps"]), d["M"], d["H"],
                                           d["out_prefix"], d["out_norm"], out_mix, None)


@pytest.mark.parametrize("out_mix,code", [
    (A + 9 * ROW + 8, ar.ATTNRES_EINVAL),   # misaligned
    (A, ar.ATTNRES_EALIAS),                  # == prefix
    (A + 3 * ROW + 64, ar.ATTNRES_EALIAS),   # inside a snapshot
    (A + 5 * ROW + 65536 - 16, ar.ATTNRES_EALIAS),  # overlaps gamma
    (A + 7 * ROW, ar.ATTNRES_EALIAS),        # == out_prefix
    (A + 8 * ROW + 16, ar.ATTNRES_EALIAS),   # overlaps out_norm
])
def test_mix_validation(out_mix, code):
    assert call_mix(base_args(), out_mix) == code
    # the same call with a valid destination but an invalid other argument is still rejected
    assert call_mix(base_args(M=-1), A + 9 * ROW) == ar.ATTNRES_EINVAL


def test_bf16_add_validation():
    lib = ar.library()
    assert lib.attnres_bf16_add(None, A, A + ROW, 8, None) == ar.ATTNRES_EINVAL
    assert lib.attnres_bf16_add(A, A + ROW, A + 2 * ROW, -1, None) == ar.ATTNRES_EINVAL
    assert lib.attnres_bf16_add(A + 2, A + ROW, A + 2 * ROW, 8, None) == ar.ATTNRES_EINVAL
    assert lib.attnres_bf16_add(A, A + ROW, A + 16, 64, None) == ar.ATTNRES_EALIAS


def test_plan_is_pure_and_sane():
    # the measured automatic dispatch at H = 7168
    assert ar.attnres_plan(1, 12, 7168) == (2, 14, 64)     # N >= 6: 1-wave chunks up to 48 tokens
    assert ar.attnres_plan(2, 8, 7168) == (2, 14, 64)
    assert ar.attnres_plan(8, 12, 7168) == (2, 14, 64)
    assert ar.attnres_plan(24, 12, 7168) == (2, 14, 64)
    assert ar.attnres_plan(32, 8, 7168) == (2, 14, 64)
    assert ar.attnres_plan(48, 12, 7168) == (2, 14, 64)
    assert ar.attnres_plan(49, 8, 7168) == (2, 14, 64)     # up to 64 with at most 8 snapshots
    assert ar.attnres_plan(64, 6, 7168) == (2, 14, 64)
    assert ar.attnres_plan(49, 9, 7168) == (2, 4, 256)     # else 4-wave chunks up to 64
    assert ar.attnres_plan(64, 12, 7168) == (2, 4, 256)
    assert ar.attnres_plan(65, 12, 7168) == (2, 14, 64)    # 1-wave again up to 88
    assert ar.attnres_plan(88, 6, 7168) == (2, 14, 64)
    assert ar.attnres_plan(89, 8, 7168) == (2, 7, 128)     # then 2-wave up to 96 from 8 snapshots on
    assert ar.attnres_plan(96, 12, 7168) == (2, 7, 128)
    assert ar.attnres_plan(96, 7, 7168) == (2, 14, 64)     # N = 7: 1-wave up to 96
    assert ar.attnres_plan(89, 6, 7168)[0] == 1            # N = 6: a workgroup per token
    assert ar.attnres_plan(97, 8, 7168)[0] == 1
    assert ar.attnres_plan(97, 7, 7168)[0] == 1
    assert ar.attnres_plan(1, 6, 7168) == (2, 14, 64)      # two exchanges from 6 snapshots on
    assert ar.attnres_plan(2, 3, 7168) == (2, 14, 64)      # 2 <= N <= 5: 1-wave chunks (one exchange)
    assert ar.attnres_plan(40, 2, 7168) == (2, 14, 64)     # up to 40 tokens at N = 2,
    assert ar.attnres_plan(41, 2, 7168)[0] == 1
    assert ar.attnres_plan(56, 3, 7168) == (2, 14, 64)     # 56 at N = 3,
    assert ar.attnres_plan(57, 3, 7168)[0] == 1
    assert ar.attnres_plan(64, 4, 7168) == (2, 14, 64)     # 64 from N = 4 on
    assert ar.attnres_plan(64, 5, 7168) == (2, 14, 64)
    assert ar.attnres_plan(65, 5, 7168)[0] == 1
    assert ar.attnres_plan(65, 4, 7168)[0] == 1
    assert ar.attnres_plan(16, 13, 7168) == (2, 14, 64)    # above 12 sources: 1-wave chunks up to 16,
    assert ar.attnres_plan(16, 20, 16384) == (2, 16, 128)  # rows longer than 8192: 2-wave chunks
    assert ar.attnres_plan(17, 31, 16384) == (2, 32, 64)   # except 1-wave from 17 to 32 tokens
    assert ar.attnres_plan(33, 13, 12288) == (2, 12, 128)
    assert ar.attnres_plan(1, 31, 12288) == (2, 12, 128)
    assert ar.attnres_plan(1, 2, 7168) == (2, 14, 64)
    assert ar.attnres_plan(1, 0, 7168) == (1, 1, 448)      # N = 0: workgroup per token
    assert ar.attnres_plan(1, 1, 7168) == (2, 14, 64)      # N = 1: 1-wave chunks up to 8 tokens
    assert ar.attnres_plan(8, 1, 7168) == (2, 14, 64)
    assert ar.attnres_plan(9, 1, 7168) == (1, 1, 448)
    assert ar.attnres_plan(64, 2, 7168) == (1, 1, 448)
    assert ar.attnres_plan(1, 2, 896) == (1, 1, 128)       # short rows stay on one workgroup per token
    assert ar.attnres_plan(64, 9, 7168) == (2, 4, 256)     # 4-wave chunks
    assert ar.attnres_plan(97, 12, 7168)[0] == 1
    assert ar.attnres_plan(256, 1, 7168) == (1, 1, 448)
    assert ar.attnres_plan(257, 12, 7168) == (3, 14, 448)  # just past the CU count: the hybrid, 1-wave
    assert ar.attnres_plan(272, 12, 7168) == (3, 14, 448)  # chunks up to 16 left-over tokens,
    assert ar.attnres_plan(273, 12, 7168) == (3, 7, 448)   # 2-wave up to 32,
    assert ar.attnres_plan(320, 12, 7168) == (3, 4, 448)   # 4-wave up to 64,
    assert ar.attnres_plan(321, 12, 7168) == (3, 2, 448)   # half rows up to 96
    assert ar.attnres_plan(352, 0, 7168) == (3, 2, 448)
    assert ar.attnres_plan(353, 12, 7168) == (1, 1, 448)
    assert ar.attnres_plan(384, 12, 7168) == (1, 1, 448)
    assert ar.attnres_plan(300, 13, 7168) == (1, 1, 448)
    assert ar.attnres_plan(513, 12, 7168)[0] == 1
    assert ar.attnres_plan(2047, 12, 7168) == (1, 1, 448)
    assert ar.attnres_plan(2048, 12, 7168) == (1, 1, 256)  # prefill-sized: four vectors per thread
    assert ar.attnres_plan(4096, 4, 8192) == (1, 1, 256)
    assert ar.attnres_plan(4096, 13, 7168) == (1, 1, 448)  # more than 12 sources: batches, two vectors
    v, c, t = ar.attnres_plan(256, 12, 7168)
    assert v == 1 and c == 1 and t % 64 == 0
    # more sources than one pass: the split up to 31 snapshots and 96 tokens,
    # else workgroup per token in batches
    assert ar.attnres_plan(1, 13, 7168) == (2, 14, 64)
    assert ar.attnres_plan(17, 20, 7168) == (2, 7, 128)    # 2-wave chunks from 17 to 32,
    assert ar.attnres_plan(32, 31, 7168) == (2, 7, 128)
    assert ar.attnres_plan(33, 31, 7168) == (2, 14, 64)    # 1-wave from 33 to 64,
    assert ar.attnres_plan(64, 13, 7168) == (2, 14, 64)
    assert ar.attnres_plan(65, 13, 7168) == (2, 7, 128)    # 2-wave from 65 to 96
    assert ar.attnres_plan(96, 31, 7168) == (2, 7, 128)
    assert ar.attnres_plan(97, 13, 7168) == (1, 1, 448)
    assert ar.attnres_plan(1, 32, 7168) == (2, 14, 128)    # 32..63 snapshots: the split's two-wave
    assert ar.attnres_plan(16, 63, 8192) == (2, 16, 128)   # form up to 16 tokens,
    assert ar.attnres_plan(17, 32, 7168) == (2, 7, 256)    # its four-wave form beyond,
    assert ar.attnres_plan(64, 39, 7168) == (2, 7, 256)    # up to 64 tokens,
    assert ar.attnres_plan(65, 39, 7168) == (1, 1, 448)
    assert ar.attnres_plan(65, 40, 8192) == (2, 8, 256)    # up to 96 from 40 snapshots on;
    assert ar.attnres_plan(96, 63, 7168) == (2, 7, 256)
    assert ar.attnres_plan(1, 40, 16384) == (2, 16, 256)   # rows past 8192: four waves at every M
    assert ar.attnres_plan(96, 40, 12288) == (2, 12, 256)
    assert ar.attnres_plan(65, 39, 16384) == (1, 1, 512)
    assert ar.attnres_plan(96, 32, 896) == (2, 2, 128)     # shorter rows: two waves up to 96
    assert ar.attnres_plan(5, 36, 1000) == (2, 2, 128)
    assert ar.attnres_plan(97, 52, 7168) == (1, 1, 448)    # then W's batches,
    assert ar.attnres_plan(1, 64, 7168) == (1, 1, 448)     # and W alone at 64 snapshots
    assert ar.attnres_plan(24, 20, 3584) == (2, 7, 64)     # shorter rows: 1-wave chunks up to 96
    assert ar.attnres_plan(96, 31, 896) == (2, 2, 64)
    assert ar.attnres_plan(97, 13, 896)[0] == 1
    assert ar.attnres_plan(256, 64, 7168) == (1, 1, 448)
    assert ar.attnres_plan(3, 40, 16384) == (2, 16, 256)
    # rows longer than 8192, one pass: the split at every N up to 96 tokens
    assert ar.attnres_plan(1, 0, 16384) == (2, 16, 128)    # 2-wave chunks up to 16 tokens,
    assert ar.attnres_plan(16, 12, 12288) == (2, 12, 128)
    assert ar.attnres_plan(17, 4, 16384) == (2, 8, 256)    # 4-wave from 17 to 32,
    assert ar.attnres_plan(33, 8, 16384) == (2, 16, 128)   # 2-wave from 33 to 48,
    assert ar.attnres_plan(49, 1, 12288) == (2, 6, 256)    # 4-wave from 49 to 96
    assert ar.attnres_plan(96, 12, 16384) == (2, 8, 256)
    assert ar.attnres_plan(97, 12, 16384)[0] == 1
    assert ar.attnres_plan(1, 12, 8192) == (2, 16, 64)     # 8192 and shorter: the rules above
    # shorter rows (a tensor-parallel rank's share of the hidden size)
    assert ar.attnres_plan(1, 12, 896) == (1, 1, 128)      # H <= 2048: workgroup per token
    assert ar.attnres_plan(256, 12, 896) == (1, 1, 128)
    assert ar.attnres_plan(8, 12, 2048) == (1, 1, 256)
    assert ar.attnres_plan(1, 12, 3584) == (2, 7, 64)      # 2048 < H < 7168: 1-wave chunks,
    assert ar.attnres_plan(32, 4, 3584) == (2, 7, 64)      # up to 32 tokens at N = 4
    assert ar.attnres_plan(33, 4, 4096)[0] == 1
    assert ar.attnres_plan(48, 5, 4096) == (2, 8, 64)      # up to 48 at N = 5..7
    assert ar.attnres_plan(48, 6, 4096) == (2, 8, 64)
    assert ar.attnres_plan(49, 7, 3584)[0] == 1
    assert ar.attnres_plan(64, 8, 3584) == (2, 7, 64)      # up to 64 at N = 8..11
    assert ar.attnres_plan(65, 11, 3584)[0] == 1
    assert ar.attnres_plan(65, 12, 3584) == (2, 7, 64)     # up to 96 at N = 12
    assert ar.attnres_plan(96, 12, 4096) == (2, 8, 64)
    assert ar.attnres_plan(97, 12, 3584)[0] == 1
    assert ar.attnres_plan(1, 3, 3584)[0] == 1             # fewer sources: workgroup per token
    with pytest.raises(ar.AttnResError):
        ar.attnres_plan(1, 65, 7168)
    with pytest.raises(ar.AttnResError):
        ar.attnres_plan(1, 4, 7170)


def test_set_exchange_validation():
    lib = ctypes.CDLL(ar.library_path)
    for mode in (0, 1, 2, 0):
        assert lib.attnres_debug_set_exchange(mode) == ar.ATTNRES_OK
    assert lib.attnres_debug_set_exchange(3) == ar.ATTNRES_EINVAL
    assert lib.attnres_debug_set_exchange(-1) == ar.ATTNRES_EINVAL


def test_set_variant_validation():
    lib = ar.library()
    assert lib.attnres_set_variant(4, 0) == ar.ATTNRES_EINVAL
    assert lib.attnres_set_variant(3, 3) == ar.ATTNRES_EINVAL
    assert lib.attnres_set_variant(1, 3) == ar.ATTNRES_EINVAL
    assert lib.attnres_set_variant(2, 9) == ar.ATTNRES_EINVAL
    assert lib.attnres_set_variant(2, 3) == ar.ATTNRES_EINVAL
    assert lib.attnres_set_variant(0, 1) == ar.ATTNRES_EINVAL
    try:
        ar.attnres_set_variant(2, 0)
        assert ar.attnres_plan(256, 4, 7168)[0] == 2
        ar.attnres_set_variant(2, 7)
        assert ar.attnres_plan(1, 4, 7168) == (2, 2, 448)
        ar.attnres_set_variant(2, 1)
        assert ar.attnres_plan(3, 4, 7168) == (2, 14, 64)
        assert ar.attnres_plan(200, 63, 7168) == (2, 14, 128)  # the two-wave form, forced past 96 tokens
        with pytest.raises(ar.AttnResError):  # more than 16 chunks of 64 vectors per token
            ar.attnres_plan(1, 40, 16384)
        with pytest.raises(ar.AttnResError):  # two record pages hold at most 63 snapshots
            ar.attnres_plan(1, 64, 7168)
        ar.attnres_set_variant(1, 1)
        assert ar.attnres_plan(1, 4, 7168) == (1, 1, 896)
        with pytest.raises(ar.AttnResError):  # no one-vector batched kernel
            ar.attnres_plan(1, 13, 7168)
        ar.attnres_set_variant(2, 2)
        assert ar.attnres_plan(1, 31, 7168) == (2, 7, 128)
        with pytest.raises(ar.AttnResError):  # 32..63: only the two- and four-wave forms
            ar.attnres_plan(1, 32, 7168)
        ar.attnres_set_variant(2, 4)
        with pytest.raises(ar.AttnResError):  # more than 12 only in the 1-2-wave family
            ar.attnres_plan(1, 13, 7168)
        assert ar.attnres_plan(1, 32, 7168) == (2, 7, 256)  # 32..63: the four-wave form
        assert ar.attnres_plan(1, 40, 16384) == (2, 16, 256)
        ar.attnres_set_variant(3, 0)
        assert ar.attnres_plan(20, 12, 7168) == (3, 14, 448)  # the hybrid, forced at a small M
        with pytest.raises(ar.AttnResError):  # its split part: one pass of sources
            ar.attnres_plan(20, 13, 7168)
        with pytest.raises(ar.AttnResError):  # rows of 513..1024 vectors only
            ar.attnres_plan(20, 4, 3584)
        ar.attnres_set_variant(3, 2)
        assert ar.attnres_plan(20, 12, 7168) == (3, 7, 448)   # its chunks forced to 2 waves
        ar.attnres_set_variant(3, 4)
        assert ar.attnres_plan(300, 12, 7168) == (3, 4, 448)
        ar.attnres_set_variant(3, 8)
        assert ar.attnres_plan(300, 12, 7168) == (3, 2, 448)  # half-row chunks
    finally:
        ar.attnres_set_variant(0, 0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from attention_residual_rmsnorm_amd import _binding

    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "library_path", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        _binding.library()
