"""The C ABI on the host: the library loads, exports every symbol include/wc.h declares, and
its argument validation returns the documented status before any HIP call (no device is
touched: every call below fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "coreset_head_rpcholesky_amd", "libwc.so")
HEADER = os.path.join(ROOT, "include", "wc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libwc.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wc_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return ctypes.CDLL(LIB)


class Problem(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in ("heads", "n", "m", "d", "dv", "r", "dtype", "bins", "options",
                                              "pivot_block")]


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"wc_rpcholesky", "wc_weights", "wc_attend", "wc_forward",
                          "wc_workspace_bytes", "wc_status_string", "wc_abi_version",
                          "wc_cache_bytes", "wc_compress", "wc_cache_append",
                          "wc_decode_workspace_bytes", "wc_decode"}
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    lib.wc_abi_version.restype = ctypes.c_int32
    assert lib.wc_abi_version() == 9
    lib.wc_status_string.restype = ctypes.c_char_p
    seen = set()
    for s in range(6):
        txt = lib.wc_status_string(s)
        assert txt
        seen.add(txt)
    assert len(seen) == 6


def ws_bytes(lib, p):
    out = ctypes.c_size_t(0)
    st = lib.wc_workspace_bytes(ctypes.byref(p), ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("fields,expect", [
    ((1, 1024, 1024, 64, 64, 32, 0), 0),
    ((768, 197, 197, 64, 64, 32, 1), 0),
    ((0, 10, 10, 64, 64, 5, 1), 0),         # no heads: valid, no work
    ((1, 10, 0, 128, 128, 10, 1), 0),       # no queries: valid
    ((1, 10, 10, 64, 64, 11, 1), 1),        # r > n
    ((1, 10, 10, 64, 64, 0, 1), 1),         # r = 0
    ((-1, 10, 10, 64, 64, 5, 1), 1),        # negative heads
    ((1, 0, 10, 64, 64, 1, 1), 1),          # no keys
    ((1, 100, 10, 32, 64, 5, 1), 2),        # unsupported d
    ((1, 100, 10, 64, 96, 5, 1), 2),        # unsupported dv
    ((1, 100, 10, 64, 64, 5, 7), 2),        # unsupported dtype
    ((1, 10000, 10, 64, 64, 4097, 1), 2),   # r above the supported maximum
    ((2, 4096, 64, 64, 64, 256, 1, 16), 0), # 16 bins
    ((2, 4096, 64, 64, 64, 256, 1, -1), 1), # negative bins
    ((2, 4004, 64, 64, 64, 256, 1, 16), 2), # bins do not divide n
    ((2, 4096, 64, 64, 64, 200, 1, 16), 2), # bins do not divide r
    ((2, 4096, 64, 64, 64, 256, 1, 16, 1), 0),  # per-bin weights option
    ((2, 4096, 64, 64, 64, 256, 1, 16, 4), 1),  # unknown option bit
    ((2, 4096, 64, 64, 64, 256, 1, 1, -1), 1),  # unknown option bits
])
def test_workspace_bytes_validation(lib, fields, expect):
    st, nbytes = ws_bytes(lib, Problem(*fields))
    assert st == expect
    if st == 0 and fields[0] > 0:
        assert nbytes > 0 and nbytes % 256 == 0


def test_null_problem_and_null_out(lib):
    out = ctypes.c_size_t(0)
    assert lib.wc_workspace_bytes(None, ctypes.byref(out)) == 1
    assert lib.wc_workspace_bytes(ctypes.byref(Problem(1, 10, 10, 64, 64, 5, 1)), None) == 1


A = ctypes.c_void_p(0x10000)      # aligned fake device address: never dereferenced
MIS = ctypes.c_void_p(0x10008)    # misaligned


def call_rpc(lib, p, K=A, piv=A, F=A, rank=A, flags=A, u=None, diag=None, trace=None, ws=A, nb=1 << 40):
    return lib.wc_rpcholesky(ctypes.byref(p), K, u, ctypes.c_uint64(1), piv, F, diag, trace, rank,
                             flags, ws, ctypes.c_size_t(nb), None)


def test_rpcholesky_argument_errors(lib):
    p = Problem(4, 300, 300, 64, 64, 16, 1)
    assert call_rpc(lib, p, K=None) == 1
    assert call_rpc(lib, p, piv=None) == 1
    assert call_rpc(lib, p, F=None) == 1
    assert call_rpc(lib, p, rank=None) == 1
    assert call_rpc(lib, p, flags=None) == 1
    assert call_rpc(lib, p, K=MIS) == 1
    assert call_rpc(lib, p, u=MIS) == 1
    assert call_rpc(lib, p, diag=MIS) == 1
    assert call_rpc(lib, p, ws=None) == 3
    assert call_rpc(lib, p, ws=MIS) == 3
    _, need = ws_bytes(lib, p)
    assert call_rpc(lib, p, nb=need - 1) == 3
    assert call_rpc(lib, Problem(4, 300, 300, 64, 64, 301, 1)) == 1
    assert call_rpc(lib, Problem(4, 300, 300, 80, 64, 16, 1)) == 2
    assert call_rpc(lib, Problem(0, 300, 300, 64, 64, 16, 1), K=None) == 0  # no heads: no-op


def test_weights_attend_forward_argument_errors(lib):
    p = Problem(2, 5000, 64, 128, 128, 256, 0)
    big = ctypes.c_size_t(1 << 40)
    u64 = ctypes.c_uint64(0)
    w = lib.wc_weights
    assert w(ctypes.byref(p), None, A, A, A, A, A, big, None) == 1
    assert w(ctypes.byref(p), A, A, A, A, None, A, big, None) == 1
    assert w(ctypes.byref(p), A, A, A, A, A, None, big, None) == 3
    at = lib.wc_attend
    assert at(ctypes.byref(p), None, A, A, A, A, A, A, A, big, None) == 1      # Q needed when m > 0
    assert at(ctypes.byref(p), A, A, A, A, A, MIS, A, A, big, None) == 1
    assert at(ctypes.byref(p), A, A, A, A, A, A, None, A, big, None) == 1      # flags required
    p0 = Problem(2, 5000, 0, 128, 128, 256, 0)
    assert at(ctypes.byref(p0), None, A, A, A, A, None, A, None, big, None) == 3  # m = 0: Q, O optional
    fw = lib.wc_forward
    assert fw(ctypes.byref(p), A, A, None, None, u64, A, None, A, A, A, big, None) == 1
    assert fw(ctypes.byref(p), A, A, A, MIS, u64, A, None, A, A, A, big, None) == 1
    assert fw(ctypes.byref(p), A, A, A, None, u64, A, MIS, A, A, A, big, None) == 1
    assert fw(ctypes.byref(p), A, A, A, None, u64, A, None, None, A, A, big, None) == 1
    assert fw(ctypes.byref(p), A, A, A, None, u64, A, None, A, A, A, ctypes.c_size_t(10), None) == 3
    assert fw(ctypes.byref(Problem(2, 5000, 64, 128, 128, 0, 0)), A, A, A, None, u64, A, None, A, A, A,
              big, None) == 1


def test_bins_only_in_forward_and_smaller_workspace(lib):
    """A binned problem is accepted by wc_workspace_bytes and wc_forward only; its factor is
    B times smaller (B bins of n/B keys and r/B pivots), so its workspace is smaller."""
    plain = Problem(8, 131072, 131072, 128, 128, 2048, 1, 1)
    binned = Problem(8, 131072, 131072, 128, 128, 2048, 1, 16)
    st1, b1 = ws_bytes(lib, plain)
    st2, b2 = ws_bytes(lib, binned)
    assert st1 == 0 and st2 == 0 and b2 < b1 / 4
    assert call_rpc(lib, binned) == 2
    # the union weights stage every key for X = exp(beta K_S K^T) [V, 1] and hold H_SS: more
    # workspace than the per-bin weights
    st3, b3 = ws_bytes(lib, Problem(8, 131072, 131072, 128, 128, 2048, 1, 16, 1))
    assert st3 == 0 and b3 < b2
    big = ctypes.c_size_t(1 << 40)
    assert lib.wc_weights(ctypes.byref(binned), A, A, A, A, A, A, big, None) == 2
    assert lib.wc_attend(ctypes.byref(binned), A, A, A, A, A, A, A, A, big, None) == 2
    # the forward validates its pointers for a binned problem like for a plain one
    assert lib.wc_forward(ctypes.byref(binned), A, None, A, None, ctypes.c_uint64(0), A, None, A, A,
                          A, big, None) == 1


def cache_bytes(lib, p, capacity):
    out = ctypes.c_size_t(0)
    st = lib.wc_cache_bytes(ctypes.byref(p), ctypes.c_int32(capacity), ctypes.byref(out))
    return st, out.value


def test_cache_bytes_scale_with_capacity_not_prefix(lib):
    """The cache holds capacity rows per head whatever the prefix length (the O(r d) memory of
    the compressed cache); fp32 problems keep hi and lo parts, so they need more."""
    a = Problem(32, 32768, 64, 128, 128, 1024, 1)
    b = Problem(32, 4096, 64, 128, 128, 1024, 1)
    st1, n1 = cache_bytes(lib, a, 1024)
    st2, n2 = cache_bytes(lib, b, 1024)
    st3, n3 = cache_bytes(lib, a, 2048)
    st4, n4 = cache_bytes(lib, Problem(32, 32768, 64, 128, 128, 1024, 0), 1024)
    assert st1 == st2 == st3 == st4 == 0
    assert n1 == n2 and n3 > 1.9 * n1 and n4 > 1.9 * n1
    # bf16: keys and weights in bf16 plus the fp32 normaliser column, rounded to 256 bytes
    assert n1 >= 32 * 1024 * (128 + 128 + 1) * 2 and n1 < 32 * 1024 * (128 + 128 + 4) * 2
    assert cache_bytes(lib, a, 0)[0] == 1


def test_cache_calls_validate_before_any_device_work(lib):
    A = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first
    u64 = ctypes.c_uint64(0)
    big = ctypes.c_size_t(1 << 40)
    p = Problem(2, 4096, 1, 64, 64, 256, 1)
    i32 = ctypes.c_int32
    # capacity below r
    assert lib.wc_compress(ctypes.byref(p), A, A, None, u64, A, i32(255), None, A, A, A, big, None) == 1
    # missing cache / rank
    assert lib.wc_compress(ctypes.byref(p), A, A, None, u64, None, i32(256), None, A, A, A, big, None) == 1
    assert lib.wc_compress(ctypes.byref(p), A, A, None, u64, A, i32(256), None, None, A, A, big, None) == 1
    # append past the capacity, negative counts
    assert lib.wc_cache_append(ctypes.byref(p), A, A, i32(10), i32(250), A, i32(256), None) == 1
    assert lib.wc_cache_append(ctypes.byref(p), A, A, i32(-1), i32(0), A, i32(256), None) == 1
    assert lib.wc_cache_append(ctypes.byref(p), A, A, i32(0), i32(0), A, i32(256), None) == 0  # nothing
    # decode: rows outside [1, capacity], workspace too small for the coreset split
    assert lib.wc_decode(ctypes.byref(p), A, A, i32(256), i32(300), A, A, A, big, None) == 1
    assert lib.wc_decode(ctypes.byref(p), A, A, i32(256), i32(0), A, A, A, big, None) == 1
    out = ctypes.c_size_t(0)
    # a few bf16 queries: up to 1024 rows in one workgroup (no workspace), more split over
    # workgroups with fp32 partials: heads x splits x m x (dv + 1) floats
    assert lib.wc_decode_workspace_bytes(ctypes.byref(p), i32(256), ctypes.byref(out)) == 0
    assert out.value == 0
    assert lib.wc_decode_workspace_bytes(ctypes.byref(p), i32(2000), ctypes.byref(out)) == 0
    assert out.value >= 2 * 2 * 1 * 65 * 4
    assert lib.wc_decode(ctypes.byref(p), A, A, i32(2048), i32(2000), A, A, None, 0, None) == 3
    # unsupported problem
    assert lib.wc_decode(ctypes.byref(Problem(2, 4096, 1, 80, 64, 256, 1)), A, A, i32(256), i32(256),
                         A, A, A, big, None) == 2



def test_key_centring_only_in_the_forward(lib):
    """WC_OPT_CENTER_KEYS (2) is accepted by wc_workspace_bytes and wc_forward (whose
    workspace grows by the centred keys) and refused by every other entry point."""
    A = ctypes.c_void_p(256)
    u64 = ctypes.c_uint64(0)
    big = ctypes.c_size_t(1 << 40)
    i32 = ctypes.c_int32
    plain = Problem(2, 5000, 64, 128, 128, 256, 1, 1, 0)
    cent = Problem(2, 5000, 64, 128, 128, 256, 1, 1, 2)
    st1, b1 = ws_bytes(lib, plain)
    st2, b2 = ws_bytes(lib, cent)
    assert st1 == st2 == 0 and b2 >= b1 + 2 * 5000 * 128 * 2
    st3, b3 = ws_bytes(lib, Problem(2, 5000, 64, 128, 128, 250, 1, 5, 3))  # with bins and per-bin weights
    assert st3 == 0 and b3 > 0
    assert call_rpc(lib, cent) == 2
    assert lib.wc_weights(ctypes.byref(cent), A, A, A, A, A, A, big, None) == 2
    assert lib.wc_attend(ctypes.byref(cent), A, A, A, A, A, A, A, A, big, None) == 2
    assert lib.wc_compress(ctypes.byref(cent), A, A, None, u64, A, i32(256), None, A, A, A, big, None) == 2
    assert lib.wc_cache_append(ctypes.byref(cent), A, A, i32(1), i32(0), A, i32(256), None) == 2
    assert lib.wc_decode(ctypes.byref(cent), A, A, i32(256), i32(256), A, A, A, big, None) == 2
    # the forward validates its pointers and workspace with the option like without it
    assert lib.wc_forward(ctypes.byref(cent), A, None, A, None, u64, A, None, A, A, A, big, None) == 1
    assert lib.wc_forward(ctypes.byref(cent), A, A, A, None, u64, A, None, A, A, A,
                          ctypes.c_size_t(b1), None) == 3


def test_pivot_block_validation(lib):
    """pivot_block: 0/1 (one pivot per step) or 16, 32, 64 dividing r (r / bins with bins);
    accepted with per-bin weights and by wc_weights (the slots fill in order)."""
    ok = [Problem(2, 4096, 64, 64, 64, 256, 1, 1, 0, 32), Problem(2, 4096, 64, 64, 64, 256, 1, 4, 0, 64),
          Problem(2, 4096, 64, 64, 64, 256, 1, 16, 0, 16), Problem(2, 4096, 64, 64, 64, 256, 1, 1, 2, 16)]
    for p in ok:
        assert ws_bytes(lib, p)[0] == 0
    assert ws_bytes(lib, Problem(2, 4096, 64, 64, 64, 256, 1, 1, 0, -1))[0] == 1
    assert ws_bytes(lib, Problem(2, 4096, 64, 64, 64, 256, 1, 1, 0, 24))[0] == 2    # not 16/32/64
    assert ws_bytes(lib, Problem(2, 4096, 64, 64, 64, 240, 1, 1, 0, 32))[0] == 2    # 32 does not divide r
    assert ws_bytes(lib, Problem(2, 4096, 64, 64, 64, 256, 1, 16, 0, 32))[0] == 2   # r / bins = 16
    assert ws_bytes(lib, Problem(2, 4096, 64, 64, 64, 256, 1, 4, 1, 32))[0] == 0    # per-bin weights
    A = ctypes.c_void_p(256)
    big = ctypes.c_size_t(1 << 40)
    blk = Problem(2, 4096, 64, 64, 64, 256, 1, 1, 0, 32)
    # the component entry points validate block problems like the others (missing pointers)
    assert lib.wc_weights(ctypes.byref(blk), A, None, A, A, A, big, big, None) == 1
    # the selection holds the candidate columns G [b][n]: more workspace than one pivot a step
    assert ws_bytes(lib, blk)[1] > ws_bytes(lib, Problem(2, 4096, 64, 64, 64, 256, 1, 1, 0, 0))[1]


DEBUG_LIB = os.path.join(ROOT, "coreset_head_rpcholesky_amd", "libwc_debug.so")


@pytest.mark.skipif(not os.path.exists(DEBUG_LIB), reason="libwc_debug.so not built")
def test_debug_library_exports_the_same_abi():
    """The debug build (pivot indices checked in the kernels that read them) is the same ABI."""
    dbg = ctypes.CDLL(DEBUG_LIB)
    for name in declared_functions():
        assert hasattr(dbg, name), name
    dbg.wc_abi_version.restype = ctypes.c_int32
    assert dbg.wc_abi_version() == 9


def test_calibrate_argument_errors(lib):
    """The calibration helper refuses unknown kinds and bad buffers before any HIP call."""
    cal = lib.wc_calibrate
    cal.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                    ctypes.c_void_p, ctypes.c_void_p]
    cal.restype = ctypes.c_int
    B = ctypes.c_void_p(0x20000000)  # a second aligned fake address, far from A
    assert cal(7, A, B, 4096, 1, None, None) == 1         # unknown kind
    assert cal(-1, A, B, 4096, 1, None, None) == 1
    for kind in (0, 1):                                   # READ, COPY
        assert cal(kind, None, B, 4096, 1, None, None) == 1
        assert cal(kind, A, None, 4096, 1, None, None) == 1
        assert cal(kind, MIS, B, 4096, 1, None, None) == 1
        assert cal(kind, A, B, 0, 1, None, None) == 1
        assert cal(kind, A, B, 4100, 1, None, None) == 1  # not a multiple of 16
    assert cal(1, A, ctypes.c_void_p(0x10000 + 4096), 8192, 1, None, None) == 1  # overlapping copy
    for kind in (2, 3):                                   # MFMA_BF16, MFMA_F32
        assert cal(kind, None, B, 0, 0, None, None) == 1  # iters < 1
        assert cal(kind, None, None, 0, 10, None, None) == 1
        assert cal(kind, None, B, 0, 10, ctypes.c_void_p(0x10004), None) == 1  # misaligned clocks
