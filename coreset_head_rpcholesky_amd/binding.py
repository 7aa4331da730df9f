"""Thin Python binding of the WildCat C ABI (include/wc.h), same names as the C entry points.

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity,
outputs and the workspace are allocated with torch, and raw device pointers plus the
current HIP stream are handed to libwc.so.  Every step of the computation runs in the HIP
kernels of that library; if it is not built this module raises on import.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# WC_DEBUG=1 selects the debug build, whose kernels check the pivot indices they read
# (WC_FLAG_BOUNDS); both are built by coreset_head_rpcholesky_amd.build
LIB_PATH = os.path.join(_HERE, "libwc_debug.so" if os.environ.get("WC_DEBUG") == "1" else "libwc.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libwc_debug.so")

WC_OK, WC_ERR_INVALID_ARG, WC_ERR_UNSUPPORTED, WC_ERR_WORKSPACE, WC_ERR_DEVICE = range(5)
WC_F32, WC_BF16 = 0, 1
WC_FLAG_BREAKDOWN, WC_FLAG_NONFINITE, WC_FLAG_DENOM, WC_FLAG_DEPENDENT, WC_FLAG_BOUNDS = 1, 2, 4, 8, 16
WC_OPT_BIN_WEIGHTS = 1
WC_OPT_CENTER_KEYS = 2


class WcProblem(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("n", ctypes.c_int32), ("m", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dv", ctypes.c_int32), ("r", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("bins", ctypes.c_int32), ("options", ctypes.c_int32),
                ("pivot_block", ctypes.c_int32)]


class WcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"WildCat HIP library not built: {LIB_PATH} is missing "
                          "(run python -m coreset_head_rpcholesky_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, u64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64
    P = ctypes.POINTER(WcProblem)
    sig = {
        "wc_abi_version": ([], ctypes.c_int32),
        "wc_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "wc_workspace_bytes": ([P, ctypes.POINTER(sz)], ctypes.c_int),
        "wc_rpcholesky": ([P, vp, vp, u64, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_weights": ([P, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_weights_keys_workspace_bytes": ([P, ctypes.POINTER(sz)], ctypes.c_int),
        "wc_weights_keys": ([P, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_attend": ([P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_forward": ([P, vp, vp, vp, vp, u64, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_forward_noalloc": ([P, vp, vp, vp, vp, u64, vp, vp, vp, vp, vp], ctypes.c_int),
        "wc_cache_bytes": ([P, ctypes.c_int32, ctypes.POINTER(sz)], ctypes.c_int),
        "wc_compress": ([P, vp, vp, vp, u64, vp, ctypes.c_int32, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_cache_append": ([P, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int32, vp], ctypes.c_int),
        "wc_decode_workspace_bytes": ([P, ctypes.c_int32, ctypes.POINTER(sz)], ctypes.c_int),
        "wc_decode": ([P, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, sz, vp], ctypes.c_int),
        "wc_calibrate": ([ctypes.c_int32, vp, vp, sz, ctypes.c_int32, vp, vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


LIB = _load()


def wc_abi_version() -> int:
    return int(LIB.wc_abi_version())


def status_string(status: int) -> str:
    return LIB.wc_status_string(int(status)).decode()


wc_status_string = status_string


def problem(heads, n, m, d, dv, r, dtype, bins: int = 1, options: int = 0,
            pivot_block: int = 1) -> WcProblem:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: WC_F32, torch.bfloat16: WC_BF16}[dtype]
    return WcProblem(int(heads), int(n), int(m), int(d), int(dv), int(r), int(dtype), int(bins),
                     int(options), int(pivot_block))


def wc_workspace_bytes(p: WcProblem) -> int:
    out = ctypes.c_size_t(0)
    st = LIB.wc_workspace_bytes(ctypes.byref(p), ctypes.byref(out))
    if st != WC_OK:
        raise WcError("wc_workspace_bytes", st)
    return int(out.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


BLOCK_DRAWS = 4  # forced uniforms per pivot slot with pivot_block > 1


def _draws(r, pivot_block):
    return BLOCK_DRAWS * r if pivot_block > 1 else r


def _check_in(name, t, dtype, shape, device):
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def workspace(p: WcProblem, device) -> torch.Tensor:
    """A workspace tensor large enough for every entry point on problem ``p``."""
    nbytes = max(wc_workspace_bytes(p), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws(p, device, ws):
    if ws is None:
        ws = workspace(p, device)
    return ws, ws.numel() * ws.element_size()


def wc_rpcholesky(K: torch.Tensor, r: int, *, u_forced=None, seed: int = 0, ws=None,
                  with_diag: bool = True, with_trace: bool = True, pivot_block: int = 1,
                  stream=None):
    """Randomly pivoted Cholesky of exp(beta K K^T) per head.  K: [H, n, d] f32 or bf16."""
    H, n, d = K.shape
    dev = K.device
    p = problem(H, n, 0, d, 64, r, K.dtype, pivot_block=pivot_block)
    if u_forced is not None:
        _check_in("u_forced", u_forced, torch.float32, (H, _draws(r, pivot_block)), dev)
    pivots = torch.empty((H, r), dtype=torch.int32, device=dev)
    F = torch.empty((H, r, n), dtype=torch.float32, device=dev)
    diag = torch.empty((H, n), dtype=torch.float32, device=dev) if with_diag else None
    trace = torch.empty((H, r + 1), dtype=torch.float64, device=dev) if with_trace else None
    rank = torch.empty((H,), dtype=torch.int32, device=dev)
    flags = torch.empty((H,), dtype=torch.int32, device=dev)
    ws, nb = _ws(p, dev, ws)
    st = LIB.wc_rpcholesky(ctypes.byref(p), _ptr(K), _ptr(u_forced), int(seed) & (2**64 - 1),
                           _ptr(pivots), _ptr(F), _ptr(diag), _ptr(trace), _ptr(rank), _ptr(flags),
                           _ptr(ws), nb, _stream(stream))
    if st != WC_OK:
        raise WcError("wc_rpcholesky", st)
    return dict(pivots=pivots, F=F, diag=diag, trace=trace, rank=rank, flags=flags)


def wc_weights(V: torch.Tensor, pivots, rank, F, *, ws=None, stream=None):
    """Nystroem weights W [H, r, dv+1] (fp32) from the factor F and pivots of wc_rpcholesky."""
    H, n, dv = V.shape
    r = pivots.shape[1]
    dev = V.device
    p = problem(H, n, 0, 64, dv, r, V.dtype)
    _check_in("pivots", pivots, torch.int32, (H, r), dev)
    _check_in("rank", rank, torch.int32, (H,), dev)
    _check_in("F", F, torch.float32, (H, r, n), dev)
    W = torch.empty((H, r, dv + 1), dtype=torch.float32, device=dev)
    ws, nb = _ws(p, dev, ws)
    st = LIB.wc_weights(ctypes.byref(p), _ptr(V), _ptr(pivots), _ptr(rank), _ptr(F), _ptr(W),
                        _ptr(ws), nb, _stream(stream))
    if st != WC_OK:
        raise WcError("wc_weights", st)
    return W


def wc_weights_keys(K: torch.Tensor, V: torch.Tensor, pivots, rank, *, flags=None, ws=None, stream=None):
    """Nystroem weights W [H, r, dv+1] (fp32) from the keys, for any pivots (slots past rank
    and pivots -1 empty); returns (W, flags)."""
    H, n, d = K.shape
    dv = V.shape[2]
    r = pivots.shape[1]
    dev = K.device
    p = problem(H, n, 0, d, dv, r, K.dtype)
    _check_in("V", V, K.dtype, (H, n, dv), dev)
    _check_in("pivots", pivots, torch.int32, (H, r), dev)
    _check_in("rank", rank, torch.int32, (H,), dev)
    if flags is None:
        flags = torch.zeros((H,), dtype=torch.int32, device=dev)
    W = torch.empty((H, r, dv + 1), dtype=torch.float32, device=dev)
    if ws is None:
        nb = ctypes.c_size_t(0)
        st = LIB.wc_weights_keys_workspace_bytes(ctypes.byref(p), ctypes.byref(nb))
        if st != WC_OK:
            raise WcError("wc_weights_keys_workspace_bytes", st)
        ws = torch.empty((max(nb.value, 1),), dtype=torch.uint8, device=dev)
    st = LIB.wc_weights_keys(ctypes.byref(p), _ptr(K), _ptr(V), _ptr(pivots), _ptr(rank), _ptr(W),
                             _ptr(flags), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if st != WC_OK:
        raise WcError("wc_weights_keys", st)
    return W, flags


def wc_attend(Q: torch.Tensor, K: torch.Tensor, pivots, rank, W, *, flags=None, ws=None,
              out=None, stream=None):
    """O = row-normalised exp(beta Q K_S^T) W; returns (O [H, m, dv], flags)."""
    H, m, d = Q.shape
    n = K.shape[1]
    r = pivots.shape[1]
    dv = W.shape[2] - 1
    dev = Q.device
    p = problem(H, n, m, d, dv, r, Q.dtype)
    _check_in("K", K, Q.dtype, (H, n, d), dev)
    _check_in("W", W, torch.float32, (H, r, dv + 1), dev)
    if flags is None:
        flags = torch.zeros((H,), dtype=torch.int32, device=dev)
    if out is None:
        O = torch.empty((H, m, dv), dtype=Q.dtype, device=dev)
    else:
        _check_in("out", out, Q.dtype, (H, m, dv), dev)
        O = out
    ws, nb = _ws(p, dev, ws)
    st = LIB.wc_attend(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(pivots), _ptr(rank), _ptr(W),
                       _ptr(O), _ptr(flags), _ptr(ws), nb, _stream(stream))
    if st != WC_OK:
        raise WcError("wc_attend", st)
    return O, flags


def wc_forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, r: int, *, u_forced=None,
               seed: int = 0, bins: int = 1, bin_weights: bool = False, center_keys: bool = False,
               pivot_block: int = 1, ws=None, out=None, stream=None):
    """The whole WildCat forward; returns dict(O, pivots, rank, flags).  bins > 1: the
    divide-and-conquer selection of the C entry point (bins must divide n and r), with weights
    over the union of the bins' coresets, or per bin when ``bin_weights``."""
    H, m, d = Q.shape
    n = K.shape[1]
    dv = V.shape[2]
    dev = Q.device
    opts = (WC_OPT_BIN_WEIGHTS if bin_weights else 0) | (WC_OPT_CENTER_KEYS if center_keys else 0)
    p = problem(H, n, m, d, dv, r, Q.dtype, bins, opts, pivot_block)
    _check_in("K", K, Q.dtype, (H, n, d), dev)
    _check_in("V", V, Q.dtype, (H, n, dv), dev)
    if u_forced is not None:
        _check_in("u_forced", u_forced, torch.float32, (H, _draws(r, pivot_block)), dev)
    if out is None:
        out = dict(O=torch.empty((H, m, dv), dtype=Q.dtype, device=dev),
                   pivots=torch.empty((H, r), dtype=torch.int32, device=dev),
                   rank=torch.empty((H,), dtype=torch.int32, device=dev),
                   flags=torch.empty((H,), dtype=torch.int32, device=dev))
    ws, nb = _ws(p, dev, ws)
    st = LIB.wc_forward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(u_forced),
                        int(seed) & (2**64 - 1), _ptr(out["O"]), _ptr(out["pivots"]),
                        _ptr(out["rank"]), _ptr(out["flags"]), _ptr(ws), nb, _stream(stream))
    if st != WC_OK:
        raise WcError("wc_forward", st)
    return out


WC_NOALLOC_MAX_WORKSPACE = 256 << 20  # bytes of the library's own workspace per device


def wc_forward_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, r: int, *, u_forced=None,
                       seed: int = 0, bins: int = 1, bin_weights: bool = False, center_keys: bool = False,
                       pivot_block: int = 1, out=None, stream=None):
    """wc_forward with the library's own workspace (no workspace argument); with ``out`` given
    the call allocates nothing.  Returns dict(O, pivots, rank, flags)."""
    H, m, d = Q.shape
    n = K.shape[1]
    dv = V.shape[2]
    dev = Q.device
    opts = (WC_OPT_BIN_WEIGHTS if bin_weights else 0) | (WC_OPT_CENTER_KEYS if center_keys else 0)
    p = problem(H, n, m, d, dv, r, Q.dtype, bins, opts, pivot_block)
    _check_in("K", K, Q.dtype, (H, n, d), dev)
    _check_in("V", V, Q.dtype, (H, n, dv), dev)
    if u_forced is not None:
        _check_in("u_forced", u_forced, torch.float32, (H, _draws(r, pivot_block)), dev)
    if out is None:
        out = dict(O=torch.empty((H, m, dv), dtype=Q.dtype, device=dev),
                   pivots=torch.empty((H, r), dtype=torch.int32, device=dev),
                   rank=torch.empty((H,), dtype=torch.int32, device=dev),
                   flags=torch.empty((H,), dtype=torch.int32, device=dev))
    st = LIB.wc_forward_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(u_forced),
                                int(seed) & (2**64 - 1), _ptr(out["O"]), _ptr(out["pivots"]),
                                _ptr(out["rank"]), _ptr(out["flags"]), _stream(stream))
    if st != WC_OK:
        raise WcError("wc_forward_noalloc", st)
    return out


def wc_cache_bytes(p: WcProblem, capacity: int) -> int:
    out = ctypes.c_size_t(0)
    st = LIB.wc_cache_bytes(ctypes.byref(p), int(capacity), ctypes.byref(out))
    if st != WC_OK:
        raise WcError("wc_cache_bytes", st)
    return int(out.value)


def wc_compress(K: torch.Tensor, V: torch.Tensor, r: int, capacity: int, *, u_forced=None,
                seed: int = 0, bins: int = 1, bin_weights: bool = False, pivot_block: int = 1,
                cache=None, ws=None, stream=None):
    """Compress the prefix K, V into rows [0, r) of a cache of ``capacity`` rows per head;
    returns dict(cache (uint8 device tensor), pivots, rank, flags)."""
    H, n, d = K.shape
    dv = V.shape[2]
    dev = K.device
    p = problem(H, n, 0, d, dv, r, K.dtype, bins, WC_OPT_BIN_WEIGHTS if bin_weights else 0,
                pivot_block)
    _check_in("V", V, K.dtype, (H, n, dv), dev)
    if u_forced is not None:
        _check_in("u_forced", u_forced, torch.float32, (H, _draws(r, pivot_block)), dev)
    if cache is None:
        cache = torch.empty(max(wc_cache_bytes(p, capacity), 256), dtype=torch.uint8, device=dev)
    out = dict(cache=cache, pivots=torch.empty((H, r), dtype=torch.int32, device=dev),
               rank=torch.empty((H,), dtype=torch.int32, device=dev),
               flags=torch.empty((H,), dtype=torch.int32, device=dev))
    ws, nb = _ws(p, dev, ws)
    st = LIB.wc_compress(ctypes.byref(p), _ptr(K), _ptr(V), _ptr(u_forced), int(seed) & (2**64 - 1),
                         _ptr(cache), int(capacity), _ptr(out["pivots"]), _ptr(out["rank"]),
                         _ptr(out["flags"]), _ptr(ws), nb, _stream(stream))
    if st != WC_OK:
        raise WcError("wc_compress", st)
    return out


def wc_cache_append(cache: torch.Tensor, K_new: torch.Tensor, V_new: torch.Tensor, row0: int,
                    capacity: int, stream=None):
    """Append K_new [H, count, d], V_new [H, count, dv] as exact rows at row0 .. row0+count-1."""
    H, count, d = K_new.shape
    dv = V_new.shape[2]
    p = problem(H, max(count, 1), 0, d, dv, 1, K_new.dtype)
    _check_in("V_new", V_new, K_new.dtype, (H, count, dv), K_new.device)
    st = LIB.wc_cache_append(ctypes.byref(p), _ptr(K_new), _ptr(V_new), int(count), int(row0),
                             _ptr(cache), int(capacity), _stream(stream))
    if st != WC_OK:
        raise WcError("wc_cache_append", st)


def wc_decode_workspace_bytes(p: WcProblem, rows: int) -> int:
    out = ctypes.c_size_t(0)
    st = LIB.wc_decode_workspace_bytes(ctypes.byref(p), int(rows), ctypes.byref(out))
    if st != WC_OK:
        raise WcError("wc_decode_workspace_bytes", st)
    return int(out.value)


def wc_decode(Q: torch.Tensor, cache: torch.Tensor, capacity: int, rows: int, dv: int, *,
              flags=None, ws=None, out=None, stream=None):
    """Attention of Q [H, m, d] over rows [0, rows) of the cache; returns (O [H, m, dv], flags)."""
    H, m, d = Q.shape
    dev = Q.device
    p = problem(H, 1, m, d, dv, 1, Q.dtype)
    if flags is None:
        flags = torch.zeros((H,), dtype=torch.int32, device=dev)
    O = torch.empty((H, m, dv), dtype=Q.dtype, device=dev) if out is None else out
    if ws is None:
        ws = torch.empty(max(wc_decode_workspace_bytes(p, rows), 256), dtype=torch.uint8, device=dev)
    st = LIB.wc_decode(ctypes.byref(p), _ptr(Q), _ptr(cache), int(capacity), int(rows), _ptr(O),
                       _ptr(flags), _ptr(ws), ws.numel(), _stream(stream))
    if st != WC_OK:
        raise WcError("wc_decode", st)
    return O, flags


# Calibration kinds (include/wc.h): measurement helpers beside the hot path, not steps of it.
WC_CAL_READ, WC_CAL_COPY, WC_CAL_MFMA_BF16, WC_CAL_MFMA_F32 = 0, 1, 2, 3
WC_CAL_RESULT_BYTES = 131072


def wc_calibrate(kind: int, dst: torch.Tensor, *, src=None, nbytes: int = 0, iters: int = 0, clocks=None,
                 stream=None) -> None:
    """Enqueue one calibration kernel (see wc.h); dst, src and clocks are device tensors."""
    st = LIB.wc_calibrate(int(kind), _ptr(src) if src is not None else None, _ptr(dst), int(nbytes), int(iters),
                          _ptr(clocks) if clocks is not None else None, _stream(stream))
    if st != WC_OK:
        raise WcError("wc_calibrate", st)
