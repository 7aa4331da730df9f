"""Helpers shared by the GPU parity tests: device upload, oracle runs per head, metrics."""
import os

import numpy as np

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow

# Output tolerances (relative Frobenius error per head): 1e-4 for fp32 inputs, 2e-2 for bf16.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# Per-row bound, relative error of one output row against the oracle's, for rows whose
# normaliser condition number kappa is below 1e3: ROW_TOL (1 + kappa).  A bf16 path rounds P,
# W and O to 8 significant bits (2^-9 each), an fp32 path carries the hi/lo splits (about
# 2^-17); the bound allows a few such roundings per row.  A row computed from the wrong keys,
# weights or normaliser misses it by orders of magnitude.
ROW_TOL = {"f32": 2.0 ** -15, "bf16": 2.0 ** -8}
# Rows with kappa >= KAPPA_EXCLUDE are left out of the per-head error (their output is
# ill-conditioned in any precision); at most MAX_EXCLUDED of the rows may be left out.
KAPPA_EXCLUDE = 1e6
MAX_EXCLUDED = 0.01
# Relative error of the device's running mass sum at step t, for the pivots' interval check:
# its residual diagonal is fp32; an entry not yet pivoted carries up to about t + 2 roundings
# of 2^-24 of its initial value H_ii (a pivoted one is exactly zero), which summed over those
# rows is (t + 2) 2^-24 sum H_ii against the current total T_t; the factor covers the rounding
# of the fp32 factor entries that feed the residual.
CDF_ERR_FACTOR = 8.0


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def dev(x, dtype="f32"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch_dtype(dtype)).contiguous()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def snapped(K, r):
    """Forced uniforms snapped to interval centres by the oracle, [H, r] float32."""
    raw = synth.raw_uniforms(K.shape[0], r)
    out = np.zeros((K.shape[0], r), np.float32)
    for h in range(K.shape[0]):
        out[h] = ow.snap_uniforms(K[h], r, raw[h])[0]
    return out


def rel(a, b):
    return ow.rel_fro(a, b)


def check_output(O, ref, kappa, dtype, what=""):
    """Per-head and per-row parity of an output block against the oracle's.

    * rows with kappa >= KAPPA_EXCLUDE (or a non-finite oracle row) are left out, and they may
      be at most MAX_EXCLUDED of the rows;
    * the relative Frobenius error over the other rows is below TOL[dtype];
    * every row with kappa < 1e3 has a relative error below ROW_TOL[dtype] (1 + kappa).
    Returns (head error, worst row error over its bound)."""
    O = np.asarray(O, np.float64)
    ref = np.asarray(ref, np.float64)
    kappa = np.asarray(kappa, np.float64)
    finite = np.all(np.isfinite(ref), axis=1)
    ok = finite & (kappa < KAPPA_EXCLUDE)
    excluded = 1.0 - ok.mean() if len(ok) else 0.0
    assert excluded <= MAX_EXCLUDED, (what, "rows left out", excluded)
    err = rel(O[ok], ref[ok]) if ok.any() else 0.0
    assert err < TOL[dtype], (what, "head error", err)
    good = ok & (kappa < 1e3)
    row_err = np.linalg.norm(O[good] - ref[good], axis=1) / np.maximum(np.linalg.norm(ref[good], axis=1), 1e-300)
    ratio = row_err / (ROW_TOL[dtype] * (1.0 + kappa[good])) if good.any() else np.zeros(1)
    worst = float(ratio.max()) if ratio.size else 0.0
    stats = os.environ.get("WC_ROW_STATS")
    if stats:
        with open(stats, "a") as fh:
            fh.write(f"{what} {dtype} rows={len(ok)} excluded={excluded:.4f} head={err:.3e} "
                     f"row_max={float(row_err.max()) if row_err.size else 0.0:.3e} "
                     f"ratio_max={worst:.3f} kappa_max={float(kappa[good].max()) if good.any() else 0.0:.2f}\n")
    assert worst <= 1.0, (what, "row error over bound", worst, float(row_err.max()))
    return err, worst


def cdf_bound(t, H_left, Tt):
    """Bound on the relative error of the device's running mass sum at pivot step t; H_left is
    the sum of the initial diagonal over the rows not pivoted yet, Tt the current total."""
    return CDF_ERR_FACTOR * (t + 2) * 2.0 ** -24 * H_left / Tt


def pivot_report(K, piv, u, beta=None):
    """Device pivots (one per step) against the oracle along the device's own path
    (ow.rpcholesky_follow): the first step whose draw the oracle resolves differently, the
    share of steps before it, and, over every step, how far u_t T_t lies outside the running-sum
    interval of the device's pivot, relative to T_t and to cdf_bound.  A pivot sequence that
    only rounding separates from the oracle's has every excess within the bound."""
    piv = np.asarray(piv)
    valid = piv[piv >= 0]
    f = ow.rpcholesky_follow(K, valid, u, beta)
    n = len(f["T"])
    uT = np.asarray(u[:n], np.float64) * f["T"]
    outside = np.maximum(np.maximum(f["lo"] - uT, uT - f["hi"]), 0.0) / f["T"]
    Hd = ow.initial_residual(K, ow.beta_of(np.asarray(K).shape[1]) if beta is None else beta)
    H_left = Hd.sum() - np.concatenate([[0.0], np.cumsum(Hd[valid[:n]])[:-1]])
    bound = np.array([cdf_bound(t, H_left[t], f["T"][t]) for t in range(n)])
    diff = np.nonzero(f["chosen"] != valid[:n])[0]
    first = int(diff[0]) if len(diff) else None
    return dict(first=first, agree=(n if first is None else first) / max(len(valid), 1), steps=n,
                outside_at_first=float(outside[first]) if first is not None else 0.0,
                bound_at_first=float(bound[first]) if first is not None else 0.0,
                excess=float(np.max(outside / bound)) if n else 0.0)


def snapped_binned(K, r, B):
    """Forced uniforms snapped bin by bin (each bin on its own keys), [H, r] float32."""
    raw = synth.raw_uniforms(K.shape[0], r)
    return np.stack([ow.snap_uniforms_binned(K[h], r, B, raw[h]) for h in range(K.shape[0])])


def snapped_block(K, r, b, B=1):
    """Forced uniforms for block pivots (b candidates per round), snapped on each round's
    start residual by the oracle, bin by bin when B > 1; [H, BLOCK_DRAWS r] float32."""
    raw = synth.raw_uniforms(K.shape[0], ow.BLOCK_DRAWS * r)
    if B == 1:
        return np.stack([ow.snap_uniforms_block(K[h], r, b, raw[h]) for h in range(K.shape[0])])
    return np.stack([ow.snap_uniforms_binned(K[h], r, B, raw[h], pivot_block=b) for h in range(K.shape[0])])
