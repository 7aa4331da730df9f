"""Helpers shared by the GPU parity tests: device upload, oracle runs per head, metrics."""
import numpy as np

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow

# Output tolerances (relative Frobenius error per head): 1e-4 for fp32 inputs, 2e-2 for bf16.
TOL = {"f32": 1e-4, "bf16": 2e-2}


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
