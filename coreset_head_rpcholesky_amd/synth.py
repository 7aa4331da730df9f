"""Seeded synthetic inputs shaped like the workloads on the WildCat pages.

This module only draws random inputs; it holds none of the method's arithmetic, so the
CPU oracle and the HIP path can both be fed from it without sharing any computation.

Workloads (per head, Q: [m, d], K: [n, d], V: [n, dv]); the pages give no input
statistics, so each recipe is the one stated with the workload name below.

* ``iid1k``    1 head, n = m = 1024, d = dv = 64, r = 32, fp32.  Q, K i.i.d. N(0,1)/d^0.25,
               rows clipped to norm 2; V ~ N(0,1).
* ``vit197``   ViT-classification-shaped (stands in for T2T-ViT on ImageNet): 64 x 12 heads,
               n = m = 197, d = dv = 64, r = 32, bf16.  Q, K from a 16-cluster Gaussian
               mixture (cluster std 0.3) clipped to norm 3; V ~ N(0,1).
* ``img4096``  image-generation-shaped (stands in for BigGAN on ImageNet): 2 x 16 heads,
               n = m = 4096, d = dv = 64, r = 256, bf16; 64-cluster mixture, clip 3.
* ``kv32k``    LM KV-cache compression (stands in for Qwen2.5-7B on LongBench-E): 32 heads,
               n = 32768 cached keys, d = dv = 128, r = 1024, m = 64 decode-step queries, bf16.
               K ~ N(0,1)/d^0.25 with 1 % of the token rows scaled to 4x norm; Q ~ N(0,1)/d^0.25.
* ``long128k`` long-context (stands in for the sequence-length sweep against FlashAttention 2):
               8 heads, n = m = 131072, d = dv = 128, r = 2048, bf16; 256-cluster mixture, clip 3.

Mixture recipe: centres mu_j ~ N(0, I_d) per head, shared by Q and K of that head; a point
is mu_z + 0.3 * eps with z uniform over the clusters and eps ~ N(0, I_d); then the norm clip
x <- x * min(1, c / |x|).  bf16 workloads are rounded to bf16 (round to nearest even) and
returned as float32 arrays holding bf16-exact values.

Every head draws from its own stream (``numpy.random.default_rng([seed, head])``), so any
subset of heads can be generated alone and matches the same heads of the full batch.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_per_batch: int
    n: int
    m: int
    d: int
    dv: int
    r: int
    dtype: str  # "f32" or "bf16"
    kind: str  # "iid_clip" | "mixture" | "kv_outlier"
    clip: float = 0.0
    clusters: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    description: str = ""

    @property
    def heads(self) -> int:
        return self.batch * self.heads_per_batch

    @property
    def tokens(self) -> int:
        """Sequence tokens per forward: batch x n (all heads run inside one call)."""
        return self.batch * self.n


WORKLOADS = {
    w.name: w
    for w in [
        Workload("iid1k", 1, 1, 1024, 1024, 64, 64, 32, "f32", "iid_clip", clip=2.0,
                 description="1 head, n=1024, d=64, r=32, fp32, iid clipped Gaussian"),
        Workload("vit197", 64, 12, 197, 197, 64, 64, 32, "bf16", "mixture", clip=3.0, clusters=16,
                 description="ViT-classification-shaped: 64x12 heads, n=197, d=64, r=32, bf16"),
        Workload("img4096", 2, 16, 4096, 4096, 64, 64, 256, "bf16", "mixture", clip=3.0, clusters=64,
                 description="image-generation-shaped: 2x16 heads, n=4096, d=64, r=256, bf16"),
        Workload("kv32k", 1, 32, 32768, 64, 128, 128, 1024, "bf16", "kv_outlier",
                 outlier_frac=0.01, outlier_scale=4.0,
                 description="LM KV-cache compression: 32 heads, n=32768, 64 queries, d=128, r=1024, bf16"),
        Workload("long128k", 1, 8, 131072, 131072, 128, 128, 2048, "bf16", "mixture", clip=3.0,
                 clusters=256,
                 description="long-context: 8 heads, n=131072, d=128, r=2048, bf16"),
    ]
}

DATA_SEED_BASE = 1000
PIVOT_SEED = 42
FORCED_UNIFORM_SEED = 7


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    out = ((bits + bias) >> 16).astype(np.uint32) << 16
    return out.view(np.float32).reshape(x.shape)


def _clip_rows(x: np.ndarray, c: float) -> np.ndarray:
    nrm = np.sqrt(np.einsum("ij,ij->i", x.astype(np.float64), x.astype(np.float64)))
    scale = np.minimum(1.0, c / np.maximum(nrm, 1e-300))
    return (x * scale[:, None]).astype(np.float32)


def _head_inputs(w: Workload, rng: np.random.Generator, n: int, m: int, d: int, dv: int):
    if w.kind == "iid_clip":
        s = np.float32(d ** -0.25)
        k = _clip_rows(rng.standard_normal((n, d), dtype=np.float32) * s, w.clip)
        q = _clip_rows(rng.standard_normal((m, d), dtype=np.float32) * s, w.clip)
    elif w.kind == "mixture":
        mu = rng.standard_normal((w.clusters, d), dtype=np.float32)
        zk = rng.integers(0, w.clusters, size=n)
        zq = rng.integers(0, w.clusters, size=m)
        k = mu[zk] + np.float32(0.3) * rng.standard_normal((n, d), dtype=np.float32)
        q = mu[zq] + np.float32(0.3) * rng.standard_normal((m, d), dtype=np.float32)
        k = _clip_rows(k, w.clip)
        q = _clip_rows(q, w.clip)
    elif w.kind == "kv_outlier":
        s = np.float32(d ** -0.25)
        k = rng.standard_normal((n, d), dtype=np.float32) * s
        n_out = int(round(w.outlier_frac * n))
        idx = rng.choice(n, size=n_out, replace=False)
        k[idx] *= np.float32(w.outlier_scale)
        q = rng.standard_normal((m, d), dtype=np.float32) * s
    else:
        raise ValueError(w.kind)
    v = rng.standard_normal((n, dv), dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def make_inputs(name: str | Workload, heads=None, seed: int | None = None, n: int | None = None,
                m: int | None = None):
    """Return float32 arrays Q [H, m, d], K [H, n, d], V [H, n, dv] for the workload.

    ``heads``: iterable of head indices to generate (default: all).  ``n``/``m`` override the
    sequence lengths (for reduced-size cases of the same distribution).
    """
    w = WORKLOADS[name] if isinstance(name, str) else name
    if seed is None:
        seed = DATA_SEED_BASE + list(WORKLOADS).index(w.name) if w.name in WORKLOADS else DATA_SEED_BASE
    heads = list(range(w.heads)) if heads is None else list(heads)
    n = w.n if n is None else n
    m = w.m if m is None else m
    Q = np.empty((len(heads), m, w.d), np.float32)
    K = np.empty((len(heads), n, w.d), np.float32)
    V = np.empty((len(heads), n, w.dv), np.float32)
    for j, h in enumerate(heads):
        rng = np.random.default_rng([seed, h])
        Q[j], K[j], V[j] = _head_inputs(w, rng, n, m, w.d, w.dv)
    return Q, K, V


def raw_uniforms(heads: int, r: int, seed: int = FORCED_UNIFORM_SEED) -> np.ndarray:
    """Raw U[0,1) draws (multiples of 2^-24, exact in fp32) for forced-uniform runs, [heads, r]."""
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 1 << 24, size=(heads, r)) * 2.0 ** -24).astype(np.float32)


def random_inputs(heads: int, n: int, m: int, d: int, dv: int, seed: int, dtype: str = "f32",
                  kind: str = "iid_clip", clip: float = 2.0, clusters: int = 8):
    """Small ad-hoc problems of a given shape drawn with one of the workload recipes."""
    w = Workload("adhoc", 1, heads, n, m, d, dv, 1, dtype, kind, clip=clip, clusters=clusters,
                 outlier_frac=0.01, outlier_scale=4.0)
    return make_inputs(w, seed=seed)
