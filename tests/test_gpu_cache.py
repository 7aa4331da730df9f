"""Parity of the compressed KV cache (wc_compress, wc_cache_append, wc_decode) with the
oracle's compress / exact_rows / decode: pivots, rank and flags bit-exact under snapped
uniforms, decode outputs within the tolerances.  Cases: one bin (resident and streaming
selection) and bins with union or per-bin weights, fp32 and bf16, d and dv of 64 and 128, one
decode query per head (the coreset split over many workgroups) and many; exact rows appended
after the coreset; a cache of exact rows only (exact attention); decode equal to the forward
for the same queries; a capacity larger than the rows in use."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow
from tests.gpu_util import TOL, dev, host, rel, snapped, snapped_binned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


# (name, dtype, kind, H, n, d, dv, r, B, mode, capacity, m)
CASES = [
    ("resident_b1", "bf16", "mixture", 3, 200, 64, 64, 32, 1, "union", 64, 1),
    ("stream_b1_f32", "f32", "iid_clip", 2, 1500, 128, 64, 48, 1, "union", 100, 7),
    ("bins_union", "bf16", "kv_outlier", 2, 4096, 128, 128, 256, 8, "union", 300, 1),
    ("bins_perbin", "bf16", "mixture", 2, 2048, 64, 128, 64, 4, "bin", 64, 33),
    ("bins_union_f32", "f32", "mixture", 2, 1536, 64, 64, 96, 3, "union", 200, 300),
]


def case_inputs(case, m):
    name, dtype, kind, H, n, d, dv, r, B, mode, cap, _ = case
    return synth.random_inputs(H, n, m, d, dv, seed=800 + CASES.index(case), dtype=dtype, kind=kind,
                               clip=2.5, clusters=8)


def uniforms(K, r, B):
    return snapped(K, r) if B == 1 else snapped_binned(K, r, B)


def oracle_rows(K, V, r, B, mode, U):
    return ow.compress(K, V, r, U, B=B, weights_mode=mode)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_compress_then_decode(wc, case):
    name, dtype, kind, H, n, d, dv, r, B, mode, cap, m = case
    Q, K, V = case_inputs(case, m)
    U = uniforms(K, r, B)
    c = wc.wc_compress(dev(K, dtype), dev(V, dtype), r, cap, u_forced=dev(U), bins=B,
                       bin_weights=mode == "bin")
    O, flags = wc.wc_decode(dev(Q, dtype), c["cache"], cap, r, dv)
    O, piv, rank, fl = host(O), host(c["pivots"]), host(c["rank"]), host(c["flags"])
    for h in range(H):
        KR, WR, rp, rk, rf = oracle_rows(K[h], V[h], r, B, mode, U[h])
        assert np.array_equal(piv[h], rp) and rank[h] == rk and fl[h] == rf, (h, rank[h], rk, fl[h], rf)
        assert rel(O[h], ow.decode(Q[h], KR, WR)) < TOL[dtype], (h, rel(O[h], ow.decode(Q[h], KR, WR)))
    assert not host(flags).any()


@pytest.mark.parametrize("case", CASES[1:3], ids=[c[0] for c in CASES[1:3]])
def test_compress_append_decode(wc, case):
    """Exact rows of later tokens appended after the coreset, in two appends; decode over the
    coreset and the appended rows."""
    name, dtype, kind, H, n, d, dv, r, B, mode, cap, m = case
    Q, K, V = case_inputs(case, m)
    U = uniforms(K, r, B)
    extra = min(cap - r, 37)
    rng = np.random.default_rng(5)
    Kn = synth.round_to_bf16(rng.standard_normal((H, extra, d)).astype(np.float32) * 0.4) if dtype == "bf16" \
        else rng.standard_normal((H, extra, d)).astype(np.float32) * 0.4
    Vn = synth.round_to_bf16(rng.standard_normal((H, extra, dv)).astype(np.float32)) if dtype == "bf16" \
        else rng.standard_normal((H, extra, dv)).astype(np.float32)
    c = wc.wc_compress(dev(K, dtype), dev(V, dtype), r, cap, u_forced=dev(U), bins=B,
                       bin_weights=mode == "bin")
    k1 = extra // 2
    wc.wc_cache_append(c["cache"], dev(Kn[:, :k1], dtype), dev(Vn[:, :k1], dtype), r, cap)
    wc.wc_cache_append(c["cache"], dev(Kn[:, k1:], dtype), dev(Vn[:, k1:], dtype), r + k1, cap)
    O = host(wc.wc_decode(dev(Q, dtype), c["cache"], cap, r + extra, dv)[0])
    for h in range(H):
        KR, WR, _, _, _ = oracle_rows(K[h], V[h], r, B, mode, U[h])
        Ke, We = ow.exact_rows(Kn[h], Vn[h])
        ref = ow.decode(Q[h], np.vstack([KR, Ke]), np.vstack([WR, We]))
        assert rel(O[h], ref) < TOL[dtype], (h, rel(O[h], ref))


@pytest.mark.parametrize("dtype,d,dv,n,m", [("bf16", 128, 128, 1000, 1), ("f32", 64, 128, 777, 50),
                                            ("bf16", 64, 64, 130, 300)])
def test_exact_rows_only_is_exact_attention(wc, dtype, d, dv, n, m):
    """A zeroed cache with every key appended as an exact row: decode is exact attention."""
    import torch

    H = 2
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=820 + n, dtype=dtype, kind="iid_clip", clip=2.0)
    cap = n + 50
    p = wc.problem(H, n, m, d, dv, 1, wc.WC_BF16 if dtype == "bf16" else wc.WC_F32)
    cache = torch.zeros(wc.wc_cache_bytes(p, cap), dtype=torch.uint8, device="cuda")
    wc.wc_cache_append(cache, dev(K, dtype), dev(V, dtype), 0, cap)
    O = host(wc.wc_decode(dev(Q, dtype), cache, cap, n, dv)[0])
    for h in range(H):
        assert rel(O[h], ow.exact_attention(Q[h], K[h], V[h])) < TOL[dtype]


@pytest.mark.parametrize("B", [1, 8])
def test_decode_matches_forward(wc, B):
    """Compress then decode gives the forward's output for the same queries (same pivots and
    weights; only the coreset split of the attention may differ)."""
    H, n, m, r = 2, 4096, 100, 128
    Q, K, V = synth.random_inputs(H, n, m, 64, 64, seed=830, dtype="bf16", kind="mixture")
    args = (dev(K, "bf16"), dev(V, "bf16"))
    f = wc.wc_forward(dev(Q, "bf16"), *args, r, seed=9, bins=B)
    c = wc.wc_compress(*args, r, r, seed=9, bins=B)
    O = host(wc.wc_decode(dev(Q, "bf16"), c["cache"], r, r, 64)[0])
    assert np.array_equal(host(f["pivots"]), host(c["pivots"]))
    assert rel(O, host(f["O"])) < 5e-3


@pytest.mark.parametrize("d,dv,n,m", [(128, 128, 1000, 1), (64, 128, 300, 8), (128, 64, 2500, 3),
                                      (64, 64, 64, 2), (64, 64, 257, 1)])
def test_decode_kernel_few_queries(wc, d, dv, n, m):
    """At most 8 bf16 queries per head take the decode kernel: one workgroup when the rows fit
    (up to 1024), split partials and a reduction beyond.  Exact rows only, so the oracle is exact
    attention; the same queries padded to 9 (the attention kernels' path) agree closely."""
    import torch

    H = 3
    Q, K, V = synth.random_inputs(H, n, 9, d, dv, seed=840 + n + m, dtype="bf16", kind="iid_clip", clip=2.0)
    cap = n + 70
    p = wc.problem(H, n, 9, d, dv, 1, wc.WC_BF16)
    cache = torch.zeros(wc.wc_cache_bytes(p, cap), dtype=torch.uint8, device="cuda")
    wc.wc_cache_append(cache, dev(K, "bf16"), dev(V, "bf16"), 0, cap)
    Qd = dev(Q, "bf16")
    O, flags = wc.wc_decode(Qd[:, :m].contiguous(), cache, cap, n, dv)
    O = host(O)
    assert np.all(host(flags) == 0)
    for h in range(H):
        assert rel(O[h], ow.exact_attention(Q[h][:m], K[h], V[h])) < TOL["bf16"]
    O9 = host(wc.wc_decode(Qd, cache, cap, n, dv)[0])
    assert rel(O, O9[:, :m]) < 5e-3, rel(O, O9[:, :m])


@pytest.mark.parametrize("dtype,m,d,dv,n,rows", [("bf16", 9, 128, 128, 300, 200), ("bf16", 1, 64, 64, 300, 70),
                                                 ("f32", 3, 64, 128, 250, 150), ("bf16", 40, 64, 64, 700, 513)])
def test_decode_prefix_of_written_rows(wc, dtype, m, d, dv, n, rows):
    """Rows written past `rows` (here every key is appended, then a shorter prefix is decoded)
    take no part in the output, on the decode kernel (m <= 8, bf16) and on the attention
    kernels (more queries, or fp32), whose scan covers whole 128-row blocks."""
    import torch

    H = 2
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=850 + rows, dtype=dtype, kind="iid_clip", clip=2.0)
    cap = n + 30
    p = wc.problem(H, n, m, d, dv, 1, wc.WC_BF16 if dtype == "bf16" else wc.WC_F32)
    cache = torch.zeros(wc.wc_cache_bytes(p, cap), dtype=torch.uint8, device="cuda")
    wc.wc_cache_append(cache, dev(K, dtype), dev(V, dtype), 0, cap)
    O, flags = wc.wc_decode(dev(Q, dtype), cache, cap, rows, dv)
    O = host(O)
    assert np.all(host(flags) == 0)
    for h in range(H):
        ref = ow.exact_attention(Q[h], K[h][:rows], V[h][:rows])
        assert rel(O[h], ref) < TOL[dtype], (h, rel(O[h], ref))
        full = ow.exact_attention(Q[h], K[h], V[h])
        assert rel(O[h], full) > 5 * TOL[dtype]  # the rows past the prefix would matter
