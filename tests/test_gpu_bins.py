"""Parity of the divide-and-conquer forward (wc_forward with bins > 1) with the binned fp64
oracle, with weights over the union of the bins' coresets (the default) and per bin: pivots
bit-exact under uniforms snapped bin by bin, rank and flags exact, outputs within the
tolerances.  Cases run the per-bin pivot loop on the resident kernel (bf16 bins of at most
256 keys and 32 pivots) and on the streaming loop, fp32 and bf16, d and dv of 64 and 128,
ragged coreset blocks (r not a multiple of 64); plus one bin equal to the plain forward, a
breakdown confined to one bin, a key repeated across bins (left out of the union once),
queries at coreset keys (exact rows under union weights), and the seeded mode."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import philox
from oracle import wildcat as ow
from tests.gpu_util import TOL, check_output, dev, host, pivot_report, rel, snapped_binned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


# (name, dtype, kind, H, n, m, d, dv, r, B)
CASES = [
    ("resident_bins", "bf16", "mixture", 2, 1024, 100, 64, 64, 32, 4),
    ("resident_bins_d128", "bf16", "kv_outlier", 2, 2048, 64, 128, 128, 64, 16),
    ("stream_bins_bf16", "bf16", "mixture", 2, 4096, 300, 64, 64, 128, 8),
    ("stream_bins_f32", "f32", "iid_clip", 2, 2048, 77, 128, 64, 64, 4),
    ("stream_bins_ragged_m", "bf16", "iid_clip", 3, 1536, 257, 64, 128, 48, 3),
    ("stream_bins_ragged_r", "bf16", "mixture", 2, 6000, 130, 128, 64, 200, 8),
    ("stream_bins_f32_d64", "f32", "mixture", 1, 3000, 50, 64, 128, 150, 3),
    # unions of 8 and 6 blocks of 64: several trailing-update and panel steps, more heads
    ("stream_bins_r512_h5", "bf16", "iid_clip", 5, 8192, 96, 64, 128, 512, 8),
    ("stream_bins_r384_f32", "f32", "iid_clip", 3, 6144, 70, 128, 64, 384, 6),
]


def case_inputs(case):
    name, dtype, kind, H, n, m, d, dv, r, B = case
    return synth.random_inputs(H, n, m, d, dv, seed=700 + CASES.index(case), dtype=dtype, kind=kind,
                               clip=2.5, clusters=8)


@pytest.mark.parametrize("mode", ["union", "bin"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_binned_forward_parity(wc, case, mode):
    name, dtype, kind, H, n, m, d, dv, r, B = case
    Q, K, V = case_inputs(case)
    U = snapped_binned(K, r, B)
    out = wc.wc_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), r, u_forced=dev(U), bins=B,
                        bin_weights=mode == "bin")
    O, piv, rank, flags = host(out["O"]), host(out["pivots"]), host(out["rank"]), host(out["flags"])
    for h in range(H):
        ref = ow.forward_binned(Q[h], K[h], V[h], r, B, U[h], weights_mode=mode)
        assert np.array_equal(piv[h], ref["pivots"]), (h, piv[h], ref["pivots"])
        assert rank[h] == ref["rank"] and flags[h] == ref["flags"], (rank[h], flags[h])
        check_output(O[h], ref["O"], ref["kappa"], dtype, f"{__name__}:{h}")


def test_one_bin_is_the_plain_forward(wc):
    Q, K, V = synth.random_inputs(2, 600, 50, 64, 64, seed=710, dtype="bf16", kind="mixture")
    args = (dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), 24)
    a = wc.wc_forward(*args, seed=3, bins=1)
    b = wc.wc_forward(*args, seed=3)
    assert np.array_equal(host(a["pivots"]), host(b["pivots"]))
    assert np.array_equal(host(a["O"]), host(b["O"]))


@pytest.mark.parametrize("mode", ["union", "bin"])
def test_breakdown_confined_to_one_bin(wc, mode):
    """Bin 0 of head 0 holds only zero keys (H = 1 there exactly, rank one in any precision):
    its other slots stay empty (-1), the head is flagged, and the output matches the oracle,
    which skips those slots too."""
    H, n, m, r, B = 2, 1024, 40, 32, 4
    Q, K, V = synth.random_inputs(H, n, m, 64, 64, seed=711, dtype="bf16", kind="mixture")
    K[0, : n // B] = 0.0
    U = snapped_binned(K, r, B)
    out = wc.wc_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), r, u_forced=dev(U), bins=B,
                        bin_weights=mode == "bin")
    piv, rank, flags, O = host(out["pivots"]), host(out["rank"]), host(out["flags"]), host(out["O"])
    ref = ow.forward_binned(Q[0], K[0], V[0], r, B, U[0], weights_mode=mode)
    assert np.array_equal(piv[0], ref["pivots"])
    assert np.all(piv[0, 1:r // B] == -1) and rank[0] == ref["rank"] == r - r // B + 1
    assert flags[0] & 1 and flags[1] == 0 and rank[1] == r
    assert rel(O[0], ref["O"]) < TOL["bf16"]


@pytest.mark.parametrize("n,r,B", [(1024, 32, 4), (4096, 64, 8)])
def test_binned_seeded_mode(wc, n, r, B):
    """Seeded mode: bin b of head h draws Philox with counter (t, h B + b)."""
    H, seed = 3, 99
    Q, K, V = synth.random_inputs(H, n, 30, 64, 64, seed=712, dtype="bf16", kind="mixture")
    out = wc.wc_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), r, seed=seed, bins=B)
    piv = host(out["pivots"])
    agree = 0
    nb, rb = n // B, r // B
    for h in range(H):
        u = np.concatenate([philox.pivot_uniforms(seed, h * B + b, rb) for b in range(B)])
        same = np.array_equal(piv[h], ow.forward_binned(Q[h], K[h], V[h], r, B, u)["pivots"])
        agree += same
        if not same:  # bin by bin, only rounding may separate the device's choice from the draw
            for b in range(B):
                rep = pivot_report(K[h][b * nb:(b + 1) * nb], piv[h][b * rb:(b + 1) * rb] - b * nb,
                                   u[b * rb:(b + 1) * rb])
                assert rep["excess"] <= 1.0, (h, b, rep)
    assert agree >= H - 1, agree


def test_union_key_repeated_across_bins(wc):
    """Bin 1 of head 0 is an exact copy of bin 0 (keys and uniforms), so its pivots repeat bin
    0's: the union keeps each such key once and leaves the copies out (weight zero,
    WC_FLAG_DEPENDENT), as the oracle does; the other head is untouched."""
    H, n, m, r, B = 2, 1024, 60, 32, 4
    nb, rb = n // B, r // B
    Q, K, V = synth.random_inputs(H, n, m, 64, 64, seed=713, dtype="bf16", kind="mixture")
    K[0, nb:2 * nb] = K[0, :nb]
    U = snapped_binned(K, r, B)
    U[0, rb:2 * rb] = U[0, :rb]
    out = wc.wc_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), r, u_forced=dev(U), bins=B)
    piv, rank, flags, O = host(out["pivots"]), host(out["rank"]), host(out["flags"]), host(out["O"])
    ref = ow.forward_binned(Q[0], K[0], V[0], r, B, U[0])
    assert np.array_equal(piv[0, rb:2 * rb], piv[0, :rb] + nb)
    assert not ref["kept"][rb:2 * rb].any() and ref["kept"][:rb].all()
    assert np.array_equal(piv[0], ref["pivots"]) and rank[0] == ref["rank"]
    assert flags[0] == ref["flags"] and flags[0] & wc.WC_FLAG_DEPENDENT
    assert not flags[1] & wc.WC_FLAG_DEPENDENT
    assert rel(O[0], ref["O"]) < TOL["bf16"], rel(O[0], ref["O"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_union_exact_rows_at_coreset_keys(wc, dtype):
    """Queries equal to coreset keys get their exact attention rows under union weights (the
    Nystroem interpolation property, which holds at any size): run once for the pivots, then
    again with those keys as the queries and the same seed."""
    H, n, r, B = 2, 4096, 128, 8
    _, K, V = synth.random_inputs(H, n, 1, 64, 64, seed=714, dtype=dtype, kind="mixture")
    Kd, Vd = dev(K, dtype), dev(V, dtype)
    piv = host(wc.wc_forward(Kd[:, :1].contiguous(), Kd, Vd, r, seed=5, bins=B)["pivots"]).astype(np.int64)
    Qp = np.stack([K[h][piv[h]] for h in range(H)])
    out = wc.wc_forward(dev(Qp, dtype), Kd, Vd, r, seed=5, bins=B)
    assert np.array_equal(host(out["pivots"]), piv)
    O = host(out["O"])
    tol = {"bf16": 2e-2, "f32": 1e-3}[dtype]
    for h in range(H):
        assert rel(O[h], ow.exact_attention(Qp[h], K[h], V[h])) < tol
