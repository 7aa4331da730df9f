"""Parity of block pivot selection (pivot_block = b candidates per round, rounds until the
slots are full) with the oracle's rpcholesky_block and the block-pivoted forward: pivots, rank
and flags bit-exact under uniforms snapped on each round's start residual; F, the residual and
the round-start traces within fp32 rounding; outputs within the tolerances.  Block sizes 16,
32 and 64, fp32 and bf16, d of 64 and 128, ragged n, keys whose mass sits on a few outliers
(later rounds fill the slots), with and without bins, both weight modes; the seeded mode."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import philox
from oracle import wildcat as ow
from tests.gpu_util import TOL, cdf_bound, check_output, dev, host, rel, snapped_block

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


# (name, dtype, kind, H, n, m, d, dv, r, b, B, mode)
CASES = [
    ("b16_bf16", "bf16", "mixture", 2, 2000, 90, 64, 64, 64, 16, 1, "union"),
    ("b32_f32", "f32", "iid_clip", 2, 1500, 60, 128, 64, 64, 32, 1, "union"),
    ("b64_bf16_d128", "bf16", "kv_outlier", 2, 5000, 64, 128, 128, 128, 64, 1, "union"),
    ("b16_bins", "bf16", "mixture", 2, 4096, 100, 64, 128, 128, 16, 4, "union"),
    ("b32_bins_outliers", "bf16", "kv_outlier", 2, 8192, 64, 128, 128, 128, 32, 4, "union"),
    ("b16_bins_perbin", "bf16", "mixture", 2, 2048, 50, 64, 64, 64, 16, 2, "bin"),
]


def case_inputs(case):
    name, dtype, kind, H, n, m, d, dv, r, b, B, mode = case
    return synth.random_inputs(H, n, m, d, dv, seed=950 + CASES.index(case), dtype=dtype, kind=kind,
                               clip=2.5, clusters=8)


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_block_selection_parity(wc, case):
    name, dtype, kind, H, n, m, d, dv, r, b, B, mode = case
    Q, K, V = case_inputs(case)
    U = snapped_block(K, r, b)
    out = wc.wc_rpcholesky(dev(K, dtype), r, u_forced=dev(U), pivot_block=b)
    piv, F, diag = host(out["pivots"]), host(out["F"]), host(out["diag"])
    trace, rank, flags = host(out["trace"]), host(out["rank"]), host(out["flags"])
    for h in range(H):
        ref = ow.rpcholesky_block(K[h], r, U[h], b)
        assert np.array_equal(piv[h], ref["pivots"]), (h, piv[h], ref["pivots"])
        assert rank[h] == ref["rank"] and flags[h] == ref["flags"]
        assert rel(F[h].T, ref["F"]) < 1e-4, rel(F[h].T, ref["F"])
        assert np.allclose(diag[h], ref["diag"], rtol=1e-4, atol=1e-4 * ref["diag"].max())
        nz = ref["trace"] != 0.0
        assert np.array_equal(trace[h] != 0.0, nz)
        assert np.allclose(trace[h][nz], ref["trace"][nz], rtol=1e-5)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_forward_parity(wc, case):
    name, dtype, kind, H, n, m, d, dv, r, b, B, mode = case
    Q, K, V = case_inputs(case)
    U = snapped_block(K, r, b, B)
    out = wc.wc_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), r, u_forced=dev(U), bins=B, pivot_block=b,
                        bin_weights=mode == "bin")
    O, piv, rank, flags = host(out["O"]), host(out["pivots"]), host(out["rank"]), host(out["flags"])
    for h in range(H):
        ref = ow.forward_binned(Q[h], K[h], V[h], r, B, U[h], weights_mode=mode, pivot_block=b)
        assert np.array_equal(piv[h], ref["pivots"]), h
        assert rank[h] == ref["rank"] and flags[h] == ref["flags"], (rank[h], flags[h], ref["rank"], ref["flags"])
        check_output(O[h], ref["O"], ref["kappa"], dtype, f"{__name__}:{h}")


def test_block_seeded_mode(wc):
    """Seeded mode: candidate j of round k of head h draws Philox with counter (k b + j, h)."""
    H, n, r, b = 3, 3000, 64, 32
    _, K, _ = synth.random_inputs(H, n, 1, 64, 64, seed=960, dtype="bf16", kind="mixture")
    out = wc.wc_rpcholesky(dev(K, "bf16"), r, seed=77, pivot_block=b)
    piv = host(out["pivots"])
    agree = 0
    for h in range(H):
        ref = ow.rpcholesky_block(K[h], r, np.array(philox.pivot_uniforms(77, h, ow.BLOCK_DRAWS * r)), b)
        diff = np.nonzero(piv[h] != ref["pivots"])[0]
        agree += len(diff) == 0
        if len(diff):
            # only rounding may separate them: some draw of the rounds up to the one that
            # filled the first differing slot lies within rounding of an interval end
            k = ref["slot_round"][diff[0]]
            f0 = int(np.nonzero(ref["slot_round"] == k)[0][0])
            Hd = ow.initial_residual(K[h], 1.0 / np.sqrt(K.shape[2]))
            bound = cdf_bound(f0, Hd.sum() - Hd[ref["pivots"][:f0]].sum(), ref["trace"][f0])
            assert np.nanmin(ref["margins"][:(k + 1) * b]) <= bound, (h, diff[0], k)
    assert agree >= H - 1, agree


def test_block_on_outlier_keys_fills_every_slot_and_matches_exact(wc):
    """kv32k-like keys (1 % of rows four times longer, holding nearly all the mass): rounds
    after the first fill the slots, and the forward stays close to exact attention."""
    H, n, m, r, b = 2, 8192, 64, 256, 64
    Q, K, V = synth.random_inputs(H, n, m, 128, 128, seed=961, dtype="bf16", kind="kv_outlier")
    out = wc.wc_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), r, seed=3, pivot_block=b)
    plain = wc.wc_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), r, seed=3)
    assert np.all(host(out["rank"]) == r)
    eb = np.mean([rel(host(out["O"])[h], ow.exact_attention(Q[h], K[h], V[h])) for h in range(H)])
    ep = np.mean([rel(host(plain["O"])[h], ow.exact_attention(Q[h], K[h], V[h])) for h in range(H)])
    assert eb < 2 * ep + 0.01, (eb, ep)
