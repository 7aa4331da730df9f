"""Pins of the divide-and-conquer (binned) oracle, forward_binned: one bin is the plain
forward; every bin at full rank is exact softmax attention; the output equals the sum over
bins of explicit pseudo-inverse Nystroem approximations written with matrix products; the
pivots of bin b lie in bin b; a breakdown in one bin leaves the others intact; and the error
against exact attention falls as the bins get more pivots."""
import numpy as np
import pytest

from oracle import wildcat as ow


def rand_problem(n=16, m=7, d=4, dv=3, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((m, d)) * 0.7, rng.standard_normal((n, d)) * 0.7,
            rng.standard_normal((n, dv)))


def test_bin_bounds_tile_keys_and_slots():
    bounds = ow.bin_bounds(12, 6, 3)
    assert bounds == [(0, 4, 0, 2), (4, 8, 2, 4), (8, 12, 4, 6)]
    with pytest.raises(ValueError):
        ow.bin_bounds(10, 6, 4)


@pytest.mark.parametrize("seed", range(3))
def test_one_bin_is_the_plain_forward(seed):
    Q, K, V = rand_problem(seed=seed)
    u = np.random.default_rng(seed).random(5)
    a = ow.forward_binned(Q, K, V, 5, 1, u)
    b = ow.forward(Q, K, V, 5, u)
    assert np.array_equal(a["pivots"], b["pivots"])
    assert np.allclose(a["O"], b["O"], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("B", [2, 4])
def test_full_rank_bins_are_exact_attention(B):
    """r = n: each bin's coreset is all of its keys, W_b = [V_b, 1], and the union attends
    exactly (pages, "Methodik" part 2: the Nystroem weights reproduce the full kernel
    features when the coreset spans them)."""
    Q, K, V = rand_problem(n=16, seed=B)
    u = np.random.default_rng(B).random(16)
    out = ow.forward_binned(Q, K, V, 16, B, u)
    assert out["rank"] == 16
    assert np.allclose(out["O"], ow.exact_attention(Q, K, V), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("B,r", [(2, 4), (4, 8), (2, 6)])
def test_sum_of_explicit_per_bin_nystroem(B, r):
    """Y = sum_b h(Q, K_Sb) h(K_Sb, K_Sb)^+ h(K_Sb, K_b) [V_b, 1], written with numpy's
    pseudo-inverse and plain matrix products (the pages' form of the weights)."""
    Q, K, V = rand_problem(n=16, seed=10 + r)
    beta = ow.beta_of(K.shape[1])
    u = np.random.default_rng(r).random(r)
    out = ow.forward_binned(Q, K, V, r, B, u)
    Y = np.zeros((Q.shape[0], V.shape[1] + 1))
    for k0, k1, s0, s1 in ow.bin_bounds(16, r, B):
        S = out["pivots"][s0:s1]
        S = S[S >= 0]
        KS, Kb = K[S], K[k0:k1]
        Vb1 = np.hstack([V[k0:k1], np.ones((k1 - k0, 1))])
        Y += np.exp(beta * Q @ KS.T) @ np.linalg.pinv(np.exp(beta * KS @ KS.T)) @ np.exp(beta * KS @ Kb.T) @ Vb1
    assert np.allclose(out["O"], Y[:, :-1] / Y[:, -1:], rtol=1e-7, atol=1e-9)


def test_pivots_stay_in_their_bin_and_follow_the_bin_loop():
    Q, K, V = rand_problem(n=24, seed=3)
    r, B = 6, 3
    u = np.random.default_rng(5).random(r)
    out = ow.forward_binned(Q, K, V, r, B, u)
    for k0, k1, s0, s1 in ow.bin_bounds(24, r, B):
        S = out["pivots"][s0:s1]
        assert np.all((S >= k0) & (S < k1))
        # the bin's pivots are the plain loop on that bin's keys, shifted to head indices
        assert np.array_equal(S - k0, ow.rpcholesky(K[k0:k1], s1 - s0, u[s0:s1])["pivots"])


def test_breakdown_in_one_bin_only():
    """Bin 0 holds identical keys (rank one): it stops after one pivot, leaves -1 and zero
    weight rows in its other slots, and bin 1 is untouched."""
    Q, K, V = rand_problem(n=16, seed=4)
    K[:8] = K[0]
    u = np.random.default_rng(6).random(6)
    out = ow.forward_binned(Q, K, V, 6, 2, u)
    assert out["rank"] == 4
    assert out["flags"] & ow.FLAG_BREAKDOWN
    assert np.all(out["pivots"][1:3] == -1) and np.all(out["W"][1:3] == 0.0)
    assert np.all(out["pivots"][3:] >= 8)
    assert np.isfinite(out["O"]).all()


def test_error_falls_with_pivots_per_bin():
    """Bounded inputs: more pivots per bin, smaller error against exact attention."""
    rng = np.random.default_rng(7)
    n, d = 256, 16
    K = rng.standard_normal((n, d))
    K *= np.minimum(1.0, 2.0 / np.linalg.norm(K, axis=1, keepdims=True))
    Q = rng.standard_normal((40, d))
    Q *= np.minimum(1.0, 2.0 / np.linalg.norm(Q, axis=1, keepdims=True))
    V = rng.standard_normal((n, 4))
    exact = ow.exact_attention(Q, K, V)
    errs = []
    for r in (8, 32, 128):
        e = [ow.rel_fro(ow.forward_binned(Q, K, V, r, 4, np.random.default_rng(s).random(r))["O"], exact)
             for s in range(3)]
        errs.append(np.mean(e))
    assert errs[0] > errs[1] > errs[2], errs


def test_snapping_per_bin_keeps_each_bins_pivots():
    Q, K, V = rand_problem(n=24, seed=8)
    raw = np.random.default_rng(9).random(6)
    U = ow.snap_uniforms_binned(K, 6, 3, raw)
    a = ow.forward_binned(Q, K, V, 6, 3, raw)
    b = ow.forward_binned(Q, K, V, 6, 3, U.astype(np.float64))
    assert np.array_equal(a["pivots"], b["pivots"])
