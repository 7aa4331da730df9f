"""Pins of the divide-and-conquer (binned) oracle, forward_binned, in both weight modes.

Both: one bin is the plain forward; every bin at full rank is exact softmax attention; the
pivots of bin b lie in bin b and follow the plain loop on that bin's keys; a breakdown in one
bin leaves the others intact; the error against exact attention falls as the bins get more
pivots.  Per-bin weights: the output equals the sum over bins of explicit pseudo-inverse
Nystroem approximations written with matrix products.  Union weights: W equals numpy's
pseudo-inverse applied to H_{S,:} [V, 1]; queries placed at coreset keys get their exact
attention rows (Nystroem interpolation); a key repeated in two bins is left out once and the
output equals the pseudo-inverse's; the dependence test agrees with the Schur complement
computed by a linear solve; union weights are more accurate than per-bin weights."""
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


@pytest.mark.parametrize("mode", ["union", "bin"])
@pytest.mark.parametrize("seed", range(3))
def test_one_bin_is_the_plain_forward(seed, mode):
    Q, K, V = rand_problem(seed=seed)
    u = np.random.default_rng(seed).random(5)
    a = ow.forward_binned(Q, K, V, 5, 1, u, weights_mode=mode)
    b = ow.forward(Q, K, V, 5, u)
    assert np.array_equal(a["pivots"], b["pivots"])
    assert np.allclose(a["O"], b["O"], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("mode", ["union", "bin"])
@pytest.mark.parametrize("B", [2, 4])
def test_full_rank_bins_are_exact_attention(B, mode):
    """r = n: each bin's coreset is all of its keys, W_b = [V_b, 1], and the union attends
    exactly (pages, "Methodik" part 2: the Nystroem weights reproduce the full kernel
    features when the coreset spans them)."""
    Q, K, V = rand_problem(n=16, seed=B)
    u = np.random.default_rng(B).random(16)
    out = ow.forward_binned(Q, K, V, 16, B, u, weights_mode=mode)
    assert out["rank"] == 16
    assert np.allclose(out["O"], ow.exact_attention(Q, K, V), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("B,r", [(2, 4), (4, 8), (2, 6)])
def test_sum_of_explicit_per_bin_nystroem(B, r):
    """Y = sum_b h(Q, K_Sb) h(K_Sb, K_Sb)^+ h(K_Sb, K_b) [V_b, 1], written with numpy's
    pseudo-inverse and plain matrix products (the pages' form of the weights)."""
    Q, K, V = rand_problem(n=16, seed=10 + r)
    beta = ow.beta_of(K.shape[1])
    u = np.random.default_rng(r).random(r)
    out = ow.forward_binned(Q, K, V, r, B, u, weights_mode="bin")
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


@pytest.mark.parametrize("mode", ["union", "bin"])
def test_breakdown_in_one_bin_only(mode):
    """Bin 0 holds identical keys (rank one): it stops after one pivot, leaves -1 and zero
    weight rows in its other slots, and bin 1 is untouched."""
    Q, K, V = rand_problem(n=16, seed=4)
    K[:8] = K[0]
    u = np.random.default_rng(6).random(6)
    out = ow.forward_binned(Q, K, V, 6, 2, u, weights_mode=mode)
    assert out["rank"] == 4
    assert out["flags"] & ow.FLAG_BREAKDOWN
    assert np.all(out["pivots"][1:3] == -1) and np.all(out["W"][1:3] == 0.0)
    assert np.all(out["pivots"][3:] >= 8)
    assert np.isfinite(out["O"]).all()


def bounded_problem(n=256, d=16, m=40, seed=7):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d))
    K *= np.minimum(1.0, 2.0 / np.linalg.norm(K, axis=1, keepdims=True))
    Q = rng.standard_normal((m, d))
    Q *= np.minimum(1.0, 2.0 / np.linalg.norm(Q, axis=1, keepdims=True))
    return Q, K, rng.standard_normal((n, 4))


@pytest.mark.parametrize("mode", ["union", "bin"])
def test_error_falls_with_pivots_per_bin(mode):
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
        e = [ow.rel_fro(ow.forward_binned(Q, K, V, r, 4, np.random.default_rng(s).random(r),
                                          weights_mode=mode)["O"], exact)
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


def test_union_weights_equal_numpy_pinv():
    """Distinct keys: nothing is left out, and W is numpy's pseudo-inverse of H_SS applied
    to H_{S,:} [V, 1] (the pages' form, "Methodik" part 2)."""
    Q, K, V = rand_problem(n=24, seed=11)
    beta = ow.beta_of(K.shape[1])
    out = ow.forward_binned(Q, K, V, 9, 3, np.random.default_rng(12).random(9))
    S = out["pivots"]
    assert np.all(S >= 0) and out["kept"].all()
    assert not out["flags"] & ow.FLAG_DEPENDENT
    V1 = np.hstack([V, np.ones((24, 1))])
    Wp = np.linalg.pinv(np.exp(beta * K[S] @ K[S].T)) @ np.exp(beta * K[S] @ K.T) @ V1
    assert np.allclose(out["W"], Wp, rtol=1e-7, atol=1e-9)


def test_union_interpolates_at_coreset_keys():
    """A query equal to a coreset key gets its exact attention row: h(k_s, S) H_SS^{-1}
    h(S, K) = h(k_s, K) for every s in S (Nystroem interpolation over the whole coreset)."""
    _, K, V = rand_problem(n=32, seed=13)
    u = np.random.default_rng(14).random(8)
    piv = ow.forward_binned(K[:1], K, V, 8, 4, u)["pivots"]
    out = ow.forward_binned(K[piv], K, V, 8, 4, u)
    assert np.allclose(out["O"], ow.exact_attention(K[piv], K, V), rtol=1e-8, atol=1e-10)


def test_union_leaves_out_a_key_repeated_across_bins():
    """Every key of bin 1 is a copy of bin 0's first pivot, so bin 1's pivots (one, or a
    second one drawn on rounding noise of the exhausted residual) duplicate it: the union
    keeps that key once, flags the dependence, and the output equals the one numpy's
    pseudo-inverse gives."""
    Q, K, V = rand_problem(n=16, seed=15)
    beta = ow.beta_of(K.shape[1])
    u = np.random.default_rng(16).random(4)
    piv0 = ow.rpcholesky(K[:8], 2, u[:2])["pivots"]
    K[8:] = K[piv0[0]]
    out = ow.forward_binned(Q, K, V, 4, 2, u)
    S = out["pivots"]
    assert S[2] >= 8 and out["rank"] in (3, 4)
    assert out["kept"].tolist() == [True, True, False, False]
    assert out["flags"] & ow.FLAG_DEPENDENT
    assert np.all(out["W"][2:] == 0.0)
    Sv = S[S >= 0]
    V1 = np.hstack([V, np.ones((16, 1))])
    Wp = np.linalg.pinv(np.exp(beta * K[Sv] @ K[Sv].T), rcond=1e-10) @ np.exp(beta * K[Sv] @ K.T) @ V1
    Y = np.exp(beta * Q @ K[Sv].T) @ Wp
    assert np.allclose(out["O"], Y[:, :-1] / Y[:, -1:], rtol=1e-7, atol=1e-9)


def test_dependence_test_matches_schur_complement():
    """independent_slots against the residual written as a Schur complement with a linear
    solve: g_j = H_jj - H[j, P] H[P, P]^{-1} H[P, j] over the kept earlier points P.  Points
    near earlier ones (a tiny perturbation) are left out, the others kept."""
    rng = np.random.default_rng(17)
    X = rng.standard_normal((10, 3)) * 0.5
    X[4] = X[1] + 1e-5 * rng.standard_normal(3)
    X[8] = X[6] + 1e-5 * rng.standard_normal(3)
    # a long key (H_jj ~ 1e8) and a near copy: the test is relative to H_jj, so the copy is
    # left out although its absolute residual is far above DEPENDENT_TOL
    X[2] *= 5.5 / np.linalg.norm(X[2])
    X[9] = X[2] + 1e-4 * rng.standard_normal(3)
    H = ow.kernel(X, X, 0.6)
    keep = ow.independent_slots(H)
    P = []
    ref = np.zeros(10, bool)
    for j in range(10):
        g = H[j, j] - (H[j, P] @ np.linalg.solve(H[np.ix_(P, P)], H[P, j]) if P else 0.0)
        if g > ow.DEPENDENT_TOL * H[j, j]:
            ref[j] = True
            P.append(j)
    assert np.array_equal(keep, ref)
    assert not keep[4] and not keep[8] and not keep[9] and keep.sum() == 7
    P9 = [j for j in range(9) if keep[j]]
    g9 = H[9, 9] - H[9, P9] @ np.linalg.solve(H[np.ix_(P9, P9)], H[P9, 9])
    assert g9 > 1e-3 and g9 < ow.DEPENDENT_TOL * H[9, 9]


def test_union_is_more_accurate_than_per_bin_weights():
    """Bounded inputs, 4 bins: the union's weights use every coreset point for every key,
    the per-bin weights only the bin's own; the union's error is the smaller one."""
    Q, K, V = bounded_problem()
    exact = ow.exact_attention(Q, K, V)
    eu, eb = [], []
    for s in range(3):
        u = np.random.default_rng(20 + s).random(32)
        eu.append(ow.rel_fro(ow.forward_binned(Q, K, V, 32, 4, u)["O"], exact))
        eb.append(ow.rel_fro(ow.forward_binned(Q, K, V, 32, 4, u, weights_mode="bin")["O"], exact))
    assert np.mean(eu) < 0.5 * np.mean(eb), (eu, eb)


@pytest.mark.parametrize("delta,kept_expected", [(0.06, True), (0.007, False)])
def test_near_dependent_pair_on_either_side_of_the_tolerance(delta, kept_expected):
    """A key near an earlier coreset key, its relative Schur residual g / H_jj a few times above
    (delta 0.06, about 2^-9) or below (delta 0.007, about 2^-15) DEPENDENT_TOL.  Above, the pair
    is kept and W is numpy's pseudo-inverse form, as for distinct keys.  Below, the point is left
    out: its weight row is zero and the others are the weights of the coreset without it, again
    in numpy's pseudo-inverse form.  Kept, the output equals the full pseudo-inverse's; left
    out, it differs from it (here by about 2 %): that is the cost of the leave-out reading on a
    12-key head whose coreset is nearly all of it, where one more point still moves the
    interpolation."""
    rng = np.random.default_rng(40)
    d, beta = 3, 0.6
    X = rng.standard_normal((12, d)) * 0.9
    e = rng.standard_normal(d)
    X[7] = X[2] + delta * e / np.linalg.norm(e)
    V = rng.standard_normal((12, 2))
    slots = np.arange(9)
    H = ow.kernel(X[slots], X[slots], beta)
    P = [j for j in range(7)]
    g = H[7, 7] - H[7, P] @ np.linalg.solve(H[np.ix_(P, P)], H[P, 7])
    rel = g / H[7, 7]
    assert (rel > ow.DEPENDENT_TOL) == kept_expected
    assert (rel > 2 * ow.DEPENDENT_TOL) if kept_expected else (rel < ow.DEPENDENT_TOL / 2)
    W, kept = ow.weights_union(X, V, slots, beta)
    V1 = np.hstack([V, np.ones((12, 1))])
    keep_idx = slots if kept_expected else np.delete(slots, 7)
    assert kept.tolist() == [True] * 7 + [kept_expected] + [True]
    Wp = np.linalg.pinv(ow.kernel(X[keep_idx], X[keep_idx], beta)) @ ow.kernel(X[keep_idx], X, beta) @ V1
    Wfull = np.zeros_like(W)
    Wfull[keep_idx] = Wp
    assert np.allclose(W, Wfull, rtol=1e-6, atol=1e-8 * np.abs(Wp).max())
    Q = rng.standard_normal((5, d)) * 0.9
    Wall = np.linalg.pinv(H) @ ow.kernel(X[slots], X, beta) @ V1
    Ya, Yb = ow.kernel(Q, X[slots], beta) @ W, ow.kernel(Q, X[slots], beta) @ Wall
    err = ow.rel_fro(Ya[:, :2] / Ya[:, 2:], Yb[:, :2] / Yb[:, 2:])
    assert (err < 1e-8) if kept_expected else (1e-4 < err < 0.1)
