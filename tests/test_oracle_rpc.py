"""Pins of the oracle's randomly pivoted Cholesky against facts the pages and the mathematics
fix: a complete pivoted Cholesky reproduces H, the partial factor is the Nystroem
approximation with L = F[S, :] the Cholesky factor of H_SS, the residual diagonal is
diag(H - F F^T), the trace only falls, pivots are distinct, the first pivot is distributed
proportionally to the diagonal, and a two-key case worked by hand."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import philox
from oracle import wildcat as ow


def H_of(K, beta):
    K = np.asarray(K, np.float64)
    return np.exp(beta * K @ K.T)


def small(n=10, d=4, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d)) * 0.7
    return K, 1.0 / np.sqrt(d)


@pytest.mark.parametrize("seed", range(4))
def test_full_rank_reproduces_kernel_matrix(seed):
    K, beta = small(seed=seed)
    n = K.shape[0]
    u = np.random.default_rng(100 + seed).random(n)
    out = ow.rpcholesky(K, n, u, beta)
    H = H_of(K, beta)
    assert out["rank"] == n
    assert np.max(np.abs(out["F"] @ out["F"].T - H)) < 1e-12 * np.max(H)
    assert np.max(np.abs(out["diag"])) < 1e-12 * np.max(H)
    assert sorted(out["pivots"]) == list(range(n))


@pytest.mark.parametrize("seed,r", [(0, 3), (1, 5), (2, 7)])
def test_partial_factor_is_nystroem(seed, r):
    K, beta = small(n=12, seed=seed)
    u = np.random.default_rng(7 + seed).random(r)
    out = ow.rpcholesky(K, r, u, beta)
    S = out["pivots"]
    F = out["F"]
    H = H_of(K, beta)
    # L = F[S, :] is lower triangular with L L^T = H_SS
    L = F[S, :]
    assert np.allclose(np.triu(L, 1), 0.0, atol=1e-15)
    assert np.all(np.diag(L) > 0)
    assert np.allclose(L @ L.T, H[np.ix_(S, S)], rtol=1e-13, atol=1e-13)
    # F F^T = H_{:,S} H_SS^{-1} H_{S,:}
    nys = H[:, S] @ np.linalg.solve(H[np.ix_(S, S)], H[S, :])
    assert np.allclose(F @ F.T, nys, rtol=1e-12, atol=1e-12)
    # H_{:,S} = F L^T (column s_t of H is what the first t+1 columns of F explain)
    assert np.allclose(F @ L.T, H[:, S], rtol=1e-13, atol=1e-13)
    # residual diagonal = diag(H - F F^T), zero at the pivots
    res = np.diag(H) - np.sum(F * F, axis=1)
    res[S] = 0.0
    assert np.allclose(out["diag"], res, atol=1e-13)


def test_factor_rows_given_pivots_match_pivot_loop():
    Q, K, V = synth.make_inputs("vit197", heads=[0])
    u = synth.raw_uniforms(1, 32)[0]
    out = ow.rpcholesky(K[0], 32, u)
    rows = [0, 5, 100, 196] + list(out["pivots"][:3])
    Fr, dr = ow.factor_rows_given_pivots(K[0], out["pivots"], rows)
    assert np.allclose(Fr, out["F"][rows], rtol=1e-9, atol=1e-10)
    nonpiv = [i for i, row in enumerate(rows) if row not in set(out["pivots"])]
    assert np.allclose(dr[nonpiv], out["diag"][np.array(rows)[nonpiv]], atol=1e-9)


def test_trace_nonincreasing_and_decrement():
    Q, K, V = synth.make_inputs("iid1k", heads=[0], n=256, m=8)
    u = synth.raw_uniforms(1, 64)[0]
    out = ow.rpcholesky(K[0], 64, u)
    tr = out["trace"]
    F = out["F"]
    assert np.all(np.diff(tr) <= 1e-12 * tr[0])
    # T_{t+1} = T_t - |F[:, t]|^2 (no residual goes negative here, so clamping is inert)
    assert np.allclose(tr[1:], tr[:-1] - np.sum(F * F, axis=0), rtol=1e-10, atol=1e-10 * tr[0])
    H0 = np.exp(np.sum(K[0].astype(np.float64) ** 2, axis=1) / 8.0)
    assert np.isclose(tr[0], H0.sum(), rtol=1e-14)


def test_pivots_distinct_and_zeroed():
    Q, K, V = synth.make_inputs("img4096", heads=[0], n=512, m=8)
    u = synth.raw_uniforms(1, 128)[0]
    out = ow.rpcholesky(K[0], 128, u)
    S = out["pivots"]
    assert len(set(S.tolist())) == 128
    # set to zero when picked; later columns only subtract rounding-level squares, so a
    # pivot's residual stays <= 0 and it can never be drawn again
    assert np.all(out["diag"][S] <= 0.0) and np.all(out["diag"][S] > -1e-20)


def test_sampling_rule_matches_linear_scan():
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 30))
        diag = rng.random(n) - 0.2  # some negative entries: they carry no mass
        diag[rng.random(n) < 0.2] = 0.0
        u = rng.random()
        s, T, C = ow.sample_pivot(diag, u)
        p = [max(x, 0.0) for x in diag]
        tot = sum(p)
        if tot <= 0:
            assert s == -1
            continue
        acc, pick = 0.0, None
        for i, pi in enumerate(p):
            acc += pi
            if acc > u * tot:
                pick = i
                break
        if pick is None:
            pick = max(i for i, pi in enumerate(p) if pi > 0)
        assert s == pick
        assert p[s] > 0


@pytest.mark.parametrize("diag,u,expect", [
    ([0.0, 1.0], 0.0, 1),             # zero-mass index never drawn, even at u = 0
    ([1.0, 0.0, 1.0], 0.5, 2),        # u T on an interval end goes right, past zero mass
    ([0.5, 0.25, 0.25], 0.75, 2),     # exact dyadic tie at C_1
    ([-1.0, 2.0, 0.0, 2.0], 0.5, 3),  # negative residuals carry no mass
    ([1.0, 1.0, 0.0], 1.0 - 2.0**-24, 1),
])
def test_sampling_rule_ties(diag, u, expect):
    assert ow.sample_pivot(np.array(diag), u)[0] == expect


def test_first_pivot_distribution():
    """P(s_0 = i) = exp(beta |k_i|^2) / T_0, checked by chi-square over Philox draws."""
    from scipy.stats import chisquare

    K, beta = small(n=8, d=4, seed=11)
    w = np.exp(beta * np.sum(K * K, axis=1))
    counts = np.zeros(8)
    draws = 20000
    for sd in range(draws):
        u = [philox.pivot_uniform(sd, 0, 0)]
        counts[ow.rpcholesky(K, 1, u, beta)["pivots"][0]] += 1
    assert chisquare(counts, draws * w / w.sum()).pvalue > 1e-4


def test_two_keys_by_hand():
    """n = 2, d = 1, beta = 1, keys a and b, first pivot forced to key a:
    F[:, 0] = (e^{a^2/2}, e^{ab - a^2/2});  residual of b = e^{b^2} (1 - e^{-(a-b)^2})."""
    a, b = 0.8, -0.3
    K = np.array([[a], [b]])
    ea, eb = np.exp(a * a), np.exp(b * b)
    u0 = 0.5 * ea / (ea + eb)  # inside key a's interval
    out = ow.rpcholesky(K, 1, [u0], beta=1.0)
    assert out["pivots"][0] == 0
    assert np.isclose(out["trace"][0], ea + eb, rtol=1e-15)
    assert np.allclose(out["F"][:, 0], [np.exp(a * a / 2), np.exp(a * b - a * a / 2)], rtol=1e-14)
    assert out["diag"][0] == 0.0
    assert np.isclose(out["diag"][1], eb * (1 - np.exp(-(a - b) ** 2)), rtol=1e-13)
    assert np.isclose(out["trace"][1], eb * (1 - np.exp(-(a - b) ** 2)), rtol=1e-13)
    # second step must take key b and then the factor is complete
    out2 = ow.rpcholesky(K, 2, [u0, 0.3], beta=1.0)
    assert list(out2["pivots"]) == [0, 1]
    assert np.isclose(out2["F"][1, 1], np.sqrt(eb * (1 - np.exp(-(a - b) ** 2))), rtol=1e-13)
    assert abs(out2["F"][0, 1]) < 1e-15  # zero up to rounding: key a is already explained


def test_breakdown_when_residual_vanishes():
    """All-zero keys: H is the all-ones matrix, exactly rank one, so step 1 finds T = 0."""
    K = np.zeros((6, 4))
    out = ow.rpcholesky(K, 4, [0.1, 0.2, 0.3, 0.4])
    assert out["rank"] == 1
    assert out["flags"] & ow.FLAG_BREAKDOWN
    assert list(out["pivots"][1:]) == [-1, -1, -1]
    assert np.all(out["F"][:, 1:] == 0.0)
    assert out["trace"][1] == 0.0


def test_nonfinite_input_flagged():
    K = np.ones((6, 4)) * 0.1
    K[2, 1] = np.nan
    out = ow.rpcholesky(K, 3, [0.1, 0.2, 0.3])
    assert out["flags"] & ow.FLAG_NONFINITE
    assert out["rank"] == 0


def test_snap_uniforms_keeps_pivots_and_centres():
    Q, K, V = synth.make_inputs("img4096", heads=[1], n=1024, m=8)
    raw = synth.raw_uniforms(1, 64)[0]
    snapped, margin = ow.snap_uniforms(K[0], 64, raw)
    a = ow.rpcholesky(K[0], 64, raw)
    b = ow.rpcholesky(K[0], 64, snapped)
    assert np.array_equal(a["pivots"], b["pivots"])
    assert np.all(margin > 0)
    assert np.all((snapped * 2**24) == np.round(snapped * 2**24))
    # the snapped value sits at the centre of the selected interval (up to 2^-24 rounding)
    diag = ow.initial_residual(K[0], 1 / 8.0)
    s, T, C = ow.sample_pivot(diag, snapped[0])
    lo = C[s - 1] if s else 0.0
    assert abs(snapped[0] * T - (lo + C[s]) / 2) <= 2.0**-24 * T


@pytest.mark.parametrize("seed", range(3))
def test_follow_own_pivots_reproduces_the_loop(seed):
    """Driven by its own pivots, the follow loop is the pivot loop: the same factor, every draw
    inside the interval of its pivot, and the draw's own choice equal to that pivot."""
    K, beta = small(n=40, d=6, seed=seed)
    r = 15
    u = np.random.default_rng(300 + seed).random(r)
    out = ow.rpcholesky(K, r, u, beta)
    f = ow.rpcholesky_follow(K, out["pivots"], u, beta)
    assert np.array_equal(f["chosen"], out["pivots"])
    assert np.array_equal(f["F"], out["F"])
    assert np.allclose(f["T"], out["trace"][:r], rtol=1e-13)
    uT = u * f["T"]
    assert np.all((f["lo"] <= uT) & (uT < f["hi"]))
    # the interval of pivot s is [sum of masses before s, ... including s) at that step
    diag = ow.initial_residual(K, beta)
    s0 = out["pivots"][0]
    assert f["lo"][0] == pytest.approx(np.sum(diag[:s0]), rel=1e-13)
    assert f["hi"][0] - f["lo"][0] == pytest.approx(diag[s0], rel=1e-12)


def test_follow_flags_a_pivot_the_draw_does_not_select():
    """A pivot sequence that departs from the draws at step k: the draw's own choice differs
    there, u_k T_k lies outside the given pivot's interval, and the steps before agree."""
    K, beta = small(n=30, d=5, seed=7)
    r, k = 10, 4
    u = np.random.default_rng(9).random(r)
    out = ow.rpcholesky(K, r, u, beta)
    piv = out["pivots"].copy()
    other = [i for i in range(30) if i not in piv[:k + 1]][0]
    piv[k] = other
    f = ow.rpcholesky_follow(K, piv, u, beta)
    assert np.array_equal(f["chosen"][:k], piv[:k])
    assert f["chosen"][k] == out["pivots"][k] != other
    uT = u[k] * f["T"][k]
    assert not (f["lo"][k] <= uT < f["hi"][k])
