"""Pins of block pivoting (rpcholesky_block): one candidate per round is the plain loop; at any
block size the factor satisfies the Nystroem identity for its pivots (F F^T =
H_{:,S} H_SS^{-1} H_{S,:}, written with a linear solve), the rows of F at the pivots are lower
triangular and the pivots fill slots 0 .. rank-1; full rank reproduces H; an index drawn twice
never happens (a round's draws are without replacement: a brute-force scan of the masses with
the earlier draws removed); a skewed residual (a few keys holding nearly all the mass) fills in
one round; snapped uniforms keep the pivots; the block-pivoted forward is close to the plain
one; a near copy of a long key is passed over (relative leave-out test)."""
import numpy as np
import pytest

from oracle import wildcat as ow


def keys(n=40, d=5, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d))
    return K * np.minimum(1.0, 1.5 / np.linalg.norm(K, axis=1, keepdims=True))


@pytest.mark.parametrize("seed", range(4))
def test_one_candidate_per_round_is_the_plain_loop(seed):
    K = keys(seed=seed)
    u = np.random.default_rng(seed).random(48)
    a = ow.rpcholesky_block(K, 12, u, 1)
    b = ow.rpcholesky(K, 12, u)
    assert np.array_equal(a["pivots"], b["pivots"]) and a["rank"] == b["rank"] == 12
    assert np.allclose(a["F"], b["F"], rtol=1e-12, atol=1e-13)
    assert np.allclose(a["diag"], b["diag"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_nystroem_identity_and_triangular_pivot_rows(b):
    K = keys(n=60, seed=10 + b)
    beta = ow.beta_of(5)
    u = np.random.default_rng(b).random(64)
    out = ow.rpcholesky_block(K, 16, u, b)
    piv, F = out["pivots"], out["F"]
    valid = piv >= 0
    assert out["rank"] == 16 and np.all(valid)
    S = piv[valid]
    Fv = F[:, valid]
    H = ow.kernel(K, K, beta)
    HS = H[:, S]
    assert np.allclose(Fv @ Fv.T, HS @ np.linalg.solve(H[np.ix_(S, S)], HS.T), rtol=1e-9, atol=1e-10)
    L = Fv[S]
    assert np.allclose(np.triu(L, 1), 0.0, atol=1e-12) and np.all(np.diag(L) > 0)
    assert np.all(F[:, ~valid] == 0.0)
    expect = np.diag(H) - np.sum(Fv ** 2, 1)
    expect[S] = 0.0
    assert np.allclose(out["diag"], expect, rtol=1e-9, atol=1e-10)
    nz = np.nonzero(out["trace"])[0]
    assert nz[0] == 0 and nz[-1] == 16 and np.all(np.diff(out["trace"][nz]) <= 1e-12)


def test_full_rank_reproduces_h():
    """Every index accepted (r = n, forced uniforms walking the remaining mass): F F^T = H."""
    K = keys(n=12, seed=3)
    beta = ow.beta_of(5)
    u = np.zeros(48)
    out = ow.rpcholesky_block(K, 12, u, 1)
    assert out["rank"] == 12
    assert np.allclose(out["F"] @ out["F"].T, ow.kernel(K, K, beta), rtol=1e-10, atol=1e-12)
    # blocks of 3, r = n: repeated draws are passed over, later rounds fill every slot
    out3 = ow.rpcholesky_block(K, 12, np.random.default_rng(4).random(48), 3)
    assert out3["rank"] == 12 and sorted(out3["pivots"]) == list(range(12))
    assert np.allclose(out3["F"] @ out3["F"].T, ow.kernel(K, K, beta), rtol=1e-9, atol=1e-11)


def test_draws_of_a_round_are_distinct():
    """The same uniform twice in a round: the second draw skips the first's index."""
    K = keys(n=30, seed=5)
    u = np.array([0.3, 0.3, 0.8, 0.1] + [0.5] * 12)
    out = ow.rpcholesky_block(K, 4, u, 4)
    assert out["rank"] == 4 and len(set(out["pivots"])) == 4
    first = ow.rpcholesky_block(K, 1, u[:4], 1)["pivots"][0]
    assert out["pivots"][0] == first


def test_skewed_residual_fills_in_one_round():
    """Three keys hold nearly all the mass: the round's first draws take them, the later ones
    (without replacement) spread over the rest, and one round fills the eight slots."""
    rng = np.random.default_rng(18)
    K = rng.standard_normal((200, 6)) * 0.3
    K[[5, 70, 150]] *= 12.0
    out = ow.rpcholesky_block(K, 8, rng.random(32), 8)
    assert out["rank"] == 8
    assert set(out["pivots"][:3]) == {5, 70, 150}
    assert np.count_nonzero(out["trace"]) == 2      # one round: totals before it and after


def test_candidates_are_draws_from_the_round_start_diagonal():
    """Well spread keys, two rounds of four: the pivots are, in order, brute-force inverse-CDF
    draws on each round's start residual with the round's earlier draws removed."""
    K = keys(n=50, seed=6)
    u = np.random.default_rng(7).random(32)
    out = ow.rpcholesky_block(K, 8, u, 4)
    assert out["rank"] == 8
    beta = ow.beta_of(5)
    diag = ow.initial_residual(K, beta)
    for k in range(2):
        drawn = []
        for j in range(4):
            p = np.maximum(diag, 0)
            p[drawn] = 0.0
            T = p.sum()
            acc, s = 0.0, None
            for i in range(50):       # brute force: first index whose running sum passes u T
                acc += p[i]
                if acc > u[4 * k + j] * T:
                    s = i
                    break
            drawn.append(s)
            assert out["pivots"][4 * k + j] == s
        Fk = out["F"][:, 4 * k: 4 * k + 4]
        diag = diag - np.sum(Fk ** 2, 1)
        diag[out["pivots"][4 * k: 4 * k + 4]] = 0.0


def test_snapping_keeps_the_pivots():
    K = keys(n=80, seed=8)
    raw = np.random.default_rng(9).random(64)
    U = ow.snap_uniforms_block(K, 16, 4, raw)
    a = ow.rpcholesky_block(K, 16, raw, 4)
    c = ow.rpcholesky_block(K, 16, U.astype(np.float64), 4)
    assert np.array_equal(a["pivots"], c["pivots"])


def test_block_forward_is_close_to_exact_and_to_the_plain_forward():
    """Block-pivoted forward (union weights over the accepted pivots): its error against exact
    attention is of the plain forward's order, and both fall with r."""
    rng = np.random.default_rng(11)
    n, d = 300, 8
    K = keys(n=n, d=d, seed=12)
    Q = keys(n=40, d=d, seed=13)
    V = rng.standard_normal((n, 3))
    ex = ow.exact_attention(Q, K, V)
    eb, ep = [], []
    for r in (16, 48):
        u = np.random.default_rng(r).random(4 * r)
        eb.append(ow.rel_fro(ow.forward_binned(Q, K, V, r, 1, u, pivot_block=8)["O"], ex))
        ep.append(ow.rel_fro(ow.forward(Q, K, V, r, u[:r])["O"], ex))
    assert eb[1] < eb[0] and ep[1] < ep[0]
    assert eb[0] < 3 * ep[0] and eb[1] < 3 * ep[1], (eb, ep)


def test_block_forward_with_bins_keeps_pivots_in_their_bins():
    K = keys(n=64, seed=14)
    Q = keys(n=5, seed=15)
    V = np.random.default_rng(16).standard_normal((64, 2))
    u = np.random.default_rng(17).random(64)
    for mode in ("union", "bin"):
        out = ow.forward_binned(Q, K, V, 16, 4, u, weights_mode=mode, pivot_block=2)
        for k0, k1, s0, s1 in ow.bin_bounds(64, 16, 4):
            S = out["pivots"][s0:s1]
            assert np.all((S >= k0) & (S < k1))
            ref = ow.rpcholesky_block(K[k0:k1], 4, u[4 * s0:4 * s1], 2)["pivots"]
            assert np.array_equal(ref + k0, S)


def test_near_copy_of_a_long_key_is_passed_over():
    """A long key (H_ss ~ 1e8) and a near copy of it hold nearly all the mass: the copy's
    residual after the key is accepted is about 1 in absolute terms but ~1e-8 of H_ss, so the
    relative test passes over it and the slot goes to a later draw."""
    rng = np.random.default_rng(19)
    K = rng.standard_normal((100, 3)) * 0.3
    K[10] = rng.standard_normal(3)
    K[10] *= 5.5 / np.linalg.norm(K[10])
    K[60] = K[10] + 1e-4 * rng.standard_normal(3)
    beta = 0.6
    u = rng.random(32)
    out = ow.rpcholesky_block(K, 4, u, 4, beta=beta)
    piv = list(out["pivots"])
    assert out["rank"] == 4
    assert (10 in piv) != (60 in piv)   # exactly one of the pair
    first = piv[0]
    other = 60 if first == 10 else 10
    g = ow.kernel(K[[other]], K[[other]], beta)[0, 0] - ow.kernel(K[[other]], K[[first]], beta)[0, 0] ** 2 / ow.kernel(K[[first]], K[[first]], beta)[0, 0]
    assert 1e-3 < g < ow.DEPENDENT_TOL * ow.kernel(K[[other]], K[[other]], beta)[0, 0]


def test_block_draw_margins_and_slot_rounds():
    """The block loop's record of each draw: the distance from u T to the nearer end of the
    interval it selects (over T), checked against a plain loop over the running sums of the
    first round's masses with the earlier candidates removed; every slot's round is one that
    ran, non-decreasing in slot order."""
    rng = np.random.default_rng(41)
    K = rng.standard_normal((60, 5)) * 0.6
    r, b = 12, 4
    u = rng.random(ow.BLOCK_DRAWS * r)
    out = ow.rpcholesky_block(K, r, u, b)
    p = ow.initial_residual(K, 1.0 / np.sqrt(5))
    taken = []
    for j in range(b):
        q = [0.0 if i in taken else p[i] for i in range(len(p))]
        T = sum(q)
        run, s = 0.0, None
        for i, x in enumerate(q):
            if x > 0 and run + x > u[j] * T:
                s, lo, hi = i, run, run + x
                break
            run += x
        taken.append(s)
        assert out["margins"][j] == pytest.approx(min(u[j] * T - lo, hi - u[j] * T) / T, rel=1e-9, abs=1e-15)
    used = out["slot_round"][: out["rank"]]
    assert np.all(used >= 0) and np.all(np.diff(used) >= 0)
    assert np.all(np.isfinite(out["margins"][: b * (used[-1] + 1)]))


def test_snap_with_pivots_returns_the_runs_pivots():
    rng = np.random.default_rng(42)
    K = rng.standard_normal((50, 4)) * 0.5
    raw = rng.random(9)
    U, margin, piv = ow.snap_uniforms(K, 9, raw, with_pivots=True)
    assert np.array_equal(piv, ow.rpcholesky(K, 9, U)["pivots"])
    assert np.array_equal(piv, ow.rpcholesky(K, 9, raw)["pivots"])
