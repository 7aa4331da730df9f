"""Pins of block pivoting (rpcholesky_block): one candidate per round is the plain loop; at any
block size the factor satisfies the Nystroem identity for its accepted pivots (F F^T =
H_{:,S} H_SS^{-1} H_{S,:}, written with a linear solve) and the rows of F at the pivots are
lower triangular in slot order; full rank (every index accepted) reproduces H; an index drawn
twice in a round is left out once; the candidates of a round are draws from the round-start
diagonal (a brute-force linear scan); the trace never grows; snapped uniforms keep the pivots."""
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
    u = np.random.default_rng(seed).random(12)
    a = ow.rpcholesky_block(K, 12, u, 1)
    b = ow.rpcholesky(K, 12, u)
    assert np.array_equal(a["pivots"], b["pivots"]) and a["rank"] == b["rank"] == 12
    assert np.allclose(a["F"], b["F"], rtol=1e-12, atol=1e-13)
    assert np.allclose(a["diag"], b["diag"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_nystroem_identity_and_triangular_pivot_rows(b):
    K = keys(n=60, seed=10 + b)
    beta = ow.beta_of(5)
    u = np.random.default_rng(b).random(16)
    out = ow.rpcholesky_block(K, 16, u, b)
    piv, F = out["pivots"], out["F"]
    valid = piv >= 0
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
    assert np.all(np.diff(out["trace"][: 16 // b * b + 1 : b]) <= 1e-12)


def test_full_rank_reproduces_h():
    """Every index accepted (r = n, forced uniforms walking the remaining mass): F F^T = H."""
    K = keys(n=12, seed=3)
    beta = ow.beta_of(5)
    u = np.zeros(12)
    out = ow.rpcholesky_block(K, 12, u, 1)
    assert out["rank"] == 12
    assert np.allclose(out["F"] @ out["F"].T, ow.kernel(K, K, beta), rtol=1e-10, atol=1e-12)
    # blocks of 3: the same keys, r = n; indices drawn twice are left out, so take the rank
    out3 = ow.rpcholesky_block(K, 12, np.random.default_rng(4).random(12), 3)
    v = out3["pivots"] >= 0
    Fv = out3["F"][:, v]
    S = out3["pivots"][v]
    assert np.allclose(Fv[S] @ Fv[S].T, ow.kernel(K[S], K[S], beta), rtol=1e-10, atol=1e-12)


def test_index_drawn_twice_is_left_out_once():
    K = keys(n=30, seed=5)
    u = np.array([0.3, 0.3, 0.8, 0.1])   # the first two candidates are the same draw
    out = ow.rpcholesky_block(K, 4, u, 4)
    assert out["pivots"][0] >= 0 and out["pivots"][1] == -1
    assert out["rank"] == 3 and np.all(out["F"][:, 1] == 0.0)


def test_candidates_are_draws_from_the_round_start_diagonal():
    K = keys(n=50, seed=6)
    u = np.random.default_rng(7).random(8)
    out = ow.rpcholesky_block(K, 8, u, 4)
    beta = ow.beta_of(5)
    diag = ow.initial_residual(K, beta)
    for k in range(2):
        p = np.maximum(diag, 0)
        T = p.sum()
        for j in range(4):
            acc, s = 0.0, None
            for i in range(50):       # brute force: first index whose running sum passes u T
                acc += p[i]
                if acc > u[4 * k + j] * T:
                    s = i
                    break
            if out["pivots"][4 * k + j] >= 0:
                assert out["pivots"][4 * k + j] == s
        Fk = out["F"][:, 4 * k: 4 * k + 4]
        diag = diag - np.sum(Fk ** 2, 1)
        diag[out["pivots"][4 * k: 4 * k + 4][out["pivots"][4 * k: 4 * k + 4] >= 0]] = 0.0


def test_snapping_keeps_the_pivots():
    K = keys(n=80, seed=8)
    raw = np.random.default_rng(9).random(16)
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
        u = np.random.default_rng(r).random(r)
        eb.append(ow.rel_fro(ow.forward_binned(Q, K, V, r, 1, u, pivot_block=8)["O"], ex))
        ep.append(ow.rel_fro(ow.forward(Q, K, V, r, u)["O"], ex))
    assert eb[1] < eb[0] and ep[1] < ep[0]
    assert eb[0] < 3 * ep[0] and eb[1] < 3 * ep[1], (eb, ep)


def test_block_forward_with_bins_keeps_pivots_in_their_bins():
    K = keys(n=64, seed=14)
    Q = keys(n=5, seed=15)
    V = np.random.default_rng(16).standard_normal((64, 2))
    u = np.random.default_rng(17).random(16)
    out = ow.forward_binned(Q, K, V, 16, 4, u, pivot_block=2)
    for k0, k1, s0, s1 in ow.bin_bounds(64, 16, 4):
        S = out["pivots"][s0:s1]
        assert np.all((S == -1) | ((S >= k0) & (S < k1)))
        ref = ow.rpcholesky_block(K[k0:k1], 4, u[s0:s1], 2)["pivots"]
        assert np.array_equal(np.where(ref >= 0, ref + k0, -1), S)
    with pytest.raises(ValueError):
        ow.forward_binned(Q, K, V, 16, 4, u, weights_mode="bin", pivot_block=2)
