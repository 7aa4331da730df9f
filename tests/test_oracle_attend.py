"""Pins of the oracle's weights, coreset attention and exact attention: closed forms at
r = n (Nystroem with every key is exact) and r = 1, interpolation at the pivot keys, the
pages' pseudo-inverse form of the weights, the factor form W = L^{-T} F^T [V, 1], error that
falls as the coreset grows, and invariances / special cases of exact softmax attention."""
import numpy as np
import pytest
from scipy.special import softmax

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow


def rand_problem(n=12, m=9, d=4, dv=3, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((m, d)) * 0.8, rng.standard_normal((n, d)) * 0.8,
            rng.standard_normal((n, dv)))


def test_exact_attention_matches_library_softmax():
    Q, K, V = rand_problem(seed=1)
    beta = 0.5
    ref = softmax(beta * Q @ K.T, axis=1) @ V
    assert np.allclose(ow.exact_attention(Q, K, V, beta), ref, rtol=1e-13, atol=1e-14)


def test_exact_attention_invariances_and_special_cases():
    Q, K, V = rand_problem(seed=2)
    O = ow.exact_attention(Q, K, V)
    # global key centring leaves softmax attention unchanged (pages, "Methodik" part 3)
    assert np.allclose(ow.exact_attention(Q, K - K.mean(axis=0), V), O, rtol=1e-12, atol=1e-13)
    # zero queries or identical keys: uniform weights -> mean of V
    assert np.allclose(ow.exact_attention(np.zeros_like(Q), K, V), np.tile(V.mean(0), (9, 1)))
    assert np.allclose(ow.exact_attention(Q, np.tile(K[:1], (12, 1)), V), np.tile(V.mean(0), (9, 1)))
    # constant values come out unchanged
    assert np.allclose(ow.exact_attention(Q, K, np.full_like(V, 2.5)), 2.5)


@pytest.mark.parametrize("seed", range(3))
def test_full_coreset_is_exact_attention(seed):
    Q, K, V = rand_problem(seed=seed)
    n = K.shape[0]
    u = np.random.default_rng(seed).random(n)
    out = ow.forward(Q, K, V, n, u)
    assert np.allclose(out["O"], ow.exact_attention(Q, K, V), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("r", [1, 3, 6])
def test_queries_at_pivot_keys_are_exact(r):
    """Nystroem interpolates at the coreset: a query equal to a pivot key gets the exact row."""
    Q, K, V = rand_problem(seed=4)
    u = np.random.default_rng(r).random(r)
    rpc = ow.rpcholesky(K, r, u)
    S = rpc["pivots"]
    W = ow.weights(K, V, S)
    O, denom, kappa = ow.attend(K[S], K, S, W)
    assert np.allclose(O, ow.exact_attention(K[S], K, V), rtol=1e-10, atol=1e-12)


def test_single_pivot_closed_form():
    """r = 1: every output row is the exact attention row of the pivot key itself."""
    Q, K, V = rand_problem(seed=5)
    out = ow.forward(Q, K, V, 1, [0.37])
    s = out["pivots"][0]
    row = softmax(K[s] @ K.T / 2.0) @ V  # beta = 1/sqrt(4)
    assert np.allclose(out["O"], np.tile(row, (Q.shape[0], 1)), rtol=1e-12, atol=1e-13)


def test_weights_equal_pages_pseudoinverse_form():
    """W = h(K_S,K_S)^+ h(K_S,K) [V, 1] as the pages write it (pseudo-inverse)."""
    Q, K, V = synth.make_inputs("vit197", heads=[3])
    u = synth.raw_uniforms(1, 32)[0]
    S = ow.rpcholesky(K[0], 32, u)["pivots"]
    Kd = K[0].astype(np.float64)
    beta = 1 / 8.0
    hSS = np.exp(beta * Kd[S] @ Kd[S].T)
    hSK = np.exp(beta * Kd[S] @ Kd.T)
    V1 = np.hstack([V[0], np.ones((197, 1))])
    ref = np.linalg.pinv(hSS, rcond=1e-13) @ hSK @ V1
    W = ow.weights(K[0], V[0], S)
    assert ow.rel_fro(W, ref) < 1e-8


def test_weights_equal_factor_form():
    """With L = F[S, :]: W = L^{-T} F^T [V, 1] (H_{:,S} = F L^T, H_SS = L L^T)."""
    from scipy.linalg import solve_triangular

    Q, K, V = synth.make_inputs("img4096", heads=[0], n=600, m=8)
    u = synth.raw_uniforms(1, 48)[0]
    rpc = ow.rpcholesky(K[0], 48, u)
    S, F = rpc["pivots"], rpc["F"]
    V1 = np.hstack([V[0], np.ones((600, 1))])
    Wf = solve_triangular(F[S, :], F.T @ V1, lower=True, trans="T")
    assert ow.rel_fro(ow.weights(K[0], V[0], S), Wf) < 1e-9


def test_error_falls_as_coreset_grows():
    """Approximation error against exact attention falls with r and vanishes at r = n
    (pages: error decays super-polynomially; the FlashAttention-2 comparison shows error
    falling; the guarantee is for bounded inputs, so rows are clipped to norm 2).  Mean over
    16 draws of the relative Frobenius error, n = 64, d = 4."""
    rs = [1, 2, 4, 8, 16, 32, 64]
    errs = np.zeros(len(rs))
    for sd in range(16):
        Q, K, V = (x[0] for x in synth.random_inputs(1, 64, 32, 4, 4, seed=100 + sd, clip=2.0))
        ex = ow.exact_attention(Q, K, V)
        rng = np.random.default_rng(sd)
        for j, r in enumerate(rs):
            out = ow.forward(Q, K, V, r, rng.random(r))
            errs[j] += ow.rel_fro(out["O"], ex) / 16
    assert np.all(np.diff(errs) < 0), errs
    assert errs[-1] < 1e-8
    assert errs[0] > 0.1


def test_denominators_positive_on_workloads():
    for name in ["iid1k", "vit197"]:
        w = synth.WORKLOADS[name]
        Q, K, V = synth.make_inputs(name, heads=[0])
        out = ow.forward(Q[0], K[0], V[0], w.r, synth.raw_uniforms(1, w.r)[0])
        assert np.all(out["denom"] > 0)
        assert out["flags"] == 0
        assert np.max(out["kappa"]) < 10
