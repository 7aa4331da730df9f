"""Pins of the compressed-KV-cache oracle (compress, exact_rows, decode): a cache of exact rows
is exact softmax attention (scipy's softmax, a different code path); a full-rank compressed
prefix followed by exact rows of the later tokens is exact attention over the whole sequence;
decode over a compressed prefix is the forward's output for the same queries, in both bin
modes; queries at coreset keys get exact rows over the prefix; empty slots are zero rows."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import wildcat as ow


def rand(n, d, dv, seed, scale=0.7):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)) * scale, rng.standard_normal((n, dv))


def test_exact_rows_are_softmax_attention():
    K, V = rand(40, 8, 3, 0)
    Q = np.random.default_rng(1).standard_normal((6, 8)) * 0.7
    KR, WR = ow.exact_rows(K, V)
    P = softmax(Q @ K.T / np.sqrt(8), axis=1)
    assert np.allclose(ow.decode(Q, KR, WR), P @ V, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("B", [1, 2])
def test_full_rank_prefix_plus_exact_suffix_is_exact(B):
    """Prefix of 16 keys compressed at r = 16 (exact Nystroem), then 10 later tokens appended as
    exact rows: decode equals exact attention over all 26 tokens."""
    K, V = rand(26, 6, 4, 2)
    Q = np.random.default_rng(3).standard_normal((5, 6)) * 0.7
    u = np.random.default_rng(4).random(16)
    KR, WR, piv, rank, _ = ow.compress(K[:16], V[:16], 16, u, B=B)
    assert rank == 16
    Ks, Ws = ow.exact_rows(K[16:], V[16:])
    O = ow.decode(Q, np.vstack([KR, Ks]), np.vstack([WR, Ws]))
    assert np.allclose(O, ow.exact_attention(Q, K, V), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("B,mode", [(1, "union"), (4, "union"), (4, "bin")])
def test_decode_over_compressed_prefix_is_the_forward(B, mode):
    K, V = rand(64, 8, 5, 5)
    Q = np.random.default_rng(6).standard_normal((7, 8)) * 0.7
    u = np.random.default_rng(7).random(12)
    KR, WR, piv, rank, flags = ow.compress(K, V, 12, u, B=B, weights_mode=mode)
    ref = ow.forward(Q, K, V, 12, u) if B == 1 else ow.forward_binned(Q, K, V, 12, B, u, weights_mode=mode)
    assert np.array_equal(piv, ref["pivots"]) and rank == ref["rank"]
    assert np.allclose(ow.decode(Q, KR, WR), ref["O"], rtol=1e-10, atol=1e-12)


def test_queries_at_coreset_keys_decode_exact_rows():
    K, V = rand(50, 6, 3, 8)
    u = np.random.default_rng(9).random(10)
    KR, WR, piv, _, _ = ow.compress(K, V, 10, u, B=2)
    assert np.allclose(ow.decode(KR, KR, WR), ow.exact_attention(KR, K, V), rtol=1e-8, atol=1e-10)


def test_empty_slots_are_zero_rows():
    """All keys of bin 0 are zero (rank one there): its other slots stay empty, and their cache
    rows are zero keys with zero weights, which add nothing."""
    K, V = rand(16, 4, 3, 10)
    K[:8] = 0.0
    u = np.random.default_rng(11).random(6)
    KR, WR, piv, rank, _ = ow.compress(K, V, 6, u, B=2)
    assert np.all(piv[1:3] == -1) and rank == 4
    assert np.all(KR[1:3] == 0.0) and np.all(WR[1:3] == 0.0)
    Q = np.random.default_rng(12).standard_normal((4, 4))
    keep = piv >= 0
    assert np.allclose(ow.decode(Q, KR, WR), ow.decode(Q, KR[keep], WR[keep]), rtol=1e-12, atol=1e-14)
