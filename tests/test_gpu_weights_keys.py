"""wc_weights_keys: the Nystroem weights from the keys for any pivot set, W = H_SS^+ H_{S,:} [V, 1]
("Methodik" part 2 of the German page), against the oracle's weights_union (the plain
definition, with the leave-out reading for numerically dependent points):
  - pivots of wc_rpcholesky, where the result also equals wc_weights from the factor;
  - random pivot sets (not selected by the pivot loop), checked through the attention output;
  - a repeated pivot (left out once: zero row, WC_FLAG_DEPENDENT), slots past the rank and -1
    slots (empty: zero rows, no flag)."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow
from tests.gpu_util import check_output, dev, host, rel, snapped

pytestmark = pytest.mark.gpu

FLAG_DEPENDENT = 8


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


def _inputs(H, n, m, d, dv, dtype, seed, kind="iid_clip"):
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=seed, dtype=dtype, kind=kind, clip=2.0)
    if dtype == "bf16":
        Q, K, V = synth.round_to_bf16(Q), synth.round_to_bf16(K), synth.round_to_bf16(V)
    return Q, K, V


@pytest.mark.parametrize("dtype,H,n,d,dv,r", [("f32", 2, 3000, 128, 64, 150), ("f32", 1, 4096, 64, 128, 256)])
def test_rpcholesky_pivots(wc, dtype, H, n, d, dv, r):
    """On the pivot loop's own pivots: equal to the oracle's weights and to wc_weights.  (bf16
    keys form H_{S,:}[V, 1] with bf16 probabilities, whose rounding the solve amplifies by the
    conditioning of H_SS: about 7 % in W already at condition 800, emulated on the CPU; bf16 is
    checked through the attention output below.)"""
    _, K, V = _inputs(H, n, 1, d, dv, dtype, seed=970 + r)
    Kd, Vd = dev(K, dtype), dev(V, dtype)
    rpc = wc.wc_rpcholesky(Kd, r, u_forced=dev(snapped(K, r)))
    W, flags = wc.wc_weights_keys(Kd, Vd, rpc["pivots"], rpc["rank"])
    Wf = host(wc.wc_weights(Vd, rpc["pivots"], rpc["rank"], rpc["F"]))
    W, piv = host(W), host(rpc["pivots"])
    assert not host(flags).any()
    tol = 1e-3   # the weights parity's fp32 tolerance
    for h in range(H):
        Wo, kept = ow.weights_union(K[h], V[h], piv[h])
        assert kept.all()
        assert rel(W[h], Wo) < tol, (h, rel(W[h], Wo))
        assert rel(W[h], Wf[h]) < tol, (h, rel(W[h], Wf[h]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_pivots_through_attention(wc, dtype):
    """Pivot sets the loop did not choose: the attention over them with these weights."""
    import torch

    H, n, m, d, dv, r = 3, 2500, 300, 64, 128, 200
    Q, K, V = _inputs(H, n, m, d, dv, dtype, seed=975)
    rng = np.random.default_rng(976)
    piv = np.stack([rng.choice(n, r, replace=False) for _ in range(H)]).astype(np.int32)
    rank = torch.full((H,), r, dtype=torch.int32, device="cuda")
    pd = torch.from_numpy(piv).cuda()
    Kd = dev(K, dtype)
    W, flags = wc.wc_weights_keys(Kd, dev(V, dtype), pd, rank)
    O, aflags = wc.wc_attend(dev(Q, dtype), Kd, pd, rank, W)
    O = host(O)
    assert not host(flags).any() and not host(aflags).any()
    for h in range(H):
        Wo, kept = ow.weights_union(K[h], V[h], piv[h])
        assert kept.all()
        if dtype == "f32":
            assert rel(host(W)[h], Wo) < 1e-3, (h, rel(host(W)[h], Wo))
        Oo, _, kappa = ow.attend(Q[h], K[h], piv[h], Wo)
        check_output(O[h], Oo, kappa, dtype, f"{__name__}:{dtype}:{h}")


def test_repeats_rank_and_empty_slots(wc):
    """Head 0 repeats a key (the later slot is left out and flagged); head 1 has a rank below
    r and a -1 slot (empty, not flagged)."""
    import torch

    H, n, d, dv, r = 2, 2000, 64, 64, 100
    _, K, V = _inputs(H, n, 1, d, dv, "f32", seed=980)
    rng = np.random.default_rng(981)
    piv = np.stack([rng.choice(n, r, replace=False) for _ in range(H)]).astype(np.int32)
    piv[0, 40] = piv[0, 7]
    piv[1, 30] = -1
    rank_h = np.array([r, 80], np.int32)
    W, flags = wc.wc_weights_keys(dev(K), dev(V), torch.from_numpy(piv).cuda(), torch.from_numpy(rank_h).cuda())
    W, flags = host(W), host(flags)
    assert flags[0] & FLAG_DEPENDENT and not (flags[1] & FLAG_DEPENDENT), flags
    for h in range(H):
        slots = np.where(np.arange(r) < rank_h[h], piv[h], -1)
        Wo, kept = ow.weights_union(K[h], V[h], slots)
        assert np.all(W[h][~kept] == 0.0)
        assert rel(W[h], Wo) < 1e-3, (h, rel(W[h], Wo))
        assert kept.sum() == (r - 1 if h == 0 else 79)


def test_union_past_the_one_launch_back_substitution(wc):
    """r = 2560: five ranges of the backward substitution (the top one holding the padding
    rows past r is full, the products below each range span 32 row blocks), still the oracle's
    weights."""
    import torch

    H, n, d, dv, r = 1, 8192, 64, 64, 2560
    _, K, V = _inputs(H, n, 1, d, dv, "f32", seed=985)
    K = K * 2.0   # spread keys: H_SS of 2560 random points at condition about 1e3
    rng = np.random.default_rng(986)
    piv = np.stack([rng.choice(n, r, replace=False) for _ in range(H)]).astype(np.int32)
    rank = torch.full((H,), r, dtype=torch.int32, device="cuda")
    W, flags = wc.wc_weights_keys(dev(K), dev(V), torch.from_numpy(piv).cuda(), rank)
    W, flags = host(W), host(flags)
    Wo, kept = ow.weights_union(K[0], V[0], piv[0])
    assert kept.all() and not flags[0] & FLAG_DEPENDENT
    assert rel(W[0], Wo) < 1e-3, rel(W[0], Wo)
