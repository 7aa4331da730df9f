"""Parity of key centring (wc_forward with WC_OPT_CENTER_KEYS) with the oracle run on
center_keys(K): pivots, rank and flags bit-exact under uniforms snapped on the centred keys,
outputs within the tolerances.  Cases: one bin on the resident and the streaming selection,
fp32 and bf16, and bins with union weights; keys carry a large common offset, which the
centring removes.  Also: against exact attention, centring lowers the error on such keys."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow
from tests.gpu_util import TOL, check_output, dev, host, rel, snapped, snapped_binned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


# (name, dtype, H, n, m, d, dv, r, B)
CASES = [
    ("resident", "bf16", 3, 197, 197, 64, 64, 32, 1),
    ("stream_bf16", "bf16", 2, 3000, 120, 128, 128, 96, 1),
    ("stream_f32", "f32", 2, 1024, 64, 64, 128, 40, 1),
    ("bins_union", "bf16", 2, 4096, 100, 64, 64, 128, 8),
]


def offset_inputs(case):
    name, dtype, H, n, m, d, dv, r, B = case
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=900 + CASES.index(case), dtype="f32",
                                  kind="mixture", clip=2.0, clusters=8)
    rng = np.random.default_rng(901 + CASES.index(case))
    K = K + (rng.standard_normal((H, 1, d)) * 0.6).astype(np.float32)   # common offset per head
    if dtype == "bf16":
        Q, K, V = (synth.round_to_bf16(x) for x in (Q, K, V))
    return Q, K, V


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_centred_forward_parity(wc, case):
    name, dtype, H, n, m, d, dv, r, B = case
    Q, K, V = offset_inputs(case)
    Kc = np.stack([ow.center_keys(K[h], dtype) for h in range(H)])
    U = snapped(Kc, r) if B == 1 else snapped_binned(Kc, r, B)
    out = wc.wc_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), r, u_forced=dev(U), bins=B,
                        center_keys=True)
    O, piv, rank, flags = host(out["O"]), host(out["pivots"]), host(out["rank"]), host(out["flags"])
    for h in range(H):
        ref = ow.forward(Q[h], Kc[h], V[h], r, U[h]) if B == 1 else ow.forward_binned(Q[h], Kc[h], V[h], r, B, U[h])
        assert np.array_equal(piv[h], ref["pivots"]), h
        assert rank[h] == ref["rank"] and flags[h] == ref["flags"], (rank[h], flags[h], ref["rank"], ref["flags"])
        check_output(O[h], ref["O"], ref["kappa"], dtype, f"{__name__}:{h}")


def test_centring_lowers_the_error_on_offset_keys(wc):
    case = CASES[1]
    name, dtype, H, n, m, d, dv, r, B = case
    Q, K, V = offset_inputs(case)
    args = (dev(Q, dtype), dev(K, dtype), dev(V, dtype), r)
    Op = host(wc.wc_forward(*args, seed=4)["O"])
    Oc = host(wc.wc_forward(*args, seed=4, center_keys=True)["O"])
    ep = np.mean([rel(Op[h], ow.exact_attention(Q[h], K[h], V[h])) for h in range(H)])
    ec = np.mean([rel(Oc[h], ow.exact_attention(Q[h], K[h], V[h])) for h in range(H)])
    assert ec < ep, (ec, ep)
