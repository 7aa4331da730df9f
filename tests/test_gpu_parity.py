"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by element.

Pivots must match bit-exactly under forced uniforms that the oracle snapped to the centres of
their CDF intervals; F, the residual diagonal, the trace, W and O must match within the
stated tolerances.  Cases span both device paths (resident: bf16, n <= 256, r <= 32;
streaming: everything else), several row tiles with ragged tails, d and dv of 64 and 128,
r = 1, r = n, r not a multiple of 32, and the degenerate inputs of the method."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import philox
from oracle import wildcat as ow
from tests.gpu_util import TOL, check_output, dev, host, pivot_report, rel, snapped

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


# (name, dtype, kind, H, n, m, d, dv, r)
CASES = [
    ("resident_vit", "bf16", "mixture", 6, 197, 197, 64, 64, 32),
    ("resident_d128", "bf16", "mixture", 3, 64, 50, 128, 128, 17),
    ("resident_d64_dv128", "bf16", "iid_clip", 2, 130, 70, 64, 128, 24),
    ("resident_r1", "bf16", "mixture", 2, 256, 33, 64, 64, 1),
    ("resident_r_eq_n", "bf16", "iid_clip", 2, 32, 40, 64, 64, 32),
    ("stream_f32_iid", "f32", "iid_clip", 1, 1024, 300, 64, 64, 32),
    ("stream_f32_d128", "f32", "iid_clip", 2, 300, 77, 128, 128, 40),
    ("stream_bf16_img", "bf16", "mixture", 2, 4096, 500, 64, 64, 64),
    ("stream_bf16_ragged", "bf16", "mixture", 3, 3001, 129, 128, 128, 48),
    ("stream_bf16_r33", "bf16", "kv_outlier", 2, 1000, 64, 64, 128, 33),
    ("stream_f32_dv64_d128", "f32", "mixture", 1, 2500, 200, 128, 64, 70),
]


def case_inputs(case):
    name, dtype, kind, H, n, m, d, dv, r = case
    seed = 500 + CASES.index(case)
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=seed, dtype=dtype, kind=kind, clip=2.5,
                                  clusters=8)
    return Q, K, V


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rpcholesky_parity(wc, case):
    name, dtype, kind, H, n, m, d, dv, r = case
    Q, K, V = case_inputs(case)
    U = snapped(K, r)
    out = wc.wc_rpcholesky(dev(K, dtype), r, u_forced=dev(U))
    piv, F, diag, trace = host(out["pivots"]), host(out["F"]), host(out["diag"]), host(out["trace"])
    rank, flags = host(out["rank"]), host(out["flags"])
    for h in range(H):
        ref = ow.rpcholesky(K[h], r, U[h])
        assert rank[h] == ref["rank"] and flags[h] == ref["flags"], (h, rank[h], flags[h])
        assert np.array_equal(piv[h], ref["pivots"]), (h, piv[h], ref["pivots"])
        assert rel(F[h].T, ref["F"]) < 1e-4, rel(F[h].T, ref["F"])
        d0 = ow.initial_residual(K[h], 1 / np.sqrt(d))
        assert np.max(np.abs(diag[h] - ref["diag"])) < 1e-5 * d0.max() * np.sqrt(r)
        assert np.allclose(trace[h], ref["trace"], rtol=1e-5, atol=1e-6 * ref["trace"][0])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_weights_and_attend_parity(wc, case):
    name, dtype, kind, H, n, m, d, dv, r = case
    Q, K, V = case_inputs(case)
    U = snapped(K, r)
    Kd, Vd, Qd = dev(K, dtype), dev(V, dtype), dev(Q, dtype)
    rpc = wc.wc_rpcholesky(Kd, r, u_forced=dev(U))
    W = host(wc.wc_weights(Vd, rpc["pivots"], rpc["rank"], rpc["F"]))
    piv = host(rpc["pivots"])
    Wor = []
    for h in range(H):
        S = piv[h][piv[h] >= 0]
        Wo = ow.weights(K[h], V[h], S)
        Wor.append(np.vstack([Wo, np.zeros((r - len(S), dv + 1))]))
        if name != "resident_r_eq_n":  # the complete factor makes H_SS too ill-conditioned
            assert rel(W[h], Wor[-1]) < 1e-3, (h, rel(W[h], Wor[-1]))
    # attention alone, fed the oracle's weights
    O, flags = wc.wc_attend(Qd, Kd, rpc["pivots"], rpc["rank"], dev(np.stack(Wor)))
    O = host(O)
    for h in range(H):
        S = piv[h][piv[h] >= 0]
        Oo, den, kappa = ow.attend(Q[h], K[h], S, Wor[h][: len(S)])
        check_output(O[h], Oo, kappa, dtype, f"{__name__}:{h}")
    assert np.all(host(flags) == 0)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_parity(wc, case):
    name, dtype, kind, H, n, m, d, dv, r = case
    Q, K, V = case_inputs(case)
    U = snapped(K, r)
    out = wc.wc_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), r, u_forced=dev(U))
    O, piv, rank = host(out["O"]), host(out["pivots"]), host(out["rank"])
    for h in range(H):
        ref = ow.forward(Q[h], K[h], V[h], r, U[h])
        assert np.array_equal(piv[h], ref["pivots"])
        assert rank[h] == ref["rank"]
        check_output(O[h], ref["O"], ref["kappa"], dtype, f"{__name__}:{h}")
    if name == "resident_r_eq_n":  # r = n: the coreset is every key, so O is exact attention
        for h in range(H):
            assert rel(O[h], ow.exact_attention(Q[h], K[h], V[h])) < TOL[dtype]


@pytest.mark.parametrize("dtype,n", [("bf16", 4), ("f32", 4), ("bf16", 300)])
def test_philox_stream_matches_oracle(wc, dtype, n):
    """Seeded mode: the device draws the same Philox4x64-10 uniforms as the oracle."""
    H, r, seed = 256, 3, 20260202
    rng = np.random.default_rng(3)
    K = np.tile((rng.standard_normal((1, n, 64)) * 0.3).astype(np.float32), (H, 1, 1))
    K = synth.round_to_bf16(K) if dtype == "bf16" else K
    out = wc.wc_rpcholesky(dev(K, dtype), r, seed=seed)
    piv = host(out["pivots"])
    agree = 0
    for h in range(H):
        u = philox.pivot_uniforms(seed, h, r)
        same = np.array_equal(piv[h], ow.rpcholesky(K[h], r, u)["pivots"])
        agree += same
        if not same:  # only rounding may separate the device's choice from the draw
            rep = pivot_report(K[h], piv[h], u)
            assert rep["excess"] <= 1.0, (h, rep)
    assert agree >= H - 1, agree


@pytest.mark.parametrize("n", [100, 700])
def test_breakdown_on_zero_keys(wc, n):
    """All-zero keys: H is exactly rank one, so the loop stops after one pivot; every query
    then attends uniformly and O is the mean of V."""
    H, m, r = 2, 20, 8
    Q, _, V = synth.random_inputs(H, n, m, 64, 64, seed=9, dtype="bf16")
    K = np.zeros((H, n, 64), np.float32)
    out = wc.wc_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), r, seed=1)
    assert np.all(host(out["rank"]) == 1)
    assert np.all(host(out["flags"]) & 1)
    piv = host(out["pivots"])
    assert np.all(piv[:, 1:] == -1) and np.all(piv[:, 0] >= 0)
    O = host(out["O"])
    for h in range(H):
        assert rel(O[h], np.tile(V[h].mean(0), (m, 1))) < 2e-2


@pytest.mark.parametrize("n,dtype", [(150, "bf16"), (600, "f32")])
def test_nonfinite_key_flagged(wc, n, dtype):
    H, r = 1, 4
    _, K, _ = synth.random_inputs(H, n, 4, 64, 64, seed=10, dtype=dtype)
    K[0, 7, 3] = np.nan
    out = wc.wc_rpcholesky(dev(K, dtype), r, seed=1)
    assert host(out["rank"])[0] == 0
    assert host(out["flags"])[0] & 2 and host(out["flags"])[0] & 1
    assert np.all(host(out["pivots"]) == -1)


@pytest.mark.parametrize("n,dtype", [(197, "bf16"), (900, "bf16")])
def test_no_queries(wc, n, dtype):
    import torch

    H, r = 2, 16
    _, K, V = synth.random_inputs(H, n, 1, 64, 64, seed=11, dtype=dtype)
    Q = torch.empty((H, 0, 64), dtype=torch.bfloat16, device="cuda")
    out = wc.wc_forward(Q, dev(K, dtype), dev(V, dtype), r, seed=5)
    torch.cuda.synchronize()
    assert out["O"].shape == (H, 0, 64)
    assert np.all(host(out["rank"]) == r)


def test_no_heads(wc):
    import torch

    z = torch.empty((0, 50, 64), dtype=torch.bfloat16, device="cuda")
    out = wc.wc_forward(torch.empty((0, 5, 64), dtype=torch.bfloat16, device="cuda"), z, z, 10)
    assert out["O"].shape == (0, 5, 64)


@pytest.mark.parametrize("n,dtype", [(197, "bf16"), (2000, "bf16"), (500, "f32")])
def test_deterministic(wc, n, dtype):
    Q, K, V = synth.random_inputs(3, n, 64, 64, 64, seed=12, dtype=dtype, kind="mixture")
    args = (dev(Q, dtype), dev(K, dtype), dev(V, dtype), 32)
    a = wc.wc_forward(*args, seed=77)
    b = wc.wc_forward(*args, seed=77)
    assert np.array_equal(host(a["pivots"]), host(b["pivots"]))
    assert np.array_equal(host(a["O"]), host(b["O"]))


@pytest.mark.parametrize("n,dtype", [(197, "bf16"), (1500, "bf16"), (600, "f32")])
def test_graph_replay_matches_eager(wc, n, dtype):
    """The forward captured in a HIP graph gives the eager result on every replay (the path
    records no memset nodes); eager work and synchronisations run between the replays."""
    import torch

    Q, K, V = synth.random_inputs(4, n, 70, 64, 64, seed=13, dtype=dtype, kind="mixture")
    Qd, Kd, Vd = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    p = wc.problem(4, n, 70, 64, 64, 32, Qd.dtype)
    ws = wc.workspace(p, "cuda")
    out = wc.wc_forward(Qd, Kd, Vd, 32, seed=99, ws=ws)
    ref = {k: v.clone() for k, v in out.items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            wc.wc_forward(Qd, Kd, Vd, 32, seed=99, ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for v in out.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (rep, k)
        wc.wc_forward(Qd, Kd, Vd, 32, seed=5, ws=ws)  # unrelated eager work in between
        torch.cuda.synchronize()


# (n, r, bins, pivot_block, options, dtype): the binned forward (union and per-bin weights), the
# block-pivot selection with and without bins, and key centring, as bench.py times them
GRAPH_PATHS = [
    (2048, 128, 4, 1, 0, "bf16"),
    (2048, 256, 4, 32, 0, "bf16"),
    (1024, 128, 1, 32, 0, "bf16"),
    (1536, 192, 3, 16, 1, "bf16"),      # per-bin weights (WC_OPT_BIN_WEIGHTS)
    (1024, 96, 2, 16, 2, "bf16"),       # centred keys (WC_OPT_CENTER_KEYS)
    (1024, 128, 4, 32, 0, "f32"),
]


@pytest.mark.parametrize("case", GRAPH_PATHS, ids=[f"n{c[0]}_r{c[1]}_B{c[2]}_b{c[3]}_o{c[4]}_{c[5]}" for c in GRAPH_PATHS])
def test_graph_replay_binned_block(wc, case):
    """The binned, block-pivot and centred-key forwards captured in a HIP graph give the eager
    result bit for bit on every replay, with unrelated eager work (another seed, so other pivots
    in the same workspace) and synchronisations between the replays: the graph holds no memset
    nodes, and nothing in it depends on what the call before left in the workspace."""
    import torch

    n, r, B, pb, opt, dtype = case
    H, m = 3, 300
    Q, K, V = synth.random_inputs(H, n, m, 64, 64, seed=41 + n + r, dtype=dtype, kind="mixture")
    Qd, Kd, Vd = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    p = wc.problem(H, n, m, 64, 64, r, Qd.dtype, B, opt, pb)
    ws = wc.workspace(p, "cuda")
    kw = dict(seed=123, bins=B, pivot_block=pb, bin_weights=bool(opt & 1), center_keys=bool(opt & 2), ws=ws)
    out = wc.wc_forward(Qd, Kd, Vd, r, **kw)
    ref = {k: v.clone() for k, v in out.items()}
    assert int(host(out["rank"]).min()) == r and int(host(out["flags"]).max()) == 0
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            wc.wc_forward(Qd, Kd, Vd, r, out=out, **kw)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for v in out.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (rep, k)
        other = dict(kw, seed=9 + rep)
        wc.wc_forward(Qd, Kd, Vd, r, **other)  # unrelated eager work in between
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,r", [(1, 1), (2, 1), (2, 2), (3, 3), (5, 2)])
def test_tiny_heads(wc, dtype, n, r):
    """Heads of one to five keys (bf16 on the resident kernel, fp32 on the streaming loop):
    pivots and rank as the oracle's, O within the tolerance, and at r = n exact attention
    (a single key gives O = its value row)."""
    H, m = 3, 7
    Q, K, V = synth.random_inputs(H, n, m, 64, 64, seed=870 + 10 * n + r, dtype=dtype, kind="iid_clip")
    U = snapped(K, r)
    out = wc.wc_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), r, u_forced=dev(U))
    O, piv, rank, flags = host(out["O"]), host(out["pivots"]), host(out["rank"]), host(out["flags"])
    for h in range(H):
        ref = ow.forward(Q[h], K[h], V[h], r, U[h])
        assert np.array_equal(piv[h], ref["pivots"]) and rank[h] == ref["rank"] == r
        assert flags[h] == 0
        assert rel(O[h], ref["O"]) < TOL[dtype], (h, rel(O[h], ref["O"]))
        if r == n:
            assert rel(O[h], ow.exact_attention(Q[h], K[h], V[h])) < TOL[dtype]


@pytest.mark.parametrize("dtype,d,r,rk", [("bf16", 128, 512, 512), ("f32", 64, 576, 576),
                                           ("bf16", 64, 512, 300), ("f32", 64, 512, 449),
                                           ("bf16", 64, 256, 256), ("f32", 128, 256, 200)])
def test_blocked_solve(wc, dtype, d, r, rk):
    """Weights with r a multiple of 64 and at least 256 take the blocked back substitution.
    Given the GPU's pivots, W and O are unique, so both are compared with the oracle's from
    those pivots.  Head 0 gets rank rk (the rank a breakdown would leave: for rk < r one block
    is cut at the rank and the later ones lie past it, and their rows must be zero); head 1
    keeps the full rank, so the two heads' blocks differ within one launch."""
    import torch

    H, n, m = 2, 2048, 120
    Q, K, V = synth.random_inputs(H, n, m, d, d, seed=880 + r + rk, dtype=dtype, kind="kv_outlier")
    Qd, Kd = dev(Q, dtype), dev(K, dtype)
    rpc = wc.wc_rpcholesky(Kd, r, seed=3, with_diag=False)
    assert np.all(host(rpc["rank"]) == r)
    ranks = [rk, r]
    rank = torch.tensor(ranks, dtype=torch.int32, device="cuda")
    W = wc.wc_weights(dev(V, dtype), rpc["pivots"], rank, rpc["F"])
    Wh = host(W)
    O, flags = wc.wc_attend(Qd, Kd, rpc["pivots"], rank, W)
    O = host(O)
    beta = 1.0 / np.sqrt(d)
    for h in range(H):
        k = ranks[h]
        S = host(rpc["pivots"])[h][:k]
        Wo = ow.weights(K[h], V[h], S, beta)
        assert rel(Wh[h][:k], Wo) < 1e-3, (h, rel(Wh[h][:k], Wo))
        assert np.all(Wh[h][k:] == 0.0)
        Oo, den, kappa = ow.attend(Q[h], K[h], S, Wo, beta)
        check_output(O[h], Oo, kappa, dtype, f"{__name__}:{h}")
    assert np.all(host(flags) == 0)
