"""wc_forward_noalloc, the forward with the library's own device workspace, against wc_forward
with a caller workspace: the same kernels on the same inputs, so pivots, rank, flags and O
agree bit for bit.  Two calls in a row, the second on a smaller problem (the array then holds
what the first call left), on the streaming one-bin path and the binned path; a problem whose
workspace exceeds the array is refused on the host; the call captured in a HIP graph replays
to the eager result."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


def same(a, b):
    for k in ("O", "pivots", "rank", "flags"):
        x, y = host(a[k]), host(b[k])
        assert np.array_equal(x, y, equal_nan=True), k


# (dtype, kind, H, n, m, d, dv, r, bins): first the larger problem, then the smaller one
PAIRS = [
    [("f32", "iid_clip", 3, 3001, 500, 64, 64, 64, 1), ("f32", "iid_clip", 2, 1000, 77, 64, 128, 40, 1)],
    [("bf16", "mixture", 2, 4096, 300, 128, 128, 256, 8), ("bf16", "kv_outlier", 1, 2048, 9, 64, 64, 128, 4)],
    [("bf16", "mixture", 4, 8192, 1000, 64, 64, 256, 1), ("bf16", "mixture", 5, 197, 197, 64, 64, 32, 1)],
]


@pytest.mark.parametrize("pair", PAIRS, ids=["stream_f32", "bins_bf16", "stream_then_resident"])
def test_noalloc_matches_forward(wc, pair):
    for i, (dtype, kind, H, n, m, d, dv, r, B) in enumerate(pair):
        print(f"case {i}: {dtype} {kind} H={H} n={n} m={m} d={d} dv={dv} r={r} bins={B}", flush=True)
        Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=870 + 10 * i + n, dtype=dtype, kind=kind,
                                      clip=2.5, clusters=8)
        Qd, Kd, Vd = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
        ref = wc.wc_forward(Qd, Kd, Vd, r, seed=11, bins=B)
        got = wc.wc_forward_noalloc(Qd, Kd, Vd, r, seed=11, bins=B)
        import torch
        torch.cuda.synchronize()
        assert np.all(host(ref["rank"]) == r)
        same(got, ref)


def test_noalloc_refuses_oversized_workspace(wc):
    import torch

    H, n, m, d, dv, r = 2, 65536, 4, 64, 64, 512  # F alone is 256 MiB
    p = wc.problem(H, n, m, d, dv, r, torch.bfloat16)
    assert wc.wc_workspace_bytes(p) > wc.WC_NOALLOC_MAX_WORKSPACE
    x = torch.zeros((H, n, d), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((H, m, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(wc.WcError) as e:
        wc.wc_forward_noalloc(q, x, x, r, seed=1)
    assert e.value.status == wc.WC_ERR_WORKSPACE


def test_noalloc_graph_replay(wc):
    import torch

    H, n, m, d, dv, r = 2, 3000, 400, 64, 64, 96
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=890, dtype="bf16", kind="mixture", clip=2.5, clusters=8)
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    ref = wc.wc_forward_noalloc(Qd, Kd, Vd, r, seed=5)
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            wc.wc_forward_noalloc(Qd, Kd, Vd, r, seed=5, out=out)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same(out, ref)
