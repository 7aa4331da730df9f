"""The seeded input generators: shapes, value ranges, bf16 exactness, reproducibility."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth


def test_round_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 7
    ours = synth.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_shapes_and_ranges(name):
    w = synth.WORKLOADS[name]
    n = min(w.n, 2048)
    m = min(w.m, 64)
    Q, K, V = synth.make_inputs(name, heads=[0, 1] if w.heads > 1 else [0], n=n, m=m)
    assert K.shape[1:] == (n, w.d) and Q.shape[1:] == (m, w.d) and V.shape[1:] == (n, w.dv)
    if w.clip:
        assert np.all(np.linalg.norm(K, axis=-1) <= w.clip * (1 + 2**-7))
        assert np.all(np.linalg.norm(Q, axis=-1) <= w.clip * (1 + 2**-7))
    if w.dtype == "bf16":
        for X in (Q, K, V):
            assert np.array_equal(X, synth.round_to_bf16(X))


def test_head_subsets_reproduce_full_batch():
    Q, K, V = synth.make_inputs("vit197")
    q, k, v = synth.make_inputs("vit197", heads=[5, 700])
    assert np.array_equal(K[[5, 700]], k) and np.array_equal(Q[[5, 700]], q)
    assert np.array_equal(V[[5, 700]], v)


def test_kv_outliers():
    Q, K, V = synth.make_inputs("kv32k", heads=[0])
    nrm = np.linalg.norm(K[0], axis=1)
    big = np.sum(nrm > 2.5 * np.median(nrm))
    assert big == 328
