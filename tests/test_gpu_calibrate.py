"""The calibration kernels behind the bench's attainable rates compute what they claim: the copy
reproduces its source, the read touches every 16-byte word once (the XOR of the per-wave words
is the XOR of the whole buffer), and the matrix-core chains run exactly `iters` rounds of eight
MFMAs per wave (all operands are 1, so each sum is a known integer).  The clock readings of
the bf16 chain give a clock in the range this part can run at."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


def test_copy_and_read(wc):
    import torch

    nb = (64 << 20) + 48  # a ragged tail past the unrolled loop
    g = torch.Generator(device="cuda").manual_seed(5)
    src = torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    wc.wc_calibrate(wc.WC_CAL_COPY, dst, src=src, nbytes=nb)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    res = torch.zeros(wc.WC_CAL_RESULT_BYTES, dtype=torch.uint8, device="cuda")
    wc.wc_calibrate(wc.WC_CAL_READ, res, src=src, nbytes=nb)
    torch.cuda.synchronize()
    words = res.cpu().numpy().view(np.uint32)
    expect = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(words) == expect


@pytest.mark.parametrize("kind,per_round", [("bf16", 2048), ("f32", 256)])
def test_mfma_chains(wc, kind, per_round):
    import torch

    iters = 100
    res = torch.full((wc.WC_CAL_RESULT_BYTES // 4,), -1.0, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(4, dtype=torch.int64, device="cuda")
    k = wc.WC_CAL_MFMA_BF16 if kind == "bf16" else wc.WC_CAL_MFMA_F32
    wc.wc_calibrate(k, res, iters=iters, clocks=clocks)
    torch.cuda.synchronize()
    waves = 512 * 4
    out = res[:waves].cpu().numpy()
    assert np.all(out == per_round * iters), (out.min(), out.max())
    c = clocks.cpu().numpy()
    assert c[2] > c[0] and c[3] > c[1]
    if kind == "bf16":
        wc.wc_calibrate(k, res, iters=20000, clocks=clocks)
        torch.cuda.synchronize()
        c = clocks.cpu().numpy().astype(np.float64)
        ghz = (c[2] - c[0]) / (c[3] - c[1]) * 0.1
        assert 0.5 < ghz < 3.0, ghz
