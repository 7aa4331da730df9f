"""The debug library, libwc_debug.so, whose kernels check the pivot indices they read from device
memory.  On valid input it computes bit for bit what the regular library computes and sets no
WC_FLAG_BOUNDS; a pivot index outside [0, n) handed to wc_attend is reported for its head alone
and the slot counts as empty (the output equals that of the same call with pivot -1 there).
The out-of-range index used below points into the next head's rows, so even an unchecked read
would stay inside the key tensor."""
import os

import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    if not os.path.exists(binding.DEBUG_LIB_PATH):
        pytest.skip("libwc_debug.so not built")
    regular = binding.LIB
    saved = binding.LIB_PATH
    binding.LIB_PATH = binding.DEBUG_LIB_PATH
    debug = binding._load()
    binding.LIB_PATH = saved
    yield binding, regular, debug
    binding.LIB = regular


@pytest.mark.parametrize("dtype,n,m,d,dv,r,bins", [("bf16", 300, 70, 64, 64, 32, 1), ("bf16", 4096, 300, 128, 128, 256, 8),
                                                   ("f32", 1000, 40, 64, 128, 48, 1)])
def test_debug_forward_matches_regular(libs, dtype, n, m, d, dv, r, bins):
    binding, regular, debug = libs
    Q, K, V = synth.random_inputs(2, n, m, d, dv, seed=870 + n, dtype=dtype, kind="mixture")
    args = (dev(Q, dtype), dev(K, dtype), dev(V, dtype))
    outs = []
    for lib in (regular, debug):
        binding.LIB = lib
        f = binding.wc_forward(*args, r, seed=3, bins=bins)
        outs.append({k: host(v) for k, v in f.items() if hasattr(v, "cpu")})
    binding.LIB = regular
    assert set(outs[0]) == set(outs[1])
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k
    assert not (outs[1]["flags"].astype(np.int64) & binding.WC_FLAG_BOUNDS).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_debug_attend_reports_out_of_range_pivot(libs, dtype):
    import torch

    binding, regular, debug = libs
    H, n, m, d, dv, r = 2, 500, 90, 64, 64, 40
    Q, K, V = synth.random_inputs(H, n, m, d, dv, seed=880, dtype=dtype, kind="iid_clip", clip=2.0)
    rng = np.random.default_rng(1)
    piv = np.stack([rng.choice(n, r, replace=False) for _ in range(H)]).astype(np.int32)
    W = rng.standard_normal((H, r, dv + 1)).astype(np.float32) * 0.1
    W[:, :, dv] = 1.0 / r
    bad, empty = piv.copy(), piv.copy()
    bad[0, 7] = n + 5       # head 0 only; an unchecked read would land in head 1's keys
    empty[0, 7] = -1
    rank = torch.full((H,), r, dtype=torch.int32, device="cuda")
    Qd, Kd, Wd = dev(Q, dtype), dev(K, dtype), dev(W)
    binding.LIB = debug
    try:
        res = {}
        for name, p in (("bad", bad), ("empty", empty)):
            flags = torch.zeros(H, dtype=torch.int32, device="cuda")
            O, _ = binding.wc_attend(Qd, Kd, torch.from_numpy(p).cuda(), rank, Wd, flags=flags)
            torch.cuda.synchronize()
            res[name] = (host(O), host(flags).astype(np.int64))
    finally:
        binding.LIB = regular
    assert res["bad"][1][0] & binding.WC_FLAG_BOUNDS
    assert not res["bad"][1][1] & binding.WC_FLAG_BOUNDS
    assert not (res["empty"][1] & binding.WC_FLAG_BOUNDS).any()
    assert np.array_equal(res["bad"][0], res["empty"][0])
