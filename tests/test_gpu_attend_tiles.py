"""The persistent bf16 attention kernel walks several tiles per workgroup, and the coreset chunks
of consecutive tiles form one stream: the next tile's queries are requested chunks ahead and its
first unit is scored in the current tile's last pipeline step.  These cases force each schedule
of that hand-over against the oracle's attend: tiles of 2, 3, 4, 6 and 8 chunks of 64 coreset
rows with more tiles than compute units, a workgroup walking tiles of 6 and of 4 chunks (the
long tiles' deferred tile-end loads followed by the short tiles' schedule), coreset splits down
to one chunk per tile, a ragged last query tile, and slots past the rank that carry pivots and
weights the kernel must ignore.  The pivots and weights are random, so the oracle is the plain
definition of the output."""
import numpy as np
import pytest

from coreset_head_rpcholesky_amd import synth
from oracle import wildcat as ow
from tests.gpu_util import check_output, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch  # noqa: F401

    from coreset_head_rpcholesky_amd import binding
    return binding


# (heads, n, m, d, dv, r, rank).  A tile is 256 queries of one head (and one coreset split when
# heads x query tiles < 512); chunks per tile = ceil(r / 128) * 2 / splits.
CASES = [
    (2, 3000, 70000, 128, 128, 128, 128),   # 548 tiles of 2 chunks
    (2, 3000, 66000, 64, 64, 256, 250),     # 516 tiles of 4 chunks, 6 slots past the rank
    (4, 3000, 33000, 64, 128, 320, 300),    # 516 tiles of 6 chunks, 20 slots past the rank
    (2, 2500, 66000, 128, 128, 512, 512),   # 516 tiles of 8 chunks
    (1, 2000, 90000, 128, 64, 384, 384),    # 2 splits: 704 tiles of 3 chunks
    (1, 2000, 51200, 128, 128, 1000, 990),  # 3 splits: 600 tiles of 6, 6 and 4 chunks, mixed
    (300, 400, 256, 64, 128, 128, 100),     # 2 splits: 600 tiles of 1 chunk
    (40, 700, 300, 128, 128, 320, 320),     # 6 splits: 480 tiles of 1 chunk, ragged query tile
]


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}_m{c[2]}_d{c[3]}_r{c[5]}" for c in CASES])
def test_attend_tile_transitions(wc, case):
    import torch

    H, n, m, d, dv, r, rk = case
    Q, K, _ = synth.random_inputs(H, n, m, d, 1, seed=900 + m + r, dtype="bf16", kind="iid_clip", clip=2.0)
    Q, K = synth.round_to_bf16(Q), synth.round_to_bf16(K)
    rng = np.random.default_rng(901 + r)
    piv = np.stack([rng.choice(n, r, replace=False) for _ in range(H)]).astype(np.int32)
    W = (rng.standard_normal((H, r, dv + 1)) * 0.05).astype(np.float32)
    W[:, :, dv] = (1.0 + 0.5 * rng.random((H, r))) / rk
    rank = torch.full((H,), rk, dtype=torch.int32, device="cuda")
    O, flags = wc.wc_attend(dev(Q, "bf16"), dev(K, "bf16"), torch.from_numpy(piv).cuda(), rank, dev(W))
    O = host(O)
    assert not host(flags).any()
    heads = range(H) if H <= 4 else sorted({0, 1, H // 2, H - 1})
    # every query of small cases; else a stride through all tiles plus the last 300 queries
    qs = np.arange(m) if m <= 4096 else np.unique(np.r_[np.arange(0, m, 97), np.arange(m - 300, m)])
    for h in heads:
        ref, _, kappa = ow.attend(Q[h][qs], K[h], piv[h][:rk], W[h][:rk].astype(np.float64))
        check_output(O[h][qs], ref, kappa, "bf16", f"tiles:{case}:h{h}")
