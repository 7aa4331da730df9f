"""Pins of oracle.philox: numpy ships Philox4x64-10 as a bit generator, so the oracle's
integer implementation is checked against that library routine."""
import numpy as np
import pytest

from oracle import philox

MASK = (1 << 64) - 1


def numpy_block(counter, key):
    # numpy's Philox increments the 256-bit counter before producing each block of four.
    c = (counter[0] | (counter[1] << 64) | (counter[2] << 128) | (counter[3] << 192)) - 1
    c &= (1 << 256) - 1
    words = np.array([(c >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=words)
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("seed", [0, 1, 42, 2**63 + 12345, MASK])
@pytest.mark.parametrize("head,step", [(0, 0), (0, 1), (3, 0), (767, 31), (7, 2047), (2**31 - 1, 4095)])
def test_block_matches_numpy(seed, head, step):
    ours = philox.philox4x64_10((step, head, 0, 0), (seed, 0))
    assert list(ours) == numpy_block((step, head, 0, 0), (seed, 0))


def test_block_matches_numpy_full_key_and_counter():
    rng = np.random.default_rng(3)
    for _ in range(20):
        ctr = [int(x) for x in rng.integers(0, 2**63, size=4)]
        key = [int(x) for x in rng.integers(0, 2**63, size=2)]
        assert list(philox.philox4x64_10(ctr, key)) == numpy_block(ctr, key)


def test_uniforms_are_24bit_dyadic_in_unit_interval():
    us = philox.pivot_uniforms(42, 5, 2000)
    for u in us:
        assert 0.0 <= u < 1.0
        assert float(u * 2**24).is_integer()
    assert len(set(us)) > 1990


def test_uniforms_pass_chi_square():
    from scipy.stats import chisquare

    us = np.array([philox.pivot_uniform(9, h, t) for h in range(20) for t in range(1000)])
    counts, _ = np.histogram(us, bins=20, range=(0.0, 1.0))
    assert chisquare(counts).pvalue > 1e-4
