"""Pins of key centring (center_keys): the rounding helper against numpy's own bf16-free
reference (exhaustive ties and a random sweep checked bit by bit against a reference written
with integer arithmetic on the float's fields); centred keys have zero mean up to the stored
precision; exact attention is unchanged by the shift (the pages' invariance); WildCat on
centred keys at full rank is exact attention of the original keys; and with a large common
offset in the keys, centring lowers WildCat's error."""
import numpy as np
import pytest

from oracle import wildcat as ow


def bf16_reference(x):
    """Round-to-nearest-even to 8 significant bits, written on mantissa and exponent with frexp."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                 # x = m 2^e, 0.5 <= |m| < 1
    scaled = m * 256.0                 # 8 significant bits kept
    r = np.round(scaled)               # numpy rounds half to even
    return np.ldexp(r / 256.0, e).astype(np.float32)


def test_round_bf16_matches_reference():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0 + 2 ** -7], np.float32)
    for v in (x, ties):
        assert np.array_equal(ow.round_bf16(v), bf16_reference(v))
    assert ow.round_bf16(np.float32([1.0 + 2 ** -8]))[0] == 1.0            # tie to even (down)
    assert ow.round_bf16(np.float32([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6  # tie to even (up)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_centred_keys_have_zero_mean(dtype):
    rng = np.random.default_rng(1)
    K = rng.standard_normal((500, 16)) + 3.0
    Kc = ow.center_keys(K, dtype)
    tol = 1e-6 if dtype == "f32" else 1e-2
    assert np.abs(Kc.mean(axis=0)).max() < tol
    assert np.abs(Kc - (K - K.mean(axis=0))).max() <= (2 ** -24 if dtype == "f32" else 2 ** -8) * np.abs(K - K.mean(0)).max() * 1.01
    # stored in the input precision: every value is a float32 (and a bf16) number
    assert np.array_equal(Kc, Kc.astype(np.float32).astype(np.float64))
    if dtype == "bf16":
        assert np.array_equal(Kc, bf16_reference(Kc).astype(np.float64))
        assert not np.array_equal(Kc, (K - K.mean(axis=0)).astype(np.float32).astype(np.float64))


def test_exact_attention_is_invariant_under_centring():
    rng = np.random.default_rng(2)
    Q, K, V = rng.standard_normal((20, 8)), rng.standard_normal((60, 8)) + 1.5, rng.standard_normal((60, 4))
    assert np.allclose(ow.exact_attention(Q, ow.center_keys(K), V), ow.exact_attention(Q, K, V),
                       rtol=1e-5, atol=1e-6)


def test_full_rank_on_centred_keys_is_exact():
    rng = np.random.default_rng(3)
    Q, K, V = rng.standard_normal((10, 6)) * 0.6, rng.standard_normal((24, 6)) * 0.6 + 0.8, rng.standard_normal((24, 3))
    u = rng.random(24)
    out = ow.forward(Q, ow.center_keys(K), V, 24, u)
    assert np.allclose(out["O"], ow.exact_attention(Q, K, V), rtol=1e-5, atol=1e-6)


def test_centring_helps_keys_with_a_common_offset():
    """Keys = bounded noise + a large common offset: the offset makes every kernel column
    nearly proportional, and the coreset sees little of the noise; centring removes it."""
    rng = np.random.default_rng(4)
    n, d = 400, 16
    K = rng.standard_normal((n, d)) * 0.5 + 2.5 * rng.standard_normal(d)
    Q = rng.standard_normal((50, d)) * 0.5
    V = rng.standard_normal((n, 4))
    exact = ow.exact_attention(Q, K, V)
    e_plain, e_cent = [], []
    for s in range(3):
        u = np.random.default_rng(10 + s).random(24)
        e_plain.append(ow.rel_fro(ow.forward(Q, K, V, 24, u)["O"], exact))
        e_cent.append(ow.rel_fro(ow.forward(Q, ow.center_keys(K), V, 24, u)["O"], exact))
    assert np.mean(e_cent) < 0.5 * np.mean(e_plain), (e_plain, e_cent)
