"""Pins of the compressor fold (reading R1), entry positions (R3) and RoPE (R4)."""
import numpy as np
from scipy.special import expit

from oracle.csa2 import compress, entry_positions, fold, project, rope

rng = np.random.default_rng(7)


def test_m1_is_identity():
    # [deep-dive §3.1]: with m = 1 nothing is compressed
    C = rng.standard_normal((37, 24))
    Z = rng.standard_normal((37, 24))
    assert np.array_equal(fold(C, Z, 1), C)


def test_constant_weights_give_block_mean():
    C = rng.standard_normal((12, 8))
    out = fold(C, np.zeros((12, 8)), 3)
    assert np.allclose(out, C.reshape(4, 3, 8).mean(1), rtol=0, atol=1e-15)


def test_two_token_closed_form():
    C = rng.standard_normal((2, 5))
    Z = rng.standard_normal((2, 5))
    a = expit(Z[0] - Z[1])
    assert np.allclose(fold(C, Z, 2)[0], a * C[0] + (1 - a) * C[1], rtol=1e-14, atol=1e-14)


def test_dominant_weight_selects_token():
    C = rng.standard_normal((4, 6))
    Z = np.zeros((4, 6))
    Z[1, :3] = 2000.0   # token 1 wins channels 0-2
    Z[3, 3:] = 2000.0   # token 3 wins channels 3-5 of block 1
    out = fold(C, Z, 2)
    assert np.array_equal(out[0, :3], C[1, :3])
    assert np.array_equal(out[1, 3:], C[3, 3:])


def test_per_channel_shift_and_permutation_invariance():
    C = rng.standard_normal((8, 6))
    Z = rng.standard_normal((8, 6))
    out = fold(C, Z, 4)
    shift = np.repeat(rng.standard_normal((2, 6)), 4, axis=0)
    assert np.allclose(fold(C, Z + shift, 4), out, atol=1e-14)
    perm = np.concatenate([rng.permutation(4), 4 + rng.permutation(4)])
    assert np.allclose(fold(C[perm], Z[perm], 4), out, atol=1e-14)
    lo = C.reshape(2, 4, 6).min(1)
    hi = C.reshape(2, 4, 6).max(1)
    assert np.all(out >= lo - 1e-15) and np.all(out <= hi + 1e-15)


def test_channels_independent_and_scalar_weight_broadcast():
    C = rng.standard_normal((6, 5))
    Z = rng.standard_normal((6, 5))
    Z2 = Z.copy()
    Z2[:, 2] += rng.standard_normal(6)
    a, b = fold(C, Z, 3), fold(C, Z2, 3)
    assert np.array_equal(np.delete(a, 2, 1), np.delete(b, 2, 1))
    z1 = rng.standard_normal((6, 1))
    assert np.allclose(fold(C, z1, 3), fold(C, np.repeat(z1, 5, 1), 3), atol=1e-15)


def test_tail_tokens_make_no_entry():
    H = rng.standard_normal((7, 4))
    W = rng.standard_normal((4, 6))
    out = compress(H, W, W, m=3, rope_dim=0)
    H2 = H.copy()
    H2[6] = 99.0
    assert out.shape == (2, 6)
    assert np.array_equal(compress(H2, W, W, m=3, rope_dim=0), out)


def test_project_upcasts_bf16_bits_exactly():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25
    H = np.array([[0x3F80, 0xC000]], dtype=np.uint16)
    W = np.array([[0x3E80], [0x3F80]], dtype=np.uint16)
    assert project(H, W)[0, 0] == 0.25 - 2.0


def test_entry_positions():
    assert list(entry_positions(4, 2)) == [1, 3, 5, 7]
    assert list(entry_positions(3, 1, pos0=10)) == [10, 11, 12]
    assert list(entry_positions(2, 2, pos0=24576)) == [24577, 24579]


def test_rope_closed_forms():
    d, r = 128, 64
    x = np.zeros((3, d))
    x[:, d - r] = 1.0           # pair i = 0 -> angle = p
    x[:, d - r + 32] = 1.0      # pair i = 16 -> angle = p * 10000**(-1/2) = p / 100
    p = np.array([0.0, 1.0, 250.0])
    y = rope(x, p, r)
    assert np.array_equal(y[0], x[0])                       # position 0: identity
    assert np.allclose(y[:, d - r], np.cos(p), atol=1e-15)
    assert np.allclose(y[:, d - r + 1], np.sin(p), atol=1e-15)
    assert np.allclose(y[:, d - r + 32], np.cos(p / 100), atol=1e-15)
    assert np.allclose(y[:, d - r + 33], np.sin(p / 100), atol=1e-15)
    assert np.array_equal(y[:, :d - r], x[:, :d - r])       # only the last r channels turn


def test_rope_norms_and_composition():
    x = rng.standard_normal((5, 96))
    p1 = rng.integers(0, 10 ** 6, 5).astype(np.float64)
    p2 = rng.integers(0, 10 ** 3, 5).astype(np.float64)
    y = rope(x, p1)
    pairs = lambda a: np.hypot(a[:, 32::2], a[:, 33::2])
    assert np.allclose(pairs(y), pairs(x), rtol=1e-13)
    assert np.allclose(rope(y, p2), rope(x, p1 + p2), atol=1e-9)
