"""Pins of the sparse attention (R13, R14) against torch's scaled-dot-product
attention (float64, CPU) and closed forms."""
import numpy as np
import torch

from oracle.codecs import e4m3_decode
from oracle.csa2 import (attend, dequant_fp4, quant_fp4, sparse_attention, swa_window_rows)

rng = np.random.default_rng(4)


def _cache(n, d):
    x = rng.standard_normal((n, d)).astype(np.float32)
    q = quant_fp4(x)
    return q.codes, q.scales


def _swa(S, d):
    import synth
    return synth.to_e4m3_codes(rng.standard_normal((S, d)).astype(np.float32))


def _sdpa(q, keys, scale):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None]
    kt = torch.from_numpy(np.asarray(keys, dtype=np.float64))[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)[0].numpy()


def test_all_entries_selected_is_dense_attention():
    n, d, H, S = 40, 64, 4, 16
    codes, scales = _cache(n, d)
    swa = _swa(S, d)
    q = rng.standard_normal((H, d))
    sel = np.concatenate([np.arange(n), -np.ones(600 - n, dtype=np.int64)])  # K >= n
    out = sparse_attention(q, codes, scales, sel, swa)
    keys = np.concatenate([dequant_fp4(codes, scales), e4m3_decode(swa)])
    assert np.allclose(out, _sdpa(q, keys, 1 / np.sqrt(d)), rtol=1e-12, atol=1e-12)


def test_single_key_returns_key_and_empty_selection_is_window_only():
    n, d, H = 10, 32, 3
    codes, scales = _cache(n, d)
    q = rng.standard_normal((H, d))
    out = sparse_attention(q, codes, scales, np.array([4, -1, -1]), np.zeros((0, d), np.uint8))
    assert np.array_equal(out, np.repeat(dequant_fp4(codes, scales)[4:5], H, 0))
    swa = _swa(8, d)
    out = sparse_attention(q, codes, scales, np.full(5, -1), swa)
    assert np.allclose(out, _sdpa(q, e4m3_decode(swa), 1 / np.sqrt(d)), rtol=1e-12, atol=1e-12)


def test_output_in_convex_hull_and_sel_order_irrelevant():
    n, d, H, S = 300, 64, 8, 32
    codes, scales = _cache(n, d)
    swa = _swa(S, d)
    q = rng.standard_normal((H, d)) * 3
    sel = np.sort(rng.choice(n, 100, replace=False))
    out = sparse_attention(q, codes, scales, sel, swa)
    keys = np.concatenate([dequant_fp4(codes, scales)[sel], e4m3_decode(swa)])
    assert np.all(out <= keys.max(0) + 1e-12) and np.all(out >= keys.min(0) - 1e-12)
    assert np.allclose(sparse_attention(q, codes, scales, sel[::-1], swa), out, atol=1e-13)


def test_swa_scale_and_window_rows():
    d = 32
    codes, scales = _cache(5, d)
    swa = _swa(12, d)
    q = rng.standard_normal((2, d))
    out = sparse_attention(q, codes, scales, np.full(4, -1), swa, swa_scale=0.5)
    assert np.allclose(out, _sdpa(q, 0.5 * e4m3_decode(swa), 1 / np.sqrt(d)), atol=1e-13)
    # window (t - n_win, t]; tokens of the buffer start at swa_pos0
    assert list(swa_window_rows(105, 12, 100, 4)) == [2, 3, 4, 5]
    assert list(swa_window_rows(101, 12, 100, 128)) == [0, 1]
    assert list(swa_window_rows(None, 3, 0, 128)) == [0, 1, 2]


def test_attend_uses_given_scale():
    k = rng.standard_normal((7, 16))
    q = rng.standard_normal((2, 16))
    assert np.allclose(attend(q, k, 0.3), _sdpa(q, k, 0.3), atol=1e-13)
