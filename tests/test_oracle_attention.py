"""Pins of the sparse attention (R13, R14) against torch's scaled-dot-product
attention (float64, CPU) and closed forms."""
import numpy as np
import torch

from oracle.codecs import e4m3_decode
from oracle.csa2 import (attend, attend_lse, dequant_fp4, quant_fp4, sparse_attention, swa_window_rows)

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


def test_attend_lse_special_cases():
    """log-sum-exp pins: n copies of one key give logit + log n; a single key gives
    its logit; no keys give -inf; shifting every logit by c shifts lse by c."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 8))
    k1 = rng.standard_normal((1, 8))
    lg = q @ k1[0] / np.sqrt(8)
    assert np.allclose(attend_lse(q, k1), lg, atol=1e-13)
    assert np.allclose(attend_lse(q, np.repeat(k1, 5, axis=0)), lg + np.log(5), atol=1e-13)
    assert np.all(attend_lse(q, np.zeros((0, 8))) == -np.inf)
    k = rng.standard_normal((7, 8))
    # a key component along q adds q·u * sc to every logit of that head
    u = np.zeros(8); u[0] = 1.0
    q0 = np.zeros((1, 8)); q0[0, 0] = 2.0
    shift = attend_lse(q0, k + 3.0 * u) - attend_lse(q0, k)
    assert np.allclose(shift, 2.0 * 3.0 / np.sqrt(8), atol=1e-12)
    # large logits do not overflow (max-shifted evaluation)
    assert np.isfinite(attend_lse(q * 1e4, k)).all()


def test_window_rows_of_a_ring_match_the_linear_history():
    """Reading R21 (window buffer as a ring): a ring of S slots written token by
    token (each new position overwriting the oldest) must give every query the
    same window tokens as the full linear history of positions gives it under
    R14 (positions (t - n_win, t]), for queries up to the last written position
    as long as the ring still holds their whole window."""
    rng = np.random.default_rng(4)
    n_win, d = 5, 3
    hist = rng.integers(0, 120, (40, d)).astype(np.uint8)        # position p -> token
    for S in (5, 7, 9):
        ring = np.zeros((S, d), np.uint8)
        for last in range(40):
            ring[last % S] = hist[last]                            # append position `last`
            for t in range(max(0, last - (S - n_win)), last + 1):  # whole window still held
                got = ring[swa_window_rows(t, S, 0, n_win)]
                lo = max(0, t - n_win + 1)
                assert np.array_equal(got, hist[lo:t + 1]), (S, last, t)
    # a linear buffer (no wrap) is the special case; an older start clips the window
    assert list(swa_window_rows(7, 10, 5, 5)) == [0, 1, 2]
    assert list(swa_window_rows(3, 10, 5, 5)) == []
