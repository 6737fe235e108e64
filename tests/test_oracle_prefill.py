"""Pins of the oracle's prefill composition (oracle.csa2.prefill_chunk).

Checked against facts fixed independently of the composition itself:
  * the causal visible-entry count of the 8,192-token chunk at m = 2 (a closed
    form: sum over t of floor((t+1)/2));
  * with K >= every visible count, Top-K keeps every visible entry, so each
    query's output must equal dense causal attention over all visible entries
    followed by its window, written out here as an explicit softmax loop;
  * visibility at the chunk edges (the first query sees only the prefix at
    m = 2, the last one sees every entry);
  * Reuse layers return the Full layer's selection unchanged.
"""
import math

import numpy as np
import pytest

from oracle.codecs import bf16_to_f64, e4m3_decode, e4m3_encode, f64_to_bf16
from oracle.csa2 import (PrefillLayerInputs, dequant_fp4, index_scores, indexer_k, prefill_chunk,
                         quant_fp4, topk, visible_count)


def test_visible_count_sum_of_the_32k_chunk():
    # chunk = the last 8,192 of 32,768 tokens, m = 2, 16,384 entries in all
    total = sum(visible_count(t, 16384, 2) for t in range(24576, 32768))
    closed = sum((x // 2) for x in range(24577, 32769))
    assert total == closed == 117_440_512


def _case(seed, Tq=12, m=2, n_pre=10, d=64, d_model=32, h_i=2, d_i=32, H_q=3, n_win=4,
          K=64, sched="FUU"):
    rng = np.random.default_rng(seed)
    pos0 = n_pre * m
    H = rng.standard_normal((Tq, d_model))
    W_kv = rng.standard_normal((d_model, d)) / np.sqrt(d_model)
    W_z = rng.standard_normal((d_model, d)) / np.sqrt(d_model)
    pre = quant_fp4(rng.standard_normal((n_pre, d)).astype(np.float32))
    W_ik = f64_to_bf16(rng.standard_normal((d, d_i)) / np.sqrt(d))
    k_pre = indexer_k(pre.codes, pre.scales, W_ik)
    swa_pos0 = max(0, pos0 - (n_win - 1))
    S = pos0 + Tq - swa_pos0
    layers = []
    for mode in sched:
        layers.append(PrefillLayerInputs(
            q_main=f64_to_bf16(rng.standard_normal((Tq, H_q, d))),
            swa=e4m3_encode(rng.standard_normal((S, d))),
            q_idx=f64_to_bf16(rng.standard_normal((Tq, h_i, d_i))) if mode == "F" else None,
            w=rng.random((Tq, h_i)) if mode == "F" else None))
    return dict(schedule=list(sched), layers=layers, H=H, W_kv=W_kv, W_z=W_z, m=m, pos0=pos0,
                codes_pre=pre.codes, scales_pre=pre.scales, k_pre=k_pre, W_ik=W_ik, K=K,
                swa_pos0=swa_pos0, n_win=n_win)


def _dense_causal(q_bits, keys):
    """softmax(q·k / sqrt(d)) · k per head, one key at a time (K = V)."""
    q = bf16_to_f64(q_bits)
    d = q.shape[-1]
    out = np.zeros_like(q)
    for h in range(q.shape[0]):
        lg = [float(np.dot(q[h], k)) / math.sqrt(d) for k in keys]
        mx = max(lg)
        ws = [math.exp(x - mx) for x in lg]
        tot = sum(ws)
        for wgt, k in zip(ws, keys):
            out[h] += (wgt / tot) * k
    return out


@pytest.mark.parametrize("m", [1, 2])
def test_prefill_equals_dense_causal_attention_when_k_covers_everything(m):
    c = _case(1, m=m, K=64)
    res = prefill_chunk(**c)
    codes = np.concatenate([c["codes_pre"], res.entries.codes])
    scales = np.concatenate([c["scales_pre"], res.entries.scales])
    x = dequant_fp4(codes, scales)
    n = x.shape[0]
    for li, layer in enumerate(c["layers"]):
        swa = e4m3_decode(layer.swa)
        for t in range(c["H"].shape[0]):
            pos = c["pos0"] + t
            vis = [j for j in range(n) if (j + 1) * m - 1 <= pos]          # p_j <= t
            win = [i for i in range(swa.shape[0])
                   if pos - c["n_win"] < c["swa_pos0"] + i <= pos]         # (t - n_win, t]
            keys = [x[j] for j in vis] + [swa[i] for i in win]
            want = _dense_causal(layer.q_main[t], keys)
            np.testing.assert_allclose(res.out[li][t], want, rtol=1e-12, atol=1e-12)
            got_sel = res.sel[li][t]
            assert list(got_sel[got_sel >= 0]) == vis


def test_prefill_chunk_edges_and_reuse():
    c = _case(2, Tq=8, m=2, n_pre=10, K=6, sched="FUU")
    res = prefill_chunk(**c)
    n_pre = c["codes_pre"].shape[0]
    sel = res.sel[0]
    # first query (position pos0, even): entries with p_j = 2j+1 <= pos0 -> the prefix only
    assert sel[0].max() < n_pre
    # last query sees every entry, so its Top-K is over all of them
    n = n_pre + res.entries.codes.shape[0]
    k_all = np.concatenate([c["k_pre"], res.k_new])
    t = 7
    s = index_scores(c["layers"][0].q_idx[t], c["layers"][0].w[t], k_all)
    assert np.array_equal(sel[t], topk(s, 6, n))
    # Reuse layers keep the Full selection of the same query
    for li in (1, 2):
        assert np.array_equal(res.sel[li], sel)


def test_prefill_rows_subset_matches_full_evaluation():
    c = _case(3, Tq=10, m=2, K=5)
    full = prefill_chunk(**c)
    part = prefill_chunk(**c, rows=[0, 4, 9])
    for li in range(3):
        assert np.array_equal(part.sel[li], full.sel[li][[0, 4, 9]])
        assert np.array_equal(part.out[li], full.out[li][[0, 4, 9]])
