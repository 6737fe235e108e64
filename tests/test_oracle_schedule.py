"""Pins of the layer schedule and the mode semantics (deep dive §3.2, §3.3)."""
import numpy as np

from conftest import read_golden
from oracle.csa2 import (FULL, REINDEX, REUSE, LayerInputs, build_pool, decode_step,
                         decoder_schedule, encoder_schedule, index_scores, quant_fp4,
                         indexer_k, reindex, sparse_attention, topk)
from oracle.codecs import f64_to_bf16

rng = np.random.default_rng(12)


def test_schedules_match_pages():
    g = dict((r[0], r[1]) for r in read_golden("schedule_and_geometry.txt"))
    assert "".join(decoder_schedule()) == g["decoder_schedule"]
    assert "".join(encoder_schedule()) == g["encoder_schedule"]
    dec = decoder_schedule()
    assert (dec.count(FULL), dec.count(REINDEX), dec.count(REUSE)) == (1, 4, 15)


def test_decode_step_modes():
    n, d, d_i, h, H, S, K = 4096, 64, 16, 4, 4, 8, 32
    x = rng.standard_normal((n, d)).astype(np.float32)
    q8 = quant_fp4(x)
    W = f64_to_bf16(rng.standard_normal((d, d_i)) / 8)
    k = indexer_k(q8.codes, q8.scales, W)
    sched = ["F", "U", "U", "R", "U"]
    import synth
    layers = [LayerInputs(q_main=f64_to_bf16(rng.standard_normal((H, d))),
                          swa=synth.to_e4m3_codes(rng.standard_normal((S, d)).astype(np.float32)),
                          q_idx=f64_to_bf16(rng.standard_normal((h, d_i))), w=rng.random(h))
              for _ in sched]
    res = decode_step(sched, layers, q8.codes, q8.scales, k, K=K, G=32, PB=16, PE=8)
    full = topk(index_scores(layers[0].q_idx, layers[0].w, k), K)
    pool = build_pool(index_scores(layers[0].q_idx, layers[0].w, k), 32, 16, 8)
    assert np.array_equal(res.sel[0], full)
    assert np.array_equal(res.sel[1], full) and np.array_equal(res.sel[2], full)   # Reuse
    assert np.array_equal(res.pool, pool) and res.pool.shape[0] == 16 * 8
    re = reindex(layers[3].q_idx, layers[3].w, k, pool, K)
    assert np.array_equal(res.sel[3], re) and np.array_equal(res.sel[4], re)
    assert set(re[re >= 0]) <= set(pool)                                           # pool only
    assert len(res.out) == len(sched)
    for li, s, o in zip(layers, res.sel, res.out):
        assert np.array_equal(o, sparse_attention(li.q_main, q8.codes, q8.scales, s, li.swa))
