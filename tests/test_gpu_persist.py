"""GPU: a cache saved from HBM and reloaded gives back the same codes and scales,
keys formed again from them bit-identical to the keys written with the cache
(and to the oracle's), and a decode step on the reloaded cache identical to the
step before saving.  Parked windows come back byte exact."""
import numpy as np
import pytest
import torch

import synth
from helpers import dev, dev_bf16, host_bf16_bits
from oracle.csa2 import indexer_k, quant_fp4

pytestmark = pytest.mark.gpu


def test_persist_reload_and_step(tmp_path):
    from kv_cache_compression_03_amd import binding as bd, persist, schedule as sch
    wl = synth.workload("decode_64k_b64", B=3, N=5000, schedule="FUUU")
    kv = np.stack([synth.main_kv(wl, b) for b in range(wl.B)])
    W = synth.w_ik(wl)
    Wd = dev_bf16(W)
    codes, scales, kidx = bd.csa2_quant_fp4(dev(kv), W_ik=Wd)
    layers = []
    for li, mode in enumerate(wl.layers):
        qm = np.stack([synth.q_main(wl, li, b) for b in range(wl.B)])
        sw = np.stack([synth.swa_tokens(wl, li, b) for b in range(wl.B)])
        qi = np.stack([synth.q_index(wl, li, b) for b in range(wl.B)]) if mode == "F" else None
        w = np.stack([synth.head_weights(wl, li, b) for b in range(wl.B)]) if mode == "F" else None
        layers.append(sch.LayerBuffers(dev_bf16(qm), dev(sw), None if qi is None else dev_bf16(qi),
                                       None if w is None else dev(w)))
    run = sch.DecodeSchedule(wl.layers, wl.B, wl.N, wl.d, wl.h_i, wl.d_i, wl.H_q, wl.S, wl.K)
    before = [o.clone() for o in run.step(codes, scales, kidx, layers)]
    persist.save_cache(str(tmp_path / "cache"), codes, scales, n_valid=[5000, 4000, 1])
    parked = persist.park_windows([lb.swa for lb in layers])
    assert all(p.is_pinned() for p in parked)
    saved_k = kidx.clone()
    del codes, scales, kidx
    for lb in layers:
        lb.swa.fill_(0)
    c2, s2, k2, nv = persist.load_cache(str(tmp_path / "cache"), W_ik=Wd)
    persist.restore_windows(parked, [lb.swa for lb in layers])
    assert nv == [5000, 4000, 1]
    assert torch.equal(k2, saved_k)
    for b in range(wl.B):
        q8 = quant_fp4(kv[b])
        assert np.array_equal(c2[b].cpu().numpy(), q8.codes)
        assert np.array_equal(s2[b].cpu().numpy(), q8.scales)
        assert np.array_equal(host_bf16_bits(k2[b]), indexer_k(q8.codes, q8.scales, W))
    after = run.step(c2, s2, k2, layers)
    for a, b in zip(before, after):
        assert torch.equal(a, b)


@pytest.mark.parametrize("n,d,d_i", [(1, 512, 128), (300, 256, 64), (2049, 512, 128)])
def test_indexer_keys_of_existing_cache(n, d, d_i):
    """csa2_indexer_keys on codes and scales alone equals the keys the quantiser
    writes (both the few-entry and the batched kernel) and the oracle's."""
    from kv_cache_compression_03_amd import binding as bd
    rng = np.random.default_rng(n + d)
    kv = rng.standard_normal((n, d)).astype(np.float32)
    W = synth.w_ik(synth.workload("decode_64k_b64", d=d, d_i=d_i))
    codes, scales, k1 = bd.csa2_quant_fp4(dev(kv), W_ik=dev_bf16(W))
    k2 = bd.csa2_indexer_keys(codes, scales, dev_bf16(W))
    assert torch.equal(k1, k2)
    q8 = quant_fp4(kv)
    assert np.array_equal(host_bf16_bits(k2), indexer_k(q8.codes, q8.scales, W))
