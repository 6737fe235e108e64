"""Exhaustive pins of the FP4 and FP8 decoding inside csa2_sparse_attn.

The attention kernels turn the cached bytes into fp16 / bf16 operands with
gfx950's scaled conversion instructions ([daily] 核心机制 and [deep-dive] §3.4:
main KV is E2M1 with one E4M3 scale per 16 channels, the window is E4M3).  With a
single key per query the softmax weight is exactly 1, so every head's output is
that key as the kernel decoded it.  These tests make every decoded value visible:

* selected entries: all 16 E2M1 codes in every nibble position, under every one
  of the 254 finite E4M3 scale codes -- output = E2M1 value x scale, exactly;
* window tokens (no selection): all 254 finite E4M3 codes -- output = value x
  swa_scale, exactly at swa_scale 1; at 0.37 the scale enters through the
  probability (a power of two split off in fp16 / a bf16 pair), so the bound is
  2^-10 relative, far below the 1/16 step between neighbouring E4M3 values;
* every kernel: few rows take the one-launch few-rows kernel (32 and 48 heads)
  or the two-launch few-rows path (64 heads); with 136 rows (each query cycling
  over the entries / window tokens) the split-K kernels, 32 heads (fp16) and 48
  heads (bf16), or the many-rows kernel (64 heads).
"""
import numpy as np
import pytest
import torch

from helpers import dev, dev_bf16
from oracle.codecs import e4m3_decode, f64_to_bf16
from oracle.csa2 import dequant_fp4

pytestmark = pytest.mark.gpu

FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 254 codes
D = 512


def bd():
    from kv_cache_compression_03_amd import binding
    return binding


def all_code_entries():
    """Entries whose 32 scale groups run through every finite E4M3 code and whose
    16 channels per group hold the 16 E2M1 codes (rotated per entry and group, so
    each code sits in both nibble positions)."""
    n = -(-FINITE_E4M3.shape[0] // (D // 16))    # 8 entries of 32 groups
    codes = np.zeros((n, D // 2), np.uint8)
    scales = np.zeros((n, D // 16), np.uint8)
    for e in range(n):
        nib = np.zeros(D, np.uint8)
        for g in range(D // 16):
            scales[e, g] = FINITE_E4M3[(e * (D // 16) + g) % FINITE_E4M3.shape[0]]
            nib[16 * g:16 * g + 16] = (np.arange(16) + e + g) % 16
        codes[e] = nib[0::2] | (nib[1::2] << 4)
    return codes, scales


@pytest.mark.parametrize("rows", [8, 136])
@pytest.mark.parametrize("H_q", [32, 48, 64])
def test_every_fp4_code_under_every_scale(H_q, rows):
    codes, scales = all_code_entries()
    n = codes.shape[0]
    assert set(scales.reshape(-1).tolist()) == set(FINITE_E4M3.tolist())
    rng = np.random.default_rng(H_q)
    q = f64_to_bf16(rng.standard_normal((1, rows, H_q, D)))
    sel = (np.arange(rows, dtype=np.int32) % n).reshape(1, rows, 1)   # query t selects entry t mod n
    swa = torch.empty(1, 0, D, dtype=torch.uint8, device="cuda")      # no window
    out = bd().csa2_sparse_attn(dev_bf16(q), dev(codes[None]), dev(scales[None]), dev(sel), swa)
    torch.cuda.synchronize()
    out = out.cpu().numpy()[0]                                         # [rows, H_q, D]
    want = dequant_fp4(codes, scales)                                   # exact, float64
    assert np.all(np.isfinite(want))
    for t in range(rows):
        bad = np.nonzero(out[t] != want[t % n][None, :].astype(np.float32))
        assert bad[0].size == 0, f"query {t}: head {bad[0][0]}, channel {bad[1][0]}: " \
                                 f"{out[t][bad[0][0], bad[1][0]]} vs {want[t % n][bad[1][0]]}"


@pytest.mark.parametrize("Tq", [4, 136])
@pytest.mark.parametrize("H_q", [32, 48, 64])
@pytest.mark.parametrize("swa_scale", [1.0, 0.37])
def test_every_fp8_window_code(H_q, swa_scale, Tq):
    tok = np.stack([FINITE_E4M3[(np.arange(D) + 37 * t) % FINITE_E4M3.shape[0]] for t in range(Tq)])
    assert set(tok[0].tolist()) == set(FINITE_E4M3.tolist())
    rng = np.random.default_rng(7 * H_q)
    q = f64_to_bf16(rng.standard_normal((1, Tq, H_q, D)))
    q_pos = np.arange(Tq, dtype=np.int32).reshape(1, Tq)            # query t sees window slot t only
    codes = torch.zeros(1, 1, D // 2, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(1, 1, D // 16, dtype=torch.uint8, device="cuda")
    sel = torch.empty(1, Tq, 0, dtype=torch.int32, device="cuda")   # K = 0: window only
    out = bd().csa2_sparse_attn(dev_bf16(q), codes, scales, sel, dev(tok[None]), swa_scale=swa_scale,
                                q_pos=dev(q_pos), swa_pos0=0, n_win=1)
    torch.cuda.synchronize()
    out = out.cpu().numpy()[0]
    for t in range(Tq):
        want = e4m3_decode(tok[t]) * swa_scale
        if swa_scale == 1.0:
            assert np.all(out[t] == want[None, :].astype(np.float32)), f"token {t}"
        else:
            assert np.all(np.abs(out[t] - want[None, :]) <= 2.0 ** -10 * np.abs(want)[None, :]), f"token {t}"
