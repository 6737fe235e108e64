"""Pins of the FP4 main-KV quantiser and the indexer key."""
import numpy as np
import torch

from conftest import read_golden
from oracle.codecs import bf16_to_f64, e4m3_decode, f64_to_bf16
from oracle.csa2 import dequant_fp4, indexer_k, quant_fp4, unpack_codes


def _cases():
    rows = read_golden("quant_fp4_cases.txt")
    cases, cur = [], None
    for r in rows:
        if r[0] == "case":
            cur = {"name": r[1]}
            cases.append(cur)
        elif r[0] == "x":
            cur["x"] = np.array([float(v) for v in r[1:]], dtype=np.float32)
        elif r[0] == "scale":
            cur["scale"] = int(r[1], 16)
        elif r[0] == "bytes":
            cur["bytes"] = np.array([int(v, 16) for v in r[1:]], dtype=np.uint8)
    return cases


def test_quant_golden_cases():
    for c in _cases():
        q = quant_fp4(c["x"][None, :])
        assert q.scales[0, 0] == c["scale"], c["name"]
        assert np.array_equal(q.codes[0], c["bytes"]), c["name"]


def test_quant_layout_multi_group():
    # two groups per entry: the scale plane holds one byte per 16 channels in channel order
    cs = _cases()
    x = np.concatenate([cs[0]["x"], cs[1]["x"]])[None, :]
    q = quant_fp4(x)
    assert list(q.scales[0]) == [cs[0]["scale"], cs[1]["scale"]]
    assert np.array_equal(q.codes[0], np.concatenate([cs[0]["bytes"], cs[1]["bytes"]]))


def test_error_bound_and_extremes():
    rng = np.random.default_rng(0)
    n, d = 4000, 64
    mag = np.exp(rng.uniform(-9, 9, (n, d // 16, 1)))
    x = (rng.standard_normal((n, d // 16, 16)) * mag).reshape(n, d).astype(np.float32)
    q = quant_fp4(x)
    xh = dequant_fp4(q.codes, q.scales)
    s = np.repeat(e4m3_decode(q.scales), 16, axis=1)
    over = np.abs(x.astype(np.float64) - xh) > s
    # with a normal E4M3 scale (relative rounding <= 2^-4) and no scale saturation, every
    # element lies within one scale step of its value (E2M1 steps are <= 2; a scale rounded
    # down saturates the group maximum by at most 6 * 2^-4 / (1 - 2^-4) < 1 step)
    amax = np.abs(x).reshape(n, d // 16, 16).max(-1)
    ok = (e4m3_decode(q.scales) >= 2.0 ** -6) & (amax <= 6 * 448)
    inrange = np.repeat(ok, 16, axis=1)
    assert inrange.mean() > 0.5
    assert not np.any(over & inrange)
    # the largest element of a group with a normal scale always becomes +-6: the scale is
    # within 2^-4 of amax/6, so amax/s lies in (5.6, 6.4] and rounds or saturates to 6
    codes = unpack_codes(q.codes).reshape(n, d // 16, 16)
    g = np.abs(x).reshape(n, d // 16, 16)
    am = g.argmax(-1)
    top = np.take_along_axis(codes, am[..., None], -1)[..., 0] & 7
    nz = e4m3_decode(q.scales) >= 2.0 ** -6
    assert np.all(top[nz] == 7)


def test_zero_scale_gives_signed_zero():
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 3] = -1e-4
    x[0, 4] = 2e-4
    q = quant_fp4(x)
    assert q.scales[0, 0] == 0
    c = unpack_codes(q.codes)[0]
    assert c[3] == 8 and c[4] == 0 and np.all(dequant_fp4(q.codes, q.scales) == 0)


def test_dequant_exact_in_bf16():
    # E2M1 (<=2 significant bits) times E4M3 (<=4 bits) fits bf16's 8 bits: a kernel may hold
    # dequantised entries as bf16 without loss
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((2000, 128)) * np.exp(rng.uniform(-6, 6, (2000, 1)))).astype(np.float32)
    q = quant_fp4(x)
    xh = dequant_fp4(q.codes, q.scales)
    assert np.array_equal(bf16_to_f64(f64_to_bf16(xh)), xh)


def test_indexer_k_linear_and_rounded_once():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    q = quant_fp4(x)
    W = f64_to_bf16(rng.standard_normal((32, 8)) / 6)
    k = bf16_to_f64(indexer_k(q.codes, q.scales, W))
    xh = dequant_fp4(q.codes, q.scales)
    exact = xh @ bf16_to_f64(W)
    # one nearest-even rounding of the exact product: agrees with torch's float64->float32->bf16
    # wherever float32 holds the product exactly; always within half a bf16 ulp
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert np.all(np.abs(k - exact) <= ulp / 2)
    # linearity: doubling W doubles k exactly (power-of-two scaling)
    k2 = bf16_to_f64(indexer_k(q.codes, q.scales, f64_to_bf16(2 * bf16_to_f64(W))))
    assert np.array_equal(k2, 2 * k)
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).double().numpy()
    same32 = exact.astype(np.float32).astype(np.float64) == exact
    assert np.array_equal(k[same32], ref[same32])
