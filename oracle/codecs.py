"""Number formats of the CSA2 state, written out from their definitions.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.

Formats and where they come from
--------------------------------
* FP4 E2M1 main-KV elements with one FP8 E4M3 scale per 16 channels: named by
  the daily report "DeepSeek V4.1 Flash 将 KV 压缩推到模型架构层" (blog.baizx.cool,
  2026-09-11, section "核心机制") and by the deep dive "DeepSeek-V4.1-Flash"
  (tanjunchen.github.io, 2026-09-13, §3.4 "FP4 Main KV 与 SWA Bounded Replay"),
  which also states that the sliding-window KV stays in FP8.
* The pages name the formats only.  Their bit layouts are the standard ones:
  E2M1 = 1 sign, 2 exponent (bias 1), 1 mantissa bit, no inf/NaN, max 6;
  E4M3FN = 1 sign, 4 exponent (bias 7), 3 mantissa bits, max 448, only
  S.1111.111 is NaN (no infinities).
* bf16 = the upper half of an IEEE binary32.

Rounding rules (readings, the pages are silent): every cast rounds to nearest
with ties to even and saturates at the format maximum instead of producing
NaN/inf.

Everything here works on float64 values.  Scaling by powers of two and
``np.rint`` (round half to even) are exact in float64 for these ranges, so each
encoder below is "divide by the grid spacing of the value's binade, round to an
integer, multiply back, look the value up in the code table".
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 value of bf16 numbers given as uint16 bit patterns."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values straight to bf16 (nearest, ties to even).

    Returns uint16 bit patterns.  One rounding only (no detour through
    float32).  Finite inputs within the bf16 range are required.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding of a non-finite value")
    a = np.abs(x)
    _, e = np.frexp(a)  # a = f * 2**e, f in [0.5, 1)
    # bf16 keeps 8 significant bits; below 2**-126 the spacing is fixed (subnormals).
    e = np.maximum(e, -125)
    spacing = np.ldexp(1.0, e - 8)
    r = np.rint(a / spacing) * spacing
    if np.any(r > 3.3895313892515355e38):
        raise ValueError("bf16 overflow")
    r = np.where(np.signbit(x), -r, r)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# FP8 E4M3FN
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of E4M3FN codes (uint8).  0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


# finite non-negative grid and its codes, ascending (codes 0x00..0x7E)
_E4M3_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_E4M3_POS_VALUES = e4m3_decode(_E4M3_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Round to E4M3FN: nearest, ties to even, saturating at +-448.  uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("E4M3 encoding of a non-finite value")
    a = np.abs(x)
    _, E = np.frexp(a)  # floor(log2 a) = E - 1 for a > 0
    # binade exponent; everything below 2**-6 shares the subnormal spacing 2**-9
    e = np.maximum(E - 1, -6)
    spacing = np.ldexp(1.0, e - 3)
    r = np.rint(a / spacing) * spacing
    r = np.minimum(r, E4M3_MAX)
    idx = np.searchsorted(_E4M3_POS_VALUES, r)
    if not np.array_equal(_E4M3_POS_VALUES[idx], r):
        raise AssertionError("E4M3 grid lookup failed")
    code = _E4M3_POS_CODES[idx]
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


# --------------------------------------------------------------------------
# FP4 E2M1
# --------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # codes 0..7


def e2m1_decode(codes) -> np.ndarray:
    """Value of E2M1 codes (low 4 bits of each integer); bit 3 is the sign."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_VALUES[c & 0x7]
    return np.where(c & 0x8, -mag, mag)


def e2m1_encode(x) -> np.ndarray:
    """Round to E2M1: nearest, ties to even, saturating at +-6.

    The sign bit is the sign bit of the input, so -0 and small negatives that
    round to zero give code 0x8.  Returns uint8 codes 0..15.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("E2M1 encoding of a non-finite value")
    a = np.abs(x)
    # grid spacing: 0.5 on [0, 2), 1 on [2, 4), 2 on [4, 6]
    spacing = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / spacing) * spacing, E2M1_MAX)
    idx = np.searchsorted(E2M1_VALUES, r)
    if not np.array_equal(E2M1_VALUES[idx], r):
        raise AssertionError("E2M1 grid lookup failed")
    code = idx.astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x8), code).astype(np.uint8)
