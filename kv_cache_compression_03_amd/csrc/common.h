// Device helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEV __device__ __forceinline__
#define CSA2_HOST_DEV __host__ __device__

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// Word 3 of a raw buffer descriptor (gfx9 family: 32-bit data format); a buffer
// access whose offset falls outside the descriptor's range reads zero / is dropped.
constexpr int kRawBufferWord3 = 0x00020000;

// ---------------------------------------------------------------- bf16

CSA2_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bf16, nearest-even (finite inputs).
CSA2_DEV uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// float64 -> bf16 with a single nearest-even rounding (finite inputs).
CSA2_DEV uint32_t f64_to_bf16_rne(double x) {
  const double tiny = 1.1754943508222875e-38;  // 2^-126, smallest normal bf16
  if (fabs(x) < tiny) {
    // subnormal range: fixed spacing 2^-133; the rounded value is exact in float
    double r = rint(x * 0x1p133) * 0x1p-133;
    return __float_as_uint((float)r) >> 16;
  }
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint64_t r = u + ((1ull << 44) - 1) + ((u >> 45) & 1ull);  // round away the low 45 mantissa bits
  uint32_t sign = (uint32_t)(r >> 63);
  int e = (int)((r >> 52) & 0x7FF) - 1023 + 127;
  uint32_t mant = (uint32_t)((r >> 45) & 0x7F);
  if (e >= 255) return (sign << 15) | 0x7F80u;  // overflow -> inf (out of the supported range)
  return (sign << 15) | ((uint32_t)e << 7) | mant;
}

// ---------------------------------------------------------------- FP8 E4M3FN

// Non-negative finite float32 -> E4M3FN code, nearest-even, saturating at 448.
CSA2_DEV uint32_t e4m3_encode_nonneg(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)rintf(v * 512.0f);  // spacing 2^-9 below 2^-6; 8 -> 0x08
  uint32_t u = __float_as_uint(v);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;  // biased exponent | 3 mantissa bits
  return r - (120u << 3);
}

// E4M3FN code -> float32 (exact).  Codes 0x7F/0xFF (NaN) are not expected.
CSA2_DEV float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// E4M3FN code -> bf16 bits (exact: 3 mantissa bits fit in 7).
CSA2_DEV uint32_t e4m3_to_bf16(uint32_t c) { return __float_as_uint(e4m3_decode(c)) >> 16; }

// ---------------------------------------------------------------- FP4 E2M1

// float32 -> E2M1 code, nearest-even, saturating at 6, sign bit of the input kept.
CSA2_DEV uint32_t e2m1_encode(float q) {
  float a = fabsf(q);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(q) >> 28) & 8u);
}

// E2M1 code (4 bits) -> float32 (exact).
CSA2_DEV float e2m1_decode(uint32_t c) {
  uint32_t mcode = c & 7u;
  uint32_t bits = mcode >= 2u ? ((((mcode >> 1) + 126u) << 23) | ((mcode & 1u) << 22))
                              : (mcode ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// ---------------------------------------------------------------- ordering keys

// Order-preserving map of a float onto uint32 (-0 is folded onto +0 first).
CSA2_DEV uint32_t mono_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
CSA2_DEV float mono_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------- MFMA

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Layout (wave64): lane l holds
// A row l%16 / B column l%16 with 8 reduction elements of slot group l/16, and D
// rows 4*(l/16)+i, column l%16 in element i.
CSA2_DEV f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

CSA2_DEV bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---------------------------------------------------------------- hardware conversions
// Both checked exhaustively against the definitions on gfx950: with a unit scale
// the FP4 one yields the exact E2M1 values of the two nibbles of byte `sel` (low
// nibble first) and the FP8 one the exact bf16 images of two E4M3 bytes (low or
// high 16-bit half of the word).  (The FP4 path applies only the exponent of a
// non-unit scale, so scales are multiplied separately.)
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

template <int SEL>
CSA2_DEV f32x2_t fp4x2_to_f32(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL); }

template <bool HI>
CSA2_DEV uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// high halves of two floats -> packed bf16 pair (exact when both are bf16 values)
CSA2_DEV uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// ---------------------------------------------------------------- barriers

// Workgroup barrier for LDS traffic only.  __syncthreads() is a workgroup fence
// plus s_barrier, and the fence makes every wave wait for all of its outstanding
// global loads first, which would serialise prefetches issued before the
// barrier.  Here only LDS operations are drained (lgkmcnt); loads in flight keep
// flying and the compiler still waits for their registers before first use.
CSA2_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- wave reductions

// All-lanes reductions without LDS traffic: DPP moves inside each 16-lane row
// (swap within quads, then rotate the row by 4 and by 8 lanes) leave every lane
// of a row holding the row's result; one v_readlane per row and three scalar
// steps finish.  (A __shfl_xor butterfly is six ds_bpermute round trips.)  Every
// lane of the wave must be active.
template <int CTRL>
CSA2_DEV int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;  // row_ror:4
constexpr int kDppRowRor8 = 0x128;  // row_ror:8
template <typename Op>
CSA2_DEV int wave_reduce_i32(int v, Op op) {
  v = op(v, dpp_mov<kDppQuadXor1>(v));
  v = op(v, dpp_mov<kDppQuadXor2>(v));
  v = op(v, dpp_mov<kDppRowRor4>(v));
  v = op(v, dpp_mov<kDppRowRor8>(v));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return op(op(a, b), op(c, d));
}
// Maximum over each 16-lane row of the wave, in every lane of the row (DPP only).
CSA2_DEV float row16_max(float v) {
  auto mx = [](int x, int y) { return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y))); };
  int x = __float_as_int(v);
  x = mx(x, dpp_mov<kDppQuadXor1>(x));
  x = mx(x, dpp_mov<kDppQuadXor2>(x));
  x = mx(x, dpp_mov<kDppRowRor4>(x));
  x = mx(x, dpp_mov<kDppRowRor8>(x));
  return __int_as_float(x);
}
CSA2_DEV float wave_max(float v) {
  return __int_as_float(wave_reduce_i32(__float_as_int(v), [](int x, int y) {
    return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y)));
  }));
}
CSA2_DEV float wave_min(float v) {
  return __int_as_float(wave_reduce_i32(__float_as_int(v), [](int x, int y) {
    return __float_as_int(fminf(__int_as_float(x), __int_as_float(y)));
  }));
}
CSA2_DEV uint32_t wave_max_u32(uint32_t v) {
  return (uint32_t)wave_reduce_i32((int)v, [](int x, int y) { return (int)max((uint32_t)x, (uint32_t)y); });
}
CSA2_DEV unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long x = __shfl_xor(v, o);
    v = x > v ? x : v;
  }
  return v;
}
