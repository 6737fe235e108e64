// FP4 main-KV quantisation and the indexer-key projection.
//
// [daily 核心机制; deep-dive §3.4] main KV as E2M1 elements with one E4M3 scale
// per 16 channels, quantised after RoPE; [deep-dive §3.1] the indexer K is a
// projection of the main KV.  Readings: absmax scale s = E4M3(amax/6), codes
// E2M1(x/s), both nearest-even and saturating; the key is projected from the
// dequantised entry and stored as bf16.
//
// quant: one thread per 16-channel group (64 B in, 8 B codes + 1 B scale out),
//        consecutive threads on consecutive groups, so loads and stores are
//        contiguous.  fp32 divisions are IEEE correctly rounded (built with
//        -fhip-fp32-correctly-rounded-divide-sqrt), which makes the codes
//        bit-identical to any other correct implementation of the same rule.
// indexer_k: 16 entries per workgroup are dequantised into LDS (fp32, exact),
//        then each thread accumulates one key channel of several entries in
//        float64 and rounds once to bf16.
// Both place entry e of their input at cache row e * cap + row (cap = 1, row = 0:
// contiguous), so a decode step can write one new entry per sequence into row n
// of a [B, cap, ...] cache.
// swa_append: one thread per 16 values of a new token's window KV, E4M3 codes
//        into one slot of each window buffer.
#include "common.h"
#include "internal.h"

namespace csa2 {

// One group of 16 channels: scale byte S = E4M3(amax / 6) and the E2M1 codes of
// x / s as two words (channel i in bits 4(i mod 8) of word i / 8).
CSA2_DEV void quant_group16(const float (&x)[16], uint32_t& w0, uint32_t& w1, uint32_t& S) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  S = e4m3_encode_nonneg(amax / 6.0f);
  const float s = e4m3_decode(S);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c = s > 0.0f ? e2m1_encode(x[i] / s) : ((__float_as_uint(x[i]) >> 28) & 8u);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  w0 = w[0];
  w1 = w[1];
}

__global__ __launch_bounds__(256) void quant_fp4_kernel(const float* __restrict__ kv,
                                                        long long ngroups, int gpe, long long cap,
                                                        long long row,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const long long e = g / gpe;
  const long long go = (e * cap + row) * gpe + (g - e * gpe);  // output group
  const float4* src = reinterpret_cast<const float4*>(kv) + g * 4;
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 v = src[i];
    x[4 * i + 0] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
  uint32_t w0, w1, S;
  quant_group16(x, w0, w1, S);
  reinterpret_cast<uint2*>(codes)[go] = make_uint2(w0, w1);
  scales[go] = (uint8_t)S;
}

hipError_t launch_quant_fp4(const float* kv, long long n, int d, uint8_t* codes, uint8_t* scales,
                            hipStream_t st, long long cap, long long row) {
  long long ngroups = n * (d / 16);
  if (ngroups == 0) return hipSuccess;
  long long blocks = (ngroups + 255) / 256;
  hipLaunchKernelGGL(quant_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, st, kv, ngroups, d / 16,
                     cap, row, codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ indexer key

// entries per workgroup: 16, or 2 for small batches (a decode step's new
// entries), where 16 would leave most of the GPU idle
template <int DI, int kIkEntries>
__global__ __launch_bounds__(256) void indexer_k_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        long long n, int d, long long cap,
                                                        long long row,
                                                        const uint16_t* __restrict__ W,
                                                        uint16_t* __restrict__ out) {
  extern __shared__ float xs[];  // [kIkEntries][d]
  const long long e0 = (long long)blockIdx.x * kIkEntries;
  const int slabs = d / 8;
  for (int t = threadIdx.x; t < kIkEntries * slabs; t += 256) {
    const int el = t / slabs, sl = t - el * slabs;
    const long long e = e0 + el, r = e * cap + row;
    float v[8];
    if (e < n) {
      uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + r * (d / 2) + sl * 4);
      float s = e4m3_decode(scales[r * (d / 16) + (sl >> 1)]);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e2m1_decode((cw >> (4 * j)) & 15u) * s;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[el * d + sl * 8 + j] = v[j];
  }
  __syncthreads();
  constexpr int GRP = 256 / DI;           // entry groups
  constexpr int PER = kIkEntries / GRP;   // entries per thread
  const int c = threadIdx.x % DI, grp = threadIdx.x / DI;
  double acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.0;
  // weights 16 rows at a time, the next 16 in flight during this block's FMAs
  // (one load per step would wait on a memory round trip every step); the sum
  // still runs over k in order
  constexpr int KB = 16;  // d is a multiple of 32
  uint32_t wb[KB], wn[KB];
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) wb[kk] = W[(size_t)kk * DI + c];
  for (int k0 = 0; k0 < d; k0 += KB) {
    const int kn = k0 + KB < d ? k0 + KB : k0;
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) wn[kk] = W[(size_t)(kn + kk) * DI + c];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const double wv = (double)bf16_to_f32(wb[kk]);
#pragma unroll
      for (int p = 0; p < PER; ++p) acc[p] = fma((double)xs[(grp + p * GRP) * d + k0 + kk], wv, acc[p]);
    }
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) wb[kk] = wn[kk];
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const long long e = e0 + grp + p * GRP;
    if (e < n) out[(e * cap + row) * DI + c] = (uint16_t)f64_to_bf16_rne(acc[p]);
  }
}

// A few hundred entries at most (a decode step's new entries): the kernel above
// would give each of a handful of workgroups the whole projection and one long
// chain of dependent float64 FMAs per thread.  Here a workgroup takes 32 key
// columns of 2 entries and its four waves split the reduction: wave w stages rows
// [w d/4, (w+1) d/4) of its [d x 32] slice of W in LDS (every load in flight at
// once) and sums them in four interleaved float64 chains; the quarters are added
// in wave order and the key is rounded to bf16 once.  Each product of a bf16
// weight and a dequantised FP4 value has at most 14 significant bits, so the
// float64 sum does not depend on its order unless its terms span more than
// about 39 binades.
constexpr int kIkCols = 32, kIkFew = 2;

static inline size_t ik_few_lds_bytes(int d) {
  return (size_t)kIkFew * d * sizeof(float) + (size_t)d * kIkCols * sizeof(uint16_t) + 4 * 64 * sizeof(double);
}

// This wave's rows [w d/4, (w+1) d/4) of the [d x 32] slice of W at column c0,
// into ws ([d][32] bf16): a row is 64 bytes = 4 x 16 B, a wave's rows are at most
// 8 loads per lane (d <= 512), all issued before any is written.
CSA2_DEV void ik_few_stage_w(const uint16_t* __restrict__ W, int DI, int c0, int d, uint16_t* ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = d / 4, k_lo = wave * kq;
  // every load is made (an index past the wave's rows repeats its last chunk) and
  // only the store is conditional, so buf stays in registers: with conditional
  // loads the compiler kept it in scratch memory
  uint4 buf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = min(i * 64 + lane, kq * 4 - 1);
    buf[i] = *reinterpret_cast<const uint4*>(W + (size_t)(k_lo + (t >> 2)) * DI + c0 + 8 * (t & 3));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = i * 64 + lane;
    if (t < kq * 4) reinterpret_cast<uint4*>(ws)[k_lo * 4 + t] = buf[i];
  }
}

// Keys of entries e0, e0+1 (dequantised values in xsf [kIkFew][d]) for columns
// c0 .. c0+31: the workgroup's waves each sum a quarter of the reduction in four
// interleaved float64 chains, the quarters are added in wave order and rounded
// to bf16 once.  Starts with a barrier (xsf and ws must be complete).
CSA2_DEV void ik_few_project(const float* xsf, const uint16_t* ws, double* qs, int d, long long e0,
                             long long n, long long cap, long long row, int DI, int c0,
                             uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = d / 4, k_lo = wave * kq;
  __syncthreads();
  const int el = lane / kIkCols, cc = lane % kIkCols;
  const float* xr = xsf + el * d;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
  for (int k = k_lo; k < k_lo + kq; k += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = fma((double)xr[k + j], (double)bf16_to_f32(ws[(k + j) * kIkCols + cc]), acc[j]);
  }
  qs[wave * 64 + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (wave != 0) return;
  const double sum = (qs[lane] + qs[64 + lane]) + (qs[128 + lane] + qs[192 + lane]);
  const long long e = e0 + el;
  if (e < n) out[(e * cap + row) * DI + c0 + cc] = (uint16_t)f64_to_bf16_rne(sum);
}

// A few hundred entries at most (a decode step's new entries): the kernel above
// would give each of a handful of workgroups the whole projection and one long
// chain of dependent float64 FMAs per thread.  Here a workgroup takes 32 key
// columns of 2 entries and its four waves split the reduction (ik_few_project).
// Each product of a bf16 weight and a dequantised FP4 value has at most 14
// significant bits, so the float64 sum does not depend on its order unless its
// terms span more than about 39 binades.
__global__ __launch_bounds__(256) void indexer_k_few_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            long long n, int d, long long cap,
                                                            long long row, const uint16_t* __restrict__ W,
                                                            int DI, uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) float xsf[];  // [kIkFew][d], [d][kIkCols] bf16, [4][64] f64
  uint16_t* ws = reinterpret_cast<uint16_t*>(xsf + kIkFew * d);
  double* qs = reinterpret_cast<double*>(ws + d * kIkCols);
  const long long e0 = (long long)blockIdx.x * kIkFew;
  const int c0 = blockIdx.y * kIkCols;
  ik_few_stage_w(W, DI, c0, d, ws);
  const int slabs = d / 8;
  for (int t = threadIdx.x; t < kIkFew * slabs; t += 256) {
    const int el = t / slabs, sl = t - el * slabs;
    const long long e = e0 + el, r = e * cap + row;
    float v[8];
    if (e < n) {
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + r * (d / 2) + sl * 4);
      const float sc = e4m3_decode(scales[r * (d / 16) + (sl >> 1)]);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e2m1_decode((cw >> (4 * j)) & 15u) * sc;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xsf[el * d + sl * 8 + j] = v[j];
  }
  ik_few_project(xsf, ws, qs, d, e0, n, cap, row, DI, c0, out);
}

hipError_t launch_indexer_k(const uint8_t* codes, const uint8_t* scales, long long n, int d,
                            const uint16_t* W_ik, int d_i, uint16_t* k_idx, hipStream_t st,
                            long long cap, long long row) {
  if (n == 0) return hipSuccess;
  if (n <= 256 && d <= 512 && (reinterpret_cast<uintptr_t>(W_ik) & 15) == 0) {
    const size_t lds = ik_few_lds_bytes(d);
    hipLaunchKernelGGL(indexer_k_few_kernel, dim3((unsigned)((n + kIkFew - 1) / kIkFew), (unsigned)(d_i / kIkCols)),
                       dim3(256), lds, st, codes, scales, n, d, cap, row, W_ik, d_i, k_idx);
    return hipGetLastError();
  }
  const int E = n >= 1024 ? 16 : 4;
  long long blocks = (n + E - 1) / E;
  size_t lds = (size_t)E * d * sizeof(float);
#define CSA2_IK(DI_, E_)                                                                      \
  hipLaunchKernelGGL((indexer_k_kernel<DI_, E_>), dim3((unsigned)blocks), dim3(256), lds, st, codes, \
                     scales, n, d, cap, row, W_ik, k_idx)
  if (d_i == 128) {
    if (E == 16) CSA2_IK(128, 16);
    else CSA2_IK(128, 4);
  } else {
    if (E == 16) CSA2_IK(64, 16);
    else CSA2_IK(64, 4);
  }
#undef CSA2_IK
  return hipGetLastError();
}

// ------------------------------------------------------------------ window append

// One group of 16 window values: E4M3 codes of x / swa_scale (IEEE division,
// nearest-even, saturating at 448, sign kept: -0 -> 0x80), as four words.
CSA2_DEV uint4 e4m3_group16(const float4* __restrict__ src, float swa_scale) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = src[i];
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y = x[j] / swa_scale;  // IEEE division (correctly rounded build)
      const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
      word |= (sign | e4m3_encode_nonneg(fabsf(y))) << (8 * j);
    }
    w[i] = word;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// win [L, B, d] f32 -> swa[l][b][slot][:] as E4M3 codes of win / swa_scale.
__global__ __launch_bounds__(256) void swa_append_kernel(const float* __restrict__ win, long long ngroups,
                                                         int gpt, int S, int slot, float swa_scale,
                                                         uint8_t* __restrict__ swa) {
  long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const long long tok = g / gpt;  // (layer, sequence)
  const int gi = (int)(g - tok * gpt);
  reinterpret_cast<uint4*>(swa + ((size_t)tok * S + slot) * (size_t)(gpt * 16))[gi] =
      e4m3_group16(reinterpret_cast<const float4*>(win) + g * 4, swa_scale);
}

// The decode-step append in one launch: the first n_key_wgs workgroups each
// quantise 2 new entries (quant_group16), keep the dequantised values in LDS
// for their 32 key columns (ik_few_project) and, for the first column slice,
// write the codes and scales into row `row`; the remaining workgroups encode
// the token's window values into slot `slot` (e4m3_group16).  The results are
// those of quant_fp4_kernel, indexer_k_few_kernel and swa_append_kernel.
__global__ __launch_bounds__(256) void cache_append_kernel(
    const float* __restrict__ kv, int B, int d, long long cap, long long row, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const uint16_t* __restrict__ W, int DI, uint16_t* __restrict__ k_idx,
    int n_key_wgs, const float* __restrict__ win, long long wgroups, int S, int slot, float swa_scale,
    uint8_t* __restrict__ swa) {
  extern __shared__ __attribute__((aligned(16))) float xsf[];  // [kIkFew][d], [d][kIkCols] bf16, [4][64] f64
  const int gpe = d / 16;
  if ((int)blockIdx.x >= n_key_wgs) {  // window slots (workgroup-uniform)
    const long long g = (long long)(blockIdx.x - n_key_wgs) * 256 + threadIdx.x;
    if (g >= wgroups) return;
    const long long tok = g / gpe;  // (layer, sequence)
    const int gi = (int)(g - tok * gpe);
    reinterpret_cast<uint4*>(swa + ((size_t)tok * S + slot) * (size_t)d)[gi] =
        e4m3_group16(reinterpret_cast<const float4*>(win) + g * 4, swa_scale);
    return;
  }
  uint16_t* ws = reinterpret_cast<uint16_t*>(xsf + kIkFew * d);
  double* qs = reinterpret_cast<double*>(ws + d * kIkCols);
  const int ncol = DI / kIkCols;
  const int ex = (int)blockIdx.x / ncol, cy = (int)blockIdx.x - ex * ncol;
  const long long e0 = (long long)ex * kIkFew;
  const int c0 = cy * kIkCols;
  ik_few_stage_w(W, DI, c0, d, ws);
  for (int t = threadIdx.x; t < kIkFew * gpe; t += 256) {
    const int el = t / gpe, gi = t - el * gpe;
    const long long e = e0 + el;
    float x[16];
    if (e < B) {
      const float4* src = reinterpret_cast<const float4*>(kv + (size_t)e * d) + gi * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = src[i];
        x[4 * i + 0] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.0f;
    }
    uint32_t w0, w1, Sc;
    quant_group16(x, w0, w1, Sc);
    const float sc = e4m3_decode(Sc);
#pragma unroll
    for (int j = 0; j < 16; ++j) xsf[el * d + gi * 16 + j] = e2m1_decode(((j < 8 ? w0 : w1) >> (4 * (j & 7))) & 15u) * sc;
    if (cy == 0 && e < B) {
      const long long go = (e * cap + row) * gpe + gi;
      reinterpret_cast<uint2*>(codes)[go] = make_uint2(w0, w1);
      scales[go] = (uint8_t)Sc;
    }
  }
  ik_few_project(xsf, ws, qs, d, e0, B, cap, row, DI, c0, k_idx);
}

bool cache_append_fused_ok(int B, int d, int d_i, const void* W_ik) {
  return B <= 256 && d <= 512 && d % 32 == 0 && (d_i == 64 || d_i == 128) &&
         (reinterpret_cast<uintptr_t>(W_ik) & 15) == 0;
}

hipError_t launch_cache_append(const float* kv, int B, int d, long long cap, long long row, uint8_t* codes,
                               uint8_t* scales, const uint16_t* W_ik, int d_i, uint16_t* k_idx,
                               const float* win, int L, int S, int slot, float swa_scale, uint8_t* swa,
                               hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int n_key_wgs = ((B + kIkFew - 1) / kIkFew) * (d_i / kIkCols);
  const long long wgroups = (L > 0 && win != nullptr) ? (long long)L * B * (d / 16) : 0;
  const long long n_win_wgs = (wgroups + 255) / 256;
  hipLaunchKernelGGL(cache_append_kernel, dim3((unsigned)(n_key_wgs + n_win_wgs)), dim3(256),
                     ik_few_lds_bytes(d), st, kv, B, d, cap, row, codes, scales, W_ik, d_i, k_idx, n_key_wgs,
                     win, wgroups, S, slot, swa_scale, swa);
  return hipGetLastError();
}

hipError_t launch_swa_append(const float* win, int L, int B, int S, int d, int slot, float swa_scale,
                             uint8_t* swa, hipStream_t st) {
  const long long ngroups = (long long)L * B * (d / 16);
  if (ngroups == 0) return hipSuccess;
  const long long blocks = (ngroups + 255) / 256;
  hipLaunchKernelGGL(swa_append_kernel, dim3((unsigned)blocks), dim3(256), 0, st, win, ngroups, d / 16,
                     S, slot, swa_scale, swa);
  return hipGetLastError();
}

}  // namespace csa2
