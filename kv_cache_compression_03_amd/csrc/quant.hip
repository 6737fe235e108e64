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
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const uint32_t S = e4m3_encode_nonneg(amax / 6.0f);
  const float s = e4m3_decode(S);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c = s > 0.0f ? e2m1_encode(x[i] / s) : ((__float_as_uint(x[i]) >> 28) & 8u);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  reinterpret_cast<uint2*>(codes)[go] = make_uint2(w[0], w[1]);
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

hipError_t launch_indexer_k(const uint8_t* codes, const uint8_t* scales, long long n, int d,
                            const uint16_t* W_ik, int d_i, uint16_t* k_idx, hipStream_t st,
                            long long cap, long long row) {
  if (n == 0) return hipSuccess;
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

// win [L, B, d] f32 -> swa[l][b][slot][:] as E4M3 codes of win / swa_scale
// (nearest-even, saturating at 448, sign kept: -0 -> 0x80).
__global__ __launch_bounds__(256) void swa_append_kernel(const float* __restrict__ win, long long ngroups,
                                                         int gpt, int S, int slot, float swa_scale,
                                                         uint8_t* __restrict__ swa) {
  long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const long long tok = g / gpt;  // (layer, sequence)
  const int gi = (int)(g - tok * gpt);
  const float4* src = reinterpret_cast<const float4*>(win) + g * 4;
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
  reinterpret_cast<uint4*>(swa + ((size_t)tok * S + slot) * (size_t)(gpt * 16))[gi] =
      make_uint4(w[0], w[1], w[2], w[3]);
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
