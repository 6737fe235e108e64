// Compressor: hidden states -> roped main-KV entries.
//
// [deep-dive §2] C = H·W_KV (entries) and Z = H·W_Z (compression weights);
// [deep-dive §3.1] each run of m tokens folds into one entry, without overlap and
// without any absolute position in the fold; [deep-dive §3.4] RoPE is applied
// before quantisation.  Readings: per-channel softmax over the block of Z
// weights the block's C; only complete blocks make entries; entry j sits at
// p_j = pos0 + (j+1)m - 1; the last rope_dim channels turn in adjacent pairs by
// p_j * theta^(-2i/r).
//
// One workgroup computes 32 tokens x 64 channels of both C and Z in float64
// (tiles of H and W staged through LDS), then folds and rotates in registers:
// each thread owns 4 consecutive tokens (whole blocks for m in {1,2,4}) of one
// channel pair, so the fold and the pair rotation need no communication.  The
// result is rounded once to float32.  This path serves cache builds; it is
// vector fp64 work, not tuned for a timed prefill.
#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kCT = 32;  // tokens per tile
constexpr int kCC = 64;  // channels per tile
constexpr int kCK = 16;  // reduction slice

template <typename TIn>
CSA2_DEV double ld(const TIn* p, size_t i);
template <>
CSA2_DEV double ld<float>(const float* p, size_t i) { return (double)p[i]; }
template <>
CSA2_DEV double ld<uint16_t>(const uint16_t* p, size_t i) { return (double)bf16_to_f32(p[i]); }

template <typename TIn, int m>
__global__ __launch_bounds__(256) void compress_kernel(const TIn* __restrict__ H, int T, int d_model,
                                                       const TIn* __restrict__ Wkv,
                                                       const TIn* __restrict__ Wz, int d, int d_z,
                                                       long long pos0, int rope_dim,
                                                       double theta, int n_ent,
                                                       float* __restrict__ out) {
  __shared__ double hs[kCT][kCK + 1];
  __shared__ double wk[kCK][kCC];
  __shared__ double wz[kCK][kCC];
  const int b = blockIdx.z;
  const int c_base = blockIdx.x * kCC;
  const int t_base = blockIdx.y * kCT;
  const int tid = threadIdx.x;
  const int pr = tid & 31, tg = tid >> 5;  // channel pair, token group
  const int c0 = c_base + 2 * pr;
  const int T_used = n_ent * m;
  const TIn* Hb = H + (size_t)b * T * d_model;
  const bool zfull = d_z != 1;

  double accC[4][2], accZ[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) accC[j][0] = accC[j][1] = accZ[j][0] = accZ[j][1] = 0.0;

  for (int k0 = 0; k0 < d_model; k0 += kCK) {
    for (int i = tid; i < kCT * kCK; i += 256) {
      const int tt = i / kCK, kk = i % kCK;
      const int t = t_base + tt, k = k0 + kk;
      hs[tt][kk] = (t < T_used && k < d_model) ? ld(Hb, (size_t)t * d_model + k) : 0.0;
    }
    for (int i = tid; i < kCK * kCC; i += 256) {
      const int kk = i / kCC, cc = i % kCC;
      const int k = k0 + kk, c = c_base + cc;
      const bool ok = k < d_model && c < d;
      wk[kk][cc] = ok ? ld(Wkv, (size_t)k * d + c) : 0.0;
      wz[kk][cc] = ok ? (zfull ? ld(Wz, (size_t)k * d_z + c) : ld(Wz, (size_t)k)) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kCK; ++kk) {
      const double w0 = wk[kk][2 * pr], w1 = wk[kk][2 * pr + 1];
      const double z0 = wz[kk][2 * pr], z1 = wz[kk][2 * pr + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double h = hs[tg * 4 + j][kk];
        accC[j][0] = fma(h, w0, accC[j][0]);
        accC[j][1] = fma(h, w1, accC[j][1]);
        accZ[j][0] = fma(h, z0, accZ[j][0]);
        accZ[j][1] = fma(h, z1, accZ[j][1]);
      }
    }
    __syncthreads();
  }

  if (c0 >= d) return;
  const int tok0 = t_base + tg * 4;  // first token of this thread (multiple of m)
#pragma unroll
  for (int e = 0; e < 4 / m; ++e) {
    const int ent = (tok0 + e * m) / m;
    if (ent >= n_ent) break;
    double kv[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      double zmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < m; ++j) zmax = fmax(zmax, accZ[e * m + j][q]);
      double num = 0.0, den = 0.0;
#pragma unroll
      for (int j = 0; j < m; ++j) {
        const double a = exp(accZ[e * m + j][q] - zmax);
        den += a;
        num += a * accC[e * m + j][q];
      }
      kv[q] = num / den;
    }
    if (c0 >= d - rope_dim) {
      const int i = (c0 - (d - rope_dim)) / 2;
      const double pos = (double)(pos0 + (long long)(ent + 1) * m - 1);
      const double ang = pos * pow(theta, -2.0 * i / rope_dim);
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double u = kv[0], v = kv[1];
      kv[0] = u * cs - v * sn;
      kv[1] = u * sn + v * cs;
    }
    float* dst = out + ((size_t)b * n_ent + ent) * d + c0;
    dst[0] = (float)kv[0];
    dst[1] = (float)kv[1];
  }
}

hipError_t launch_compress(const void* H, bool bf16_in, int B, int T, int d_model, const void* W_kv,
                           const void* W_z, int d, int d_z, int m, long long pos0, int rope_dim,
                           double rope_theta, float* kv_out, hipStream_t st) {
  const int n_ent = T / m;
  if (B == 0 || n_ent == 0) return hipSuccess;
  dim3 grid((d + kCC - 1) / kCC, (n_ent * m + kCT - 1) / kCT, B);
#define CSA2_COMP(TIN, M_)                                                                          \
  hipLaunchKernelGGL((compress_kernel<TIN, M_>), grid, dim3(256), 0, st, static_cast<const TIN*>(H), \
                     T, d_model, static_cast<const TIN*>(W_kv), static_cast<const TIN*>(W_z), d, d_z, \
                     pos0, rope_dim, rope_theta, n_ent, kv_out)
  if (bf16_in) {
    if (m == 1) CSA2_COMP(uint16_t, 1);
    else if (m == 2) CSA2_COMP(uint16_t, 2);
    else CSA2_COMP(uint16_t, 4);
  } else {
    if (m == 1) CSA2_COMP(float, 1);
    else if (m == 2) CSA2_COMP(float, 2);
    else CSA2_COMP(float, 4);
  }
#undef CSA2_COMP
  return hipGetLastError();
}

}  // namespace csa2
