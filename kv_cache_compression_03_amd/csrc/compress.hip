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
// result is rounded once to float32.  This path serves float32 inputs and a
// scalar Z; bf16 inputs take the MFMA kernel below.
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

// ---------------------------------------------------------------- bf16 on MFMA
// For bf16 hidden states and weights (a timed prefill: thousands of tokens at
// d_model 5,120) the projections run on MFMA with fp32 accumulation.  A
// workgroup computes 256 tokens x 64 channels of C and the same 64 channels of
// Z; a wave owns 64 tokens x all 128 columns (its A fragments are reused over
// 8 column tiles).  H and W pass through LDS in 64-deep slices, double-buffered
// and fetched one slice ahead; W is transposed on the way in so that every
// fragment is one 16-byte LDS read.  An MFMA output lane holds 4 consecutive
// tokens of one channel in C and in Z, so the fold (m in {1,2,4}) needs no
// communication; the RoPE partner channel sits in the neighbouring lane.
constexpr int kMT = 256;        // tokens per workgroup
constexpr int kMC = 64;         // channels of C (and of Z) per workgroup
constexpr int kMK = 64;         // reduction slice
constexpr int kMP = kMK + 8;    // LDS pitch (bf16) of a staged H row / W column: 16 B pad

template <int M>
__global__ __launch_bounds__(256, 1) void compress_mfma_kernel(
    const uint16_t* __restrict__ H, int T, int d_model, const uint16_t* __restrict__ Wkv,
    const uint16_t* __restrict__ Wz, int d, long long pos0, int rope_dim, double theta, int n_ent,
    int n_cg, int n_per_seq, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t hs[2][kMT * kMP];
  __shared__ __attribute__((aligned(16))) uint16_t wsm[2][2 * kMC * kMP];
  // workgroup -> (token group, channel group); the channel groups of one token
  // group get ids equal mod 8, i.e. one XCD, and share its H slice in that L2
  const int L = blockIdx.x;
  const int tg = (L & 7) + 8 * (L / (8 * n_cg));
  const int cg = (L >> 3) % n_cg;
  const int b = blockIdx.y;
  const int T_used = n_ent * M;
  const int t_base = tg * kMT, c_base = cg * kMC;
  if (t_base >= T_used) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  const uint16_t* Hb = H + (size_t)b * T * d_model;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  // staging: H rows (token) x 8 chunks of 16 B per slice, 8 chunks per thread;
  // W: thread = (4 reduction rows kq, 8 columns co) of the 64 x 128 slice
  u32x4 sh[8], sw[4];
  const int kq = tid & 15, co = tid >> 4;
  const uint16_t* wsrc = co < 8 ? Wkv + c_base + 8 * co : Wz + c_base + 8 * (co - 8);
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = tid + 256 * u, row = c >> 3, part = c & 7;
      const int t = min(t_base + row, T_used - 1);
      sh[u] = *reinterpret_cast<const u32x4*>(Hb + (size_t)t * d_model + k0 + 8 * part);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sw[r] = *reinterpret_cast<const u32x4*>(wsrc + (size_t)(k0 + 4 * kq + r) * d);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = tid + 256 * u, row = c >> 3, part = c & 7;
      *reinterpret_cast<u32x4*>(&hs[buf][row * kMP + 8 * part]) = sh[u];
    }
    // column 8co + j gets reduction rows 4kq .. 4kq+3 (8 bytes)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int hi = j & 1, wd = j >> 1;
      const uint32_t e0 = sw[0][wd], e1 = sw[1][wd], e2 = sw[2][wd], e3 = sw[3][wd];
      const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
      const u32x2 v = {__builtin_amdgcn_perm(e1, e0, sel), __builtin_amdgcn_perm(e3, e2, sel)};
      *reinterpret_cast<u32x2*>(&wsm[buf][(8 * co + j) * kMP + 4 * kq]) = v;
    }
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int n_k = d_model / kMK;
  fetch(0);
  stash(0);
  fetch(min(1, n_k - 1) * kMK);
  lds_barrier();
  for (int kc = 0; kc < n_k; ++kc) {
    const int buf = kc & 1;
#pragma unroll
    for (int s = 0; s < kMK / 32; ++s) {
      bf16x8_t a[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        a[rt] = *reinterpret_cast<const bf16x8_t*>(&hs[buf][(64 * wave + 16 * rt + col) * kMP + 32 * s + 8 * g]);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&wsm[buf][(16 * ct + col) * kMP + 32 * s + 8 * g]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt][ct] = mfma16x16x32(a[rt], bv, acc[rt][ct]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // buffer buf^1 was last read in pass kc-1, before that pass's barrier
    stash(buf ^ 1);
    fetch(min(kc + 2, n_k - 1) * kMK);
    lds_barrier();
  }

  // ---- fold and RoPE: lane holds tokens t0+i (i = 0..3) of channel c in C and Z
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int t0 = t_base + 64 * wave + 16 * rt + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int c = c_base + 16 * ct + col;
      const f32x4_t cv = acc[rt][ct], zv = acc[rt][ct + 4];
#pragma unroll
      for (int e = 0; e < 4 / M; ++e) {
        float zmax = zv[e * M];
#pragma unroll
        for (int j = 1; j < M; ++j) zmax = fmaxf(zmax, zv[e * M + j]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
          const float a = expf(zv[e * M + j] - zmax);
          den += a;
          num = fmaf(a, cv[e * M + j], num);
        }
        float kv = num / den;
        const int ent = (t0 + e * M) / M;
        if (rope_dim > 0 && c_base + kMC > d - rope_dim) {  // workgroup-uniform
          const float other = __shfl_xor(kv, 1);
          if (c >= d - rope_dim) {
            const int i = (c - (d - rope_dim)) >> 1;
            // position inside its own sequence (n_per_seq < n_ent when short
            // sequences were laid end to end)
            const double pos = (double)(pos0 + (long long)(ent % n_per_seq + 1) * M - 1);
            double sn, cs;
            sincos(pos * pow(theta, -2.0 * i / rope_dim), &sn, &cs);
            const double u = (c & 1) ? other : kv, v = (c & 1) ? kv : other;
            kv = (float)((c & 1) ? u * sn + v * cs : u * cs - v * sn);
          }
        }
        if (ent < n_ent) out[((size_t)b * n_ent + ent) * d + c] = kv;
      }
    }
  }
}

// ---- a few tokens (a decode step's new blocks): at most 64 tokens in all
// (B sequences of T tokens laid end to end).  The prefill kernel gives each
// workgroup the whole 5,120-deep reduction for 64 channels, which at 64 tokens
// leaves the GPU nearly idle.  Here a workgroup owns 8 channels (16 MFMA
// columns: 8 of C, 8 of Z) of one 16-token tile, and its NW waves (16 when
// d_model allows, else 4) split the reduction: wave w sums dims
// [w*d_model/NW, (w+1)*d_model/NW) into a partial [16 tokens x 16 columns]
// tile, the tiles are added through LDS in wave order, and the first wave runs
// the fold and RoPE as in the prefill kernel (a lane holds 4 consecutive tokens
// of one column; Z of the same channel is 8 lanes away).  A workgroup moves its
// tile's hidden states and its channels' weight columns: one tile per
// workgroup keeps the bytes through each CU small and spreads the work over
// four times as many CUs as whole-batch workgroups would.
// Per 32-deep step a wave loads its 16 weight columns (16 B per lane: 8 channels
// of W_KV or of W_Z of one reduction row), transposes them through a private LDS
// tile and reads the tile's A operand straight from global memory; the next
// step's loads are in flight during this step's MFMA.
constexpr int kFewTok = 64;   // tokens the kernel takes in all
constexpr int kFewCh = 8;     // channels per workgroup
constexpr int kFewTP = 40;    // LDS pitch (bf16) of a transposed weight column

template <int M, int NW>
__global__ __launch_bounds__(64 * NW) void compress_few_kernel(
    const uint16_t* __restrict__ H, int n_tok, int d_model, const uint16_t* __restrict__ Wkv,
    const uint16_t* __restrict__ Wz, int d, long long pos0, int rope_dim, double theta,
    int n_per_seq, int n_cg, int n_tt, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[NW][16 * kFewTP];  // per wave: [column][k]
  __shared__ __attribute__((aligned(16))) float part[NW][64 * 4];         // per wave: 64 lanes x 4
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  // Workgroups go to the 8 XCDs round-robin by id.  The token tiles of a
  // channel group, and consecutive channel groups, are placed on one XCD (when
  // the channel groups are a multiple of 8), so each 128-byte line of weights
  // is fetched into one XCD's L2, not into all eight.
  int cg, tt;
  if (n_cg & 7) {
    cg = (int)blockIdx.x / n_tt;
    tt = (int)blockIdx.x - cg * n_tt;
  } else {
    const int k = (int)(blockIdx.x >> 3);
    cg = (int)(blockIdx.x & 7) * (n_cg >> 3) + k / n_tt;
    tt = k % n_tt;
  }
  const int c0 = cg * kFewCh;
  const int kq = d_model / NW, k_lo = wave * kq;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // weight loads: lane l = reduction row l/2 of the step, W_KV (l even) or W_Z (odd)
  const uint16_t* wsrc = ((lane & 1) ? Wz : Wkv) + (size_t)(k_lo + (lane >> 1)) * d + c0;
  // A rows: token 16 tt + col (clamped: rows past n_tok repeat the last token and are never stored)
  const uint16_t* hrow = H + (size_t)min(16 * tt + col, n_tok - 1) * d_model + k_lo + 8 * g;
  u32x4 wv, ha, wv_n, ha_n;
  auto load = [&](int s, u32x4& w, u32x4& h) {
    w = *reinterpret_cast<const u32x4*>(wsrc + (size_t)s * 32 * d);
    h = *reinterpret_cast<const u32x4*>(hrow + 32 * s);
  };
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int n_steps = kq / 32;
  uint16_t* tile = wt[wave];
  load(0, wv, ha);
  for (int s = 0; s < n_steps; ++s) {
    if (s + 1 < n_steps) load(s + 1, wv_n, ha_n);
    // transpose: column (lane&1)*8 + j gets reduction row lane/2
    {
      const uint16_t* v = reinterpret_cast<const uint16_t*>(&wv);
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[((lane & 1) * 8 + j) * kFewTP + (lane >> 1)] = v[j];
    }
    // the wave reads back what it wrote: LDS serves one wave in order; the wait
    // keeps the compiler from moving the read above the writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&tile[col * kFewTP + 8 * g]);
    acc = mfma16x16x32(as_bf16x8(make_uint4(ha[0], ha[1], ha[2], ha[3])), b, acc);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is rewritten next step
    if (s + 1 < n_steps) {
      wv = wv_n;
      ha = ha_n;
    }
  }
  // ---- the NW partial tiles, added in wave order
  reinterpret_cast<float4*>(part[wave])[lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (wave != 0) return;
  // lane holds tokens 16 tt + 4g + i of column col
  f32x4_t tot = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    float4 a[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) a[w] = reinterpret_cast<const float4*>(part[w])[lane];
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += f32x4_t{a[w].x, a[w].y, a[w].z, a[w].w};
  }
  // columns 0-7 hold C, 8-15 Z of channels c0 .. c0+7: the Z of this lane's
  // channel is 8 lanes away
  f32x4_t zv;
#pragma unroll
  for (int i = 0; i < 4; ++i) zv[i] = __shfl_xor(tot[i], 8);
  const bool is_c = col < 8;
  const int c = c0 + (col & 7);
  const int t0 = 16 * tt + 4 * g;
#pragma unroll
  for (int e = 0; e < 4 / M; ++e) {
    float zmax = zv[e * M];
#pragma unroll
    for (int j = 1; j < M; ++j) zmax = fmaxf(zmax, zv[e * M + j]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const float a = expf(zv[e * M + j] - zmax);
      den += a;
      num = fmaf(a, tot[e * M + j], num);
    }
    float kv = num / den;
    const int ent = (t0 + e * M) / M;
    if (rope_dim > 0 && c0 + kFewCh > d - rope_dim) {  // workgroup-uniform
      const float other = __shfl_xor(kv, 1);
      if (c >= d - rope_dim) {
        const int i = (c - (d - rope_dim)) >> 1;
        const double pos = (double)(pos0 + (long long)(ent % n_per_seq + 1) * M - 1);
        double sn, cs;
        sincos(pos * pow(theta, -2.0 * i / rope_dim), &sn, &cs);
        const double u = (c & 1) ? other : kv, v = (c & 1) ? kv : other;
        kv = (float)((c & 1) ? u * sn + v * cs : u * cs - v * sn);
      }
    }
    if (is_c && t0 + e * M < n_tok) out[(size_t)ent * d + c] = kv;
  }
}

bool compress_mfma_ok(bool bf16_in, int d_model, int d, int d_z) {
  return bf16_in && d_z == d && d % kMC == 0 && d_model % kMK == 0;
}

hipError_t launch_compress(const void* H, bool bf16_in, int B, int T, int d_model, const void* W_kv,
                           const void* W_z, int d, int d_z, int m, long long pos0, int rope_dim,
                           double rope_theta, float* kv_out, hipStream_t st) {
  const int n_ent = T / m;
  if (B == 0 || n_ent == 0) return hipSuccess;
  if (compress_mfma_ok(bf16_in, d_model, d, d_z) && (long long)B * T <= kFewTok && T % m == 0 &&
      d_model % 128 == 0 && d % kFewCh == 0) {
    const int nt = B * T;
    const int n_cg = d / kFewCh, n_tt = (nt + 15) / 16;
#define CSA2_FEW(M_, NW_)                                                                             \
  hipLaunchKernelGGL((compress_few_kernel<M_, NW_>), dim3(n_cg * n_tt), dim3(64 * NW_), 0, st,        \
                     static_cast<const uint16_t*>(H), nt, d_model, static_cast<const uint16_t*>(W_kv), \
                     static_cast<const uint16_t*>(W_z), d, pos0, rope_dim, rope_theta, n_ent, n_cg, n_tt, \
                     kv_out)
    if (d_model % (32 * 16) == 0) {
      if (m == 1) CSA2_FEW(1, 16);
      else if (m == 2) CSA2_FEW(2, 16);
      else CSA2_FEW(4, 16);
    } else {
      if (m == 1) CSA2_FEW(1, 4);
      else if (m == 2) CSA2_FEW(2, 4);
      else CSA2_FEW(4, 4);
    }
#undef CSA2_FEW
    return hipGetLastError();
  }
  if (compress_mfma_ok(bf16_in, d_model, d, d_z)) {
    // Sequences shorter than a token tile whose tokens all fold (a decode step's
    // new block per sequence) are laid end to end as one run of B*T tokens: the
    // rows of [B, T, d_model] are contiguous and blocks never cross a sequence,
    // so only the RoPE position changes (taken inside each sequence).
    const bool flat = B > 1 && T % m == 0 && T < kMT;
    const int Bl = flat ? 1 : B, Tl = flat ? B * T : T, nl = flat ? B * n_ent : n_ent;
    const int n_tg = (nl * m + kMT - 1) / kMT, n_cg = d / kMC;
    dim3 g2((unsigned)(8 * ((n_tg + 7) / 8) * n_cg), (unsigned)Bl);
#define CSA2_COMPM(M_)                                                                                \
  hipLaunchKernelGGL((compress_mfma_kernel<M_>), g2, dim3(256), 0, st, static_cast<const uint16_t*>(H), \
                     Tl, d_model, static_cast<const uint16_t*>(W_kv), static_cast<const uint16_t*>(W_z), d, \
                     pos0, rope_dim, rope_theta, nl, n_cg, n_ent, kv_out)
    if (m == 1) CSA2_COMPM(1);
    else if (m == 2) CSA2_COMPM(2);
    else CSA2_COMPM(4);
#undef CSA2_COMPM
    return hipGetLastError();
  }
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
