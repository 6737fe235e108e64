// Sparse attention: main Q attends to (selected FP4 entries ++ layer-local FP8 window).
//
// [deep-dive §3.1] Main Q attends to the selected main KV plus the layer-local
// SWA KV; [digest 已确认] the selected entries are concatenated with the windowed
// KV; [reading §4.2] every layer has its own query and window.  Readings: K = V =
// the whole dequantised entry, shared by all query heads; one softmax over all
// keys; window tokens are E4M3 values times swa_scale.
//
// All H_q heads share each key, so per query the work is a dense
// [H_q x d]·[d x keys] and [H_q x keys]·[keys x d] pair: at 64 heads it is about
// 200 flops per byte of keys, so both products run on MFMA (16x16x32 bf16):
//   * a workgroup owns one query row, 16*WAVES heads (one wave per 16 heads) and
//     a contiguous range of 32-key chunks (split-K over the keys);
//   * per chunk the workgroup dequantises the 32 keys once into LDS, exactly, as
//     bf16 (E2M1 x E4M3 and E4M3 values fit bf16), in two layouts: key-major for
//     S^T = K·Q^T and dim-major for O += P·V;
//   * S^T puts heads on MFMA columns, so each lane owns one head's 8 logits and
//     the softmax row reductions are two cross-lane steps; the probabilities in
//     that layout are directly the A operand of P·V (the key order inside the
//     reduction is permuted consistently in P and V);
//   * P is split into bf16 hi + lo parts (two MFMAs), so P·V keeps ~16 bits of
//     the fp32 probabilities; logits and sums stay in fp32;
//   * online softmax in base 2; per-split (O, m, l) partials are merged by a
//     small combine kernel (or written directly when there is one split).
#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kKC = 32;  // keys per chunk

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

AttnPlan attn_plan(int B, int Tq, int H_q, int K, int L_max) {
  AttnPlan p;
  const int hpw = H_q / 16;
  p.waves = (hpw % 4 == 0) ? 4 : ((hpw % 2 == 0) ? 2 : 1);
  p.head_groups = hpw / p.waves;
  const long long base = (long long)B * Tq * p.head_groups;
  const int max_chunks = (L_max + kKC - 1) / kKC;
  long long want = (256 + base - 1) / base;
  int ns = (int)(want < 1 ? 1 : (want > max_chunks ? max_chunks : want));
  if (ns < 1) ns = 1;
  p.chunks_per_split = (max_chunks + ns - 1) / ns;
  if (p.chunks_per_split < 1) p.chunks_per_split = 1;
  p.n_splits = max_chunks > 0 ? (max_chunks + p.chunks_per_split - 1) / p.chunks_per_split : 1;
  return p;
}

size_t attn_ws_bytes(int B, int Tq, int H_q, int d, int K, int L_max) {
  AttnPlan p = attn_plan(B, Tq, H_q, K, L_max);
  if (p.n_splits <= 1) return 0;
  const size_t rows = (size_t)B * Tq;
  return align256(rows * p.n_splits * H_q * d * sizeof(float)) +
         align256(rows * p.n_splits * H_q * 2 * sizeof(float));
}

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int chunks_per_split,
    int n_splits, float* __restrict__ part_o, float* __restrict__ part_ml,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = WAVES * 64;
  constexpr int KSTR = D + 8;     // key-major row stride (bf16): 16 B pad
  constexpr int VSTR = kKC + 4;   // dim-major row stride (bf16): 72 B
  __shared__ __attribute__((aligned(16))) uint16_t Krow[kKC * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];
  __shared__ int s_src[kKC];      // >= 0 entry, <= -2 window token (-2 - row), -1 none
  __shared__ float s_ksc[kKC];
  __shared__ int s_nsel;

  const int split = blockIdx.x, row = blockIdx.y, hg = blockIdx.z;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  const int head0 = (hg * WAVES + wave) * 16;

  // valid selections form a prefix (ascending list padded with -1)
  const int* srow = sel + (size_t)row * K;
  if (tid == 0) s_nsel = 0;
  __syncthreads();
  int cv = 0;
  for (int i = tid; i < K; i += NT) cv += srow[i] >= 0 ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cv += __shfl_xor(cv, o);
  if (lane == 0) atomicAdd(&s_nsel, cv);
  __syncthreads();
  const int n_sel = s_nsel;

  int swa_lo = 0, n_swa = S;
  if (q_pos != nullptr) {
    const long long t = q_pos[row];
    long long lo = t - n_win + 1 - swa_pos0, hi = t - swa_pos0 + 1;
    lo = lo < 0 ? 0 : lo;
    hi = hi > S ? S : hi;
    swa_lo = (int)lo;
    n_swa = hi > lo ? (int)(hi - lo) : 0;
  }
  const int L = n_sel + n_swa;
  const int n_chunks = (L + kKC - 1) / kKC;
  const int c_begin = split * chunks_per_split;
  const int c_end = min(n_chunks, c_begin + chunks_per_split);

  bf16x8_t qb[D / 32];
  {
    const uint4* qr = reinterpret_cast<const uint4*>(q + ((size_t)row * H_q + head0 + col) * D);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qb[s] = as_bf16x8(qr[4 * s + g]);
  }
  f32x4_t o[D / 16];
#pragma unroll
  for (int n = 0; n < D / 16; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int c = c_begin; c < c_end; ++c) {
    __syncthreads();
    if (tid < kKC) {
      const int slot = c * kKC + tid;
      int src = -1;
      float ksc = 0.0f;
      if (slot < n_sel) {
        const int e = srow[slot];
        if (e >= 0 && e < N) {
          src = e;
          ksc = 1.0f;
        }
      } else if (slot < L) {
        src = -2 - (swa_lo + (slot - n_sel));
        ksc = swa_scale;
      }
      s_src[tid] = src;
      s_ksc[tid] = ksc;
    }
    __syncthreads();
    // ---- dequantise 32 keys into both LDS layouts; a thread owns 8 keys x 8 dims
    for (int bid = tid; bid < (kKC / 8) * (D / 8); bid += NT) {
      const int kg = bid / (D / 8), dg = bid - kg * (D / 8);
      uint32_t v[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int src = s_src[8 * kg + j];
        if (src >= 0) {
          const size_t ent = (size_t)b * N + src;
          const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + ent * (D / 2) + 4 * dg);
          const float sc = e4m3_decode(scales[ent * (D / 16) + (dg >> 1)]);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float lo = e2m1_decode((cw >> (8 * p)) & 15u) * sc;
            const float hi = e2m1_decode((cw >> (8 * p + 4)) & 15u) * sc;
            v[j][p] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
          }
        } else if (src <= -2) {
          const size_t tok = (size_t)b * S + (size_t)(-2 - src);
          const uint2 raw = *reinterpret_cast<const uint2*>(swa + tok * D + 8 * dg);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t wd = p < 2 ? raw.x : raw.y;
            const uint32_t b0 = (wd >> (16 * (p & 1))) & 0xFFu, b1 = (wd >> (16 * (p & 1) + 8)) & 0xFFu;
            v[j][p] = e4m3_to_bf16(b0) | (e4m3_to_bf16(b1) << 16);
          }
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) v[j][p] = 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint4*>(&Krow[(8 * kg + j) * KSTR + 8 * dg]) =
            make_uint4(v[j][0], v[j][1], v[j][2], v[j][3]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sh = 16 * (i & 1), p = i >> 1;
        uint32_t wds[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          wds[jj] = ((v[2 * jj][p] >> sh) & 0xFFFFu) | (((v[2 * jj + 1][p] >> sh) & 0xFFFFu) << 16);
        uint2* dst = reinterpret_cast<uint2*>(&Vt[(8 * dg + i) * VSTR + 8 * kg]);
        dst[0] = make_uint2(wds[0], wds[1]);
        dst[1] = make_uint2(wds[2], wds[3]);
      }
    }
    __syncthreads();

    // ---- S^T = K·Q^T: rows = keys (two 16-key tiles), columns = this wave's heads
    f32x4_t st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&Krow[col * KSTR + 32 * s + 8 * g]);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(&Krow[(16 + col) * KSTR + 32 * s + 8 * g]);
      st0 = mfma16x16x32(a0, qb[s], st0);
      st1 = mfma16x16x32(a1, qb[s], st1);
    }
    // lane owns head `col`, keys 4g+i (tile 0) and 16+4g+i (tile 1)
    float lg[8], ks[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = 4 * g + i, k1 = 16 + 4 * g + i;
      ks[i] = s_ksc[k0];
      ks[4 + i] = s_ksc[k1];
      lg[i] = s_src[k0] != -1 ? st0[i] * ks[i] * sm_log2 : -INFINITY;
      lg[4 + i] = s_src[k1] != -1 ? st1[i] * ks[4 + i] * sm_log2 : -INFINITY;
    }
    float cmax = lg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, lg[i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    float alpha = 1.0f, p[8], psum = 0.0f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.0f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2f(lg[i] - m_new);
        psum += p[i];
      }
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale: this lane's O rows are heads 4g+i
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= al[i];
    }
    // P (scaled by the key's value scale) as hi + lo bf16 A operands
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float x0 = p[2 * jj] * ks[2 * jj], x1 = p[2 * jj + 1] * ks[2 * jj + 1];
      const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
      const uint32_t l0 = f32_to_bf16_rne(x0 - bf16_to_f32(h0));
      const uint32_t l1 = f32_to_bf16_rne(x1 - bf16_to_f32(h1));
      hw[jj] = h0 | (h1 << 16);
      lw[jj] = l0 | (l1 << 16);
    }
    const bf16x8_t ahi = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
    const bf16x8_t alo = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
    // ---- O += P·V, one 16-dim tile per step; V slots follow P's key order
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const uint16_t* vr = &Vt[(16 * n + col) * VSTR];
      const uint2 v0 = *reinterpret_cast<const uint2*>(vr + 4 * g);
      const uint2 v1 = *reinterpret_cast<const uint2*>(vr + 16 + 4 * g);
      const bf16x8_t bv = as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
      o[n] = mfma16x16x32(ahi, bv, o[n]);
      o[n] = mfma16x16x32(alo, bv, o[n]);
    }
  }

  // ---- epilogue
  float lr[4], mr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lr[i] = __shfl(l_run, 4 * g + i);
    mr[i] = __shfl(m_run, 4 * g + i);
  }
  if (n_splits == 1) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t h = (size_t)row * H_q + head0 + 4 * g + i;
        out[h * D + 16 * n + col] = lr[i] > 0.0f ? o[n][i] / lr[i] : 0.0f;
      }
    }
    if (lse != nullptr && lane < 16)
      lse[(size_t)row * H_q + head0 + col] =
          l_run > 0.0f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  } else {
    const size_t base = ((size_t)row * n_splits + split) * H_q;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) part_o[(base + head0 + 4 * g + i) * D + 16 * n + col] = o[n][i];
    }
    if (lane < 16) {
      part_ml[(base + head0 + col) * 2 + 0] = m_run;
      part_ml[(base + head0 + col) * 2 + 1] = l_run;
    }
  }
}

__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, int H_q, int D,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int row = blockIdx.x, h = blockIdx.y;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s)
    M = fmaxf(M, part_ml[(((size_t)row * n_splits + s) * H_q + h) * 2]);
  float wsum = 0.0f;
  for (int s = 0; s < n_splits; ++s) {
    const size_t ix = (((size_t)row * n_splits + s) * H_q + h) * 2;
    const float ms = part_ml[ix];
    if (ms != -INFINITY) wsum += part_ml[ix + 1] * exp2f(ms - M);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  for (int dd = threadIdx.x; dd < D; dd += 128) {
    float acc = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
      const size_t ix = ((size_t)row * n_splits + s) * H_q + h;
      const float ms = part_ml[ix * 2];
      if (ms != -INFINITY) acc += part_o[ix * D + dd] * exp2f(ms - M);
    }
    out[((size_t)row * H_q + h) * D + dd] = acc * inv;
  }
  if (lse != nullptr && threadIdx.x == 0)
    lse[(size_t)row * H_q + h] = wsum > 0.0f ? (M + log2f(wsum)) * 0.69314718055994531f : -INFINITY;
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, int N,
                              const int* sel, int K, const uint8_t* swa, float swa_scale, int S,
                              long long swa_pos0, int n_win, const int* q_pos, int B, int Tq,
                              int H_q, int d, float sm_scale, float* out, float* lse, void* ws,
                              hipStream_t st) {
  const int rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const int L_max = K + S;  // same bound as the workspace query
  const AttnPlan p = attn_plan(B, Tq, H_q, K, L_max);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (p.n_splits > 1) {
    part_o = static_cast<float*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       align256((size_t)rows * p.n_splits * H_q * d * sizeof(float)));
  }
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  dim3 grid(p.n_splits, rows, p.head_groups);
#define CSA2_ATTN(D_, W_)                                                                          \
  hipLaunchKernelGGL((sparse_attn_kernel<D_, W_>), grid, dim3(W_ * 64), 0, st, q, codes, scales, N, \
                     sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq, H_q, sm_log2,           \
                     p.chunks_per_split, p.n_splits, part_o, part_ml, out, lse)
  if (d == 512) {
    if (p.waves == 4) CSA2_ATTN(512, 4);
    else if (p.waves == 2) CSA2_ATTN(512, 2);
    else CSA2_ATTN(512, 1);
  } else {
    if (p.waves == 4) CSA2_ATTN(256, 4);
    else if (p.waves == 2) CSA2_ATTN(256, 2);
    else CSA2_ATTN(256, 1);
  }
#undef CSA2_ATTN
  if (p.n_splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3(rows, H_q), dim3(128), 0, st, part_o, part_ml,
                       p.n_splits, H_q, d, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
