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
//   * a workgroup owns one query row, up to 64 heads and a contiguous range of
//     32-key chunks (split-K over the keys); its waves are (16-head group) x
//     (half of the dims): a wave reduces QK over its half of the dims (the pair
//     sums partial logits through LDS) and accumulates O for its half, so it
//     holds 32 registers of Q and 64 of O, and two waves fit per SIMD;
//   * workgroup ids are mapped XCD-aware: a row's splits and head groups share
//     one XCD's L2;
//   * LDS layouts and the lane-to-data mapping of the dequantisation keep bank
//     conflicts at or below 2-way;
//   * per chunk the workgroup dequantises the 32 keys once into LDS, exactly, as
//     bf16 (E2M1 x E4M3 and E4M3 values fit bf16; hardware FP4/FP8 conversions),
//     in two layouts: key-major for S^T = K·Q^T and dim-major for O += P·V; the
//     next chunk's bytes are loaded while the current chunk is multiplied;
//   * S^T puts heads on MFMA columns, so each lane owns one head's 8 logits and
//     the softmax row reductions are two cross-lane steps; the probabilities in
//     that layout are directly the A operand of P·V (the key order inside the
//     reduction is permuted consistently in P and V);
//   * P is split into bf16 hi + lo parts (two MFMAs), so P·V keeps ~16 bits of
//     the fp32 probabilities; logits and sums stay in fp32;
//   * online softmax in base 2 against a lazily moved reference maximum (no
//     cross-lane traffic on the common path); per-split
//     (O, m, l) partials are merged by a small combine kernel (or written
//     directly when there is one split).
#include "attn_common.h"
#include "common.h"
#include "internal.h"

namespace csa2 {

#ifndef CSA2_ROWS_MAX
#define CSA2_ROWS_MAX 64  // query rows up to which the few-rows kernel runs (measured: faster up to 64)
#endif
#ifndef CSA2_SPLIT_ROWS_MAX
#define CSA2_SPLIT_ROWS_MAX 8  // query rows up to which the two-launch few-rows path runs (measured: faster up to 8)
#endif
#ifndef CSA2_ROWS_DP4_MAX
#define CSA2_ROWS_DP4_MAX 16  // rows up to which it splits the output dims in four (d = 512)
#endif
#ifndef CSA2_WIDE_MIN_WGS
// (row, 64-head group) units from which the many-rows kernel runs: above the
// few-rows kernel's 64 rows it beats the split-K kernels at every row count
// measured (66-128 rows: 44 vs 50-58 us per layer; 384 rows: 67 vs 108 us)
#define CSA2_WIDE_MIN_WGS 65
#endif
#ifndef CSA2_ROWS_DP2_MAX
#define CSA2_ROWS_DP2_MAX 128  // (row, 16-head group) units up to which it splits the output dims in two
#endif

#ifndef CSA2_ATTN_TARGET_WGS
#define CSA2_ATTN_TARGET_WGS 256  // workgroups a launch aims for (splits = target / rows)
#endif

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Waves of a workgroup: HG head groups of 16 heads x DS halves of the output dims.
static inline void attn_shape(int H_q, int d, int& hg, int& ds) {
  const int hpw = H_q / 16;
  hg = (hpw % 4 == 0) ? 4 : ((hpw % 2 == 0) ? 2 : 1);
  ds = 2;
  (void)d;
}

AttnPlan attn_plan(int B, int Tq, int H_q, int K, int L_max) {
  AttnPlan p;
  int hg, ds;
  attn_shape(H_q, 0, hg, ds);
  p.waves = hg * ds;
  p.head_groups = (H_q / 16) / hg;
  const long long base = (long long)B * Tq * p.head_groups;
  const int max_chunks = (K + kKC - 1) / kKC + (L_max - K + kKC - 1) / kKC;  // selection, then window
  long long want = (CSA2_ATTN_TARGET_WGS + base - 1) / base;
  int ns = (int)(want < 1 ? 1 : (want > max_chunks ? max_chunks : want));
  if (ns > kMaxSplits) ns = kMaxSplits;
  if (ns < 1) ns = 1;  // a row with no keys at all (no selection slots, no window)
  p.chunks_per_split = (max_chunks + ns - 1) / ns;
  if (p.chunks_per_split < 1) p.chunks_per_split = 1;
  p.n_splits = (max_chunks + p.chunks_per_split - 1) / p.chunks_per_split;
  return p;
}

size_t attn_ws_bytes(int B, int Tq, int H_q, int d, int K, int L_max) {
  AttnPlan p = attn_plan(B, Tq, H_q, K, L_max);
  const size_t rows = (size_t)B * Tq;
  size_t need = 0;
  if (p.n_splits > 1)
    need = align256(rows * p.n_splits * H_q * d * sizeof(float)) +
           align256(rows * p.n_splits * H_q * 2 * sizeof(float));
  // the two-launch few-rows path (its window bound is checked at launch)
  if (rows <= CSA2_SPLIT_ROWS_MAX && attn_split_supported(H_q, d, K, 0, 0, false, 1.0f)) {
    const size_t s = attn_split_ws_bytes((int)rows, K, L_max - K);
    need = s > need ? s : need;
  }
  return need;
}

template <int D, int HG>
__global__ __launch_bounds__(HG * 2 * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int chunks_per_split,
    int n_splits, int rows, int head_groups, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int DS = 2;                       // output-dim halves
  constexpr int NT = HG * DS * 64;
  constexpr int DH = D / DS;                  // output dims per wave
  constexpr int KSTR = D + 8;                 // key-major row stride (bf16): 16 B pad
  constexpr int VSTR = kKC + 8;               // dim-major row stride (bf16): 80 B
  constexpr int NB = (kKC / 4) * (D / 8);     // 4-key x 8-dim dequantisation blocks
  constexpr int ITER = (NB + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t Krow[kKC * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];
  __shared__ __attribute__((aligned(16))) float s_part[HG * 2 * 64 * 8];  // partial logits
  __shared__ int s_ent[kMaxSel];  // entry of each selection slot this split reads
  __shared__ float s_ksc[kKC];
  __shared__ int s_valid[kKC];

  int row, split, hgrp;
  if (!xcd_map(blockIdx.x, rows, n_splits * head_groups, row, split)) return;
  hgrp = split % head_groups;
  split /= head_groups;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  const int head0 = (hgrp * HG + (wave % HG)) * 16;
  const int dim0 = (wave / HG) * DH;

  // the selection occupies K slots (ascending, -1 padded); slots that are not a
  // valid entry are masked, so no pass over the list is needed first
  const int* srow = sel + (size_t)row * K;
  const int n_sel = N > 0 ? K : 0;

  const WinRange win = window_of(q_pos, row, S, swa_pos0, n_win);
  const int n_swa = win.n;
  // chunks hold keys of one kind: first the selected entries, then the window
  const int nm = (n_sel + kKC - 1) / kKC;
  const int n_chunks = nm + (n_swa + kKC - 1) / kKC;
  const int c_begin = split * chunks_per_split;
  const int c_end = min(n_chunks, c_begin + chunks_per_split);
  // the entries of this split's selection slots, staged once (invalid -> entry 0)
  const int sl_lo = c_begin * kKC, sl_hi = min(c_end, nm) * kKC;
  for (int i = sl_lo + tid; i < sl_hi; i += NT) {
    const int v = i < n_sel ? srow[i] : -1;
    s_ent[i - sl_lo] = (v >= 0 && v < N) ? v : -1;
  }
  __syncthreads();
  // raw bytes of one chunk: per 4-key x 8-dim block, ra = 4 code bytes (or window
  // bytes 0-3), rb = the scale byte (or window bytes 4-7)
  uint32_t ra[ITER][4], rb[ITER][4];
  auto load_chunk = [&](int c) {
    const bool main = c < nm;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int bid = tid + it * NT;
      if (bid < NB) {
        const int kq = bid & 7, dg = bid >> 3;  // 8 key quads per lane octet: conflict-free LDS writes
        if (main) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = max(s_ent[c * kKC + 4 * kq + j - sl_lo], 0);
            const size_t ent = (size_t)b * N + e;
            ra[it][j] = *reinterpret_cast<const uint32_t*>(codes + ent * (D / 2) + 4 * dg);
            rb[it][j] = scales[ent * (D / 16) + (dg >> 1)];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = (c - nm) * kKC + 4 * kq + j;
            const size_t tok = (size_t)b * S + window_slot(win, t < n_swa ? t : 0, S);
            const uint2 raw = *reinterpret_cast<const uint2*>(swa + tok * D + 8 * dg);
            ra[it][j] = raw.x;
            rb[it][j] = raw.y;
          }
        }
      }
    }
  };

  // this wave's half of the QK reduction: dims [dim0, dim0 + DH)
  bf16x8_t qb[DH / 32];
  {
    const uint4* qr = reinterpret_cast<const uint4*>(q + ((size_t)row * H_q + head0 + col) * D + dim0);
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) qb[s] = as_bf16x8(qr[4 * s + g]);
    // Wait for the query here, once.  Otherwise the wait for it is placed inside
    // the chunk loop (the compiler cannot prove it done on loop entry), and since
    // loads retire in order that wait also drains the next chunk's prefetch.
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) asm volatile("" : "+v"(qb[s]));
  }
  f32x4_t o[DH / 16];
#pragma unroll
  for (int n = 0; n < DH / 16; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.0f;

  if (c_begin < c_end) load_chunk(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    const bool main = c < nm;
    lds_barrier();  // the previous chunk's LDS reads are done
    if (tid < kKC) {
      bool valid;
      if (main) {
        valid = s_ent[c * kKC + tid - sl_lo] >= 0;
      } else {
        valid = (c - nm) * kKC + tid < n_swa;
      }
      s_valid[tid] = valid ? 1 : 0;
      s_ksc[tid] = valid ? (main ? 1.0f : swa_scale) : 0.0f;
    }
    // ---- dequantise (exactly, to bf16) into the key-major and dim-major layouts
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int bid = tid + it * NT;
      if (bid < NB) {
        const int kq = bid & 7, dg = bid >> 3;  // 8 key quads per lane octet: conflict-free LDS writes
        uint32_t v[4][4];  // [key][dim pair] packed bf16 pairs
        if (main) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float sc = e4m3_decode(rb[it][j]);
            const uint32_t cw = ra[it][j];
            f32x2_t x;
            x = fp4x2_to_f32<0>(cw); v[j][0] = pack_hi16(x[0] * sc, x[1] * sc);
            x = fp4x2_to_f32<1>(cw); v[j][1] = pack_hi16(x[0] * sc, x[1] * sc);
            x = fp4x2_to_f32<2>(cw); v[j][2] = pack_hi16(x[0] * sc, x[1] * sc);
            x = fp4x2_to_f32<3>(cw); v[j][3] = pack_hi16(x[0] * sc, x[1] * sc);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j][0] = e4m3x2_to_bf16x2<false>(ra[it][j]);
            v[j][1] = e4m3x2_to_bf16x2<true>(ra[it][j]);
            v[j][2] = e4m3x2_to_bf16x2<false>(rb[it][j]);
            v[j][3] = e4m3x2_to_bf16x2<true>(rb[it][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(&Krow[(4 * kq + j) * KSTR + 8 * dg]) =
              make_uint4(v[j][0], v[j][1], v[j][2], v[j][3]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // dim 8dg+i of keys 4kq..4kq+3: low halves for even i, high halves for odd i
          const uint32_t sel2 = (i & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t w0 = __builtin_amdgcn_perm(v[1][i >> 1], v[0][i >> 1], sel2);
          const uint32_t w1 = __builtin_amdgcn_perm(v[3][i >> 1], v[2][i >> 1], sel2);
          *reinterpret_cast<uint2*>(&Vt[(8 * dg + i) * VSTR + 4 * kq]) = make_uint2(w0, w1);
        }
      }
    }
    lds_barrier();
    // the next chunk's loads fly while this chunk is multiplied
    if (c + 1 < c_end) load_chunk(c + 1);

    // ---- S^T = K·Q^T: rows = keys (two 16-key tiles), columns = this wave's heads
    // each wave of a pair reduces over its half of the dims; the halves are summed
    // through LDS (a + b == b + a, so both waves hold identical logits)
    f32x4_t st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&Krow[col * KSTR + dim0 + 32 * s + 8 * g]);
      const bf16x8_t a1 =
          *reinterpret_cast<const bf16x8_t*>(&Krow[(16 + col) * KSTR + dim0 + 32 * s + 8 * g]);
      st0 = mfma16x16x32(a0, qb[s], st0);
      st1 = mfma16x16x32(a1, qb[s], st1);
    }
    {
      float4* mine = reinterpret_cast<float4*>(&s_part[(wave * 64 + lane) * 8]);
      mine[0] = make_float4(st0[0], st0[1], st0[2], st0[3]);
      mine[1] = make_float4(st1[0], st1[1], st1[2], st1[3]);
      lds_barrier();
      const float4* other = reinterpret_cast<const float4*>(&s_part[(((wave + HG) % (2 * HG)) * 64 + lane) * 8]);
      const float4 o0 = other[0], o1 = other[1];
      st0[0] += o0.x; st0[1] += o0.y; st0[2] += o0.z; st0[3] += o0.w;
      st1[0] += o1.x; st1[1] += o1.y; st1[2] += o1.z; st1[3] += o1.w;
    }
    // lane owns head `col`, keys 4g+i (tile 0) and 16+4g+i (tile 1)
    float lg[8], ks[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = 4 * g + i, k1 = 16 + 4 * g + i;
      ks[i] = s_ksc[k0];
      ks[4 + i] = s_ksc[k1];
      lg[i] = s_valid[k0] ? st0[i] * ks[i] * sm_log2 : -INFINITY;
      lg[4 + i] = s_valid[k1] ? st1[i] * ks[4 + i] * sm_log2 : -INFINITY;
    }
    // Lazy reference maximum: the four lane groups of a head only need to agree on
    // it when one of them sees a logit more than 2^kLazy above it (the first chunk,
    // or rarely later); then, and only then, the maximum is reduced across lanes.
    float lmax = lg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) lmax = fmaxf(lmax, lg[i]);
    const bool grow = lmax > m_ref + kLazy || (m_ref == -INFINITY && lmax != -INFINITY);
    float alpha = 1.0f;
    if (__ballot(grow)) {
      float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      if (cmax > m_ref + kLazy || (m_ref == -INFINITY && cmax != -INFINITY)) {
        alpha = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - cmax);
        m_ref = cmax;
      }
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int n = 0; n < DH / 16; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= al[i];
      }
    }
    // probabilities (this lane's share of the row sum is kept per lane)
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lg[i] - m_ref);
      l_run += p[i];
    }
    // P (scaled by the key's value scale) as hi + lo bf16 A operands: hi keeps the
    // top 8 significant bits, lo the next 8 of the exact remainder
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float x0 = p[2 * jj] * ks[2 * jj], x1 = p[2 * jj + 1] * ks[2 * jj + 1];
      const float h0 = __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u);
      const float h1 = __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u);
      hw[jj] = pack_hi16(h0, h1);
      lw[jj] = pack_hi16(x0 - h0, x1 - h1);
    }
    const bf16x8_t ahi = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
    const bf16x8_t alo = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
    // ---- O += P·V over this wave's dims; V slots follow P's key order.  Each V
    // fragment is read once and used by the hi and the lo MFMA.
#pragma unroll
    for (int n0 = 0; n0 < DH / 16; n0 += 4) {
      bf16x8_t bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint16_t* vr = &Vt[(dim0 + 16 * (n0 + u) + col) * VSTR];
        const uint2 v0 = *reinterpret_cast<const uint2*>(vr + 4 * g);
        const uint2 v1 = *reinterpret_cast<const uint2*>(vr + 16 + 4 * g);
        bv[u] = as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) o[n0 + u] = mfma16x16x32(ahi, bv[u], o[n0 + u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) o[n0 + u] = mfma16x16x32(alo, bv[u], o[n0 + u]);
    }
  }

  // ---- epilogue: row sums were kept per lane group
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float lr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lr[i] = __shfl(l_run, 4 * g + i);
  if (n_splits == 1) {
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t h = (size_t)row * H_q + head0 + 4 * g + i;
        out[h * D + dim0 + 16 * n + col] = lr[i] > 0.0f ? o[n][i] / lr[i] : 0.0f;
      }
    }
    if (lse != nullptr && lane < 16 && dim0 == 0)
      lse[(size_t)row * H_q + head0 + col] =
          l_run > 0.0f ? (m_ref + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  } else {
    const size_t base = ((size_t)row * n_splits + split) * H_q;
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part_o[(base + head0 + 4 * g + i) * D + dim0 + 16 * n + col] = o[n][i];
    }
    if (lane < 16 && dim0 == 0) {
      part_ml[(base + head0 + col) * 2 + 0] = m_ref;
      part_ml[(base + head0 + col) * 2 + 1] = l_run;
    }
  }
}

__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, int H_q, int D, int rows,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[2];
  int row, h;
  if (!xcd_map(blockIdx.x, rows, H_q, row, h)) return;
  const int tid = threadIdx.x;
  const size_t base = (size_t)row * n_splits * H_q + h;  // split s of this head: base + s*H_q
  float ms = -INFINITY, ls = 0.0f;
  if (tid < n_splits) {
    ms = part_ml[(base + (size_t)tid * H_q) * 2];
    ls = part_ml[(base + (size_t)tid * H_q) * 2 + 1];
  }
  float M = ms;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (tid < 64 && (tid & 63) == 0) red[0] = M;
  __syncthreads();
  M = red[0];
  const float e = (tid < n_splits && ms != -INFINITY) ? exp2f(ms - M) : 0.0f;
  float wsum = ls * e;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o);
  if (tid == 0) red[1] = wsum;
  if (tid < n_splits) wgt[tid] = e;
  __syncthreads();
  wsum = red[1];
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  for (int d4 = tid; d4 < D / 4; d4 += 128) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // splits in batches whose loads are all in flight together (one memory round
    // trip per batch rather than per split); summed in split order
    constexpr int BATCH = 8;
    for (int s0 = 0; s0 < n_splits; s0 += BATCH) {
      float4 v[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int s = s0 + u;
        v[u] = s < n_splits ? reinterpret_cast<const float4*>(part_o + (base + (size_t)s * H_q) * D)[d4]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int s = s0 + u;
        const float ws = s < n_splits ? wgt[s] : 0.0f;
        if (ws != 0.0f) {
          acc.x += v[u].x * ws;
          acc.y += v[u].y * ws;
          acc.z += v[u].z * ws;
          acc.w += v[u].w * ws;
        }
      }
    }
    reinterpret_cast<float4*>(out + ((size_t)row * H_q + h) * D)[d4] =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (lse != nullptr && tid == 0)
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
  const float sm_log2_rows = sm_scale * 1.4426950408889634f;
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(scales) |
                           reinterpret_cast<uintptr_t>(swa) | reinterpret_cast<uintptr_t>(q) |
                           reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  // Few rows at 64 heads and 512 dims: each key decoded and scored once per row,
  // then P·V over (row, 16 heads, 64 dims) workgroups.
  // (a call with no keys at all needs no workspace: only the second launch runs)
  if (aligned16 && rows <= CSA2_SPLIT_ROWS_MAX &&
      attn_split_supported(H_q, d, K, S, n_win, q_pos != nullptr, swa_scale) &&
      (ws != nullptr || attn_split_ws_bytes(rows, K, S) == 0))
    return launch_sparse_attn_split(q, codes, scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win,
                                    q_pos, Tq, sm_log2_rows, rows, ws, out, lse, st);
  // Few rows (decode steps): every key of a row inside one workgroup per (row, 16
  // heads, output-dim part), no split partials and no combine launch.
  if (aligned16 && rows <= CSA2_ROWS_MAX &&
      attn_rows_supported(H_q, d, K, S, n_win, q_pos != nullptr, swa_scale)) {
    // output-dim parts: more workgroups (each with less to merge) when rows are few
    const int dp = (rows <= CSA2_ROWS_DP4_MAX && d == 512) ? 4 : rows * (H_q / 16) <= CSA2_ROWS_DP2_MAX ? 2 : 1;
    return launch_sparse_attn_rows(q, codes, scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win,
                                   q_pos, Tq, H_q, d, sm_log2_rows, rows, dp, out, lse, st);
  }
  // More rows (prefill chunks, several queries per sequence): a workgroup per (row,
  // 64 heads), every logit and softmax term computed once, no split partials.
  if (aligned16 && (long long)rows * (H_q / 64) >= CSA2_WIDE_MIN_WGS &&
      attn_wide_supported(H_q, d, K, N, S, swa_scale))
    return launch_sparse_attn_wide(q, codes, scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win,
                                   q_pos, Tq, H_q, d, sm_log2_rows, rows, out, lse, st);
  const bool f16 = attn_f16_supported(H_q, d, swa_scale);
  AttnPlan p = attn_plan(B, Tq, H_q, K, L_max);
  // Rows so few that every split holds a single chunk: the fp16 kernel runs each
  // row as two 32-head workgroups instead (each chunk decoded twice) over half
  // as many splits, which halves the split partials written, flushed and merged
  // (8 rows x 64 heads: 16.6 -> 15.0 us per layer).  With more chunks per split
  // the extra decode costs more than it saves.
  const bool split_heads = f16 && (H_q / 32) % 2 == 0 && p.n_splits > 1 && p.chunks_per_split == 1;
  if (split_heads) p = attn_plan(2 * B, Tq, H_q, K, L_max);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (p.n_splits > 1) {
    part_o = static_cast<float*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       align256((size_t)rows * p.n_splits * H_q * d * sizeof(float)));
  }
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  const bool aligned = ((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(scales) |
                         reinterpret_cast<uintptr_t>(swa)) & 15) == 0;
  if (aligned && f16) {
    hipError_t e = launch_sparse_attn_f16(q, codes, scales, N, sel, K, swa, swa_scale, S, swa_pos0,
                                          n_win, q_pos, Tq, H_q, d, sm_log2, p, rows,
                                          split_heads ? 1 : ((H_q / 32) % 2 == 0 ? 2 : 1), part_o,
                                          part_ml, out, lse, st);
    if (e != hipSuccess) return e;
  } else {
    dim3 grid(xcd_grid(rows, p.n_splits * p.head_groups));
    const int hg = p.waves / 2;
  #define CSA2_ATTN(D_, HG_)                                                                          \
    hipLaunchKernelGGL((sparse_attn_kernel<D_, HG_>), grid, dim3(HG_ * 2 * 64), 0, st, q, codes, scales, \
                       N, sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq, H_q, sm_log2,          \
                       p.chunks_per_split, p.n_splits, rows, p.head_groups, part_o, part_ml, out, lse)
    if (d == 512) {
      if (hg == 4) CSA2_ATTN(512, 4);
      else if (hg == 2) CSA2_ATTN(512, 2);
      else CSA2_ATTN(512, 1);
    } else {
      if (hg == 4) CSA2_ATTN(256, 4);
      else if (hg == 2) CSA2_ATTN(256, 2);
      else CSA2_ATTN(256, 1);
    }
#undef CSA2_ATTN
  }
  if (p.n_splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3(xcd_grid(rows, H_q)), dim3(128), 0, st, part_o,
                       part_ml, p.n_splits, H_q, d, rows, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
