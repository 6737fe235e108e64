// Sparse attention for many query rows (prefill chunks): main Q attends to
// (selected FP4 entries ++ layer-local FP8 window).  Same function and readings as
// the other sparse-attention kernels (attn_f16.hip, attn_rows.hip, attn.hip).
//
// [deep-dive §3.1] Main Q attends to the selected main KV plus the layer-local
// SWA KV; [digest 已确认] the selected entries are concatenated with the windowed
// KV; [reading §4.2] every layer has its own query and window.  Readings: K = V =
// the whole dequantised entry, shared by all query heads; one softmax over all
// keys; window tokens are E4M3 values times swa_scale.
//
// Work split: a workgroup owns one query row and 64 heads, in eight waves, two per
// SIMD.  Wave w = (head tile w%4, half h = w/4) owns heads 16(w%4) .. +15 and the
// dims [hD/2, (h+1)D/2): it holds its heads' query over those dims, computes the
// partial S^T of a chunk's 32 keys over them and swaps the partial tiles with its
// partner (the other half of the head tile) through LDS; both then hold the same
// logits, run the same softmax (bitwise equal) and accumulate O for their own
// half of the output dims, so no partial outputs are merged.
// The row's keys pass in 32-key chunks (selected entries first, then window
// tokens), each decoded once, exactly to fp16, into a key-major LDS buffer by all
// 512 threads.  Three buffers and one barrier per step: step c decodes chunk c+2,
// forms the partial logits of chunk c+1 and finishes chunk c.
//   * S^T = K·Q^T on MFMA 16x16x32 f16: two 16-key tiles; A = keys read from LDS
//     (16 bytes per lane), B = the wave's fp16 query half in registers;
//   * lazy online softmax in the S^T layout (lane = one head, 8 keys);
//   * O += P·V on MFMA 16x16x32 f16 over the wave's D/32 output tiles: the 8
//     probabilities a lane holds (4 keys of each tile) are exactly its A operand,
//     and V comes from the same LDS rows through two transposing reads
//     (ds_read_b64_tr_b16), one per key tile.
// LDS layout of a chunk: key r at byte r(2D+32) + 16[r >= 16].  A 16-byte LDS
// access by a wave is served per 32-lane half and is conflict-free when each half
// hits distinct 4-byte banks out of 128 (measured): with a row stride of 32 mod 512
// bytes the K reads (16 keys x two 16-byte columns per half) are, the transposing
// V reads (8 keys x 32 bytes per half) are, and the 16-byte shift of the second
// tile keeps the decode writes (32 keys, one column) apart as well.
// The bf16 query is moved into fp16 exactly by a power of two per head (the
// head's largest |q| lands in [2^14, 2^15)), which is undone on the logits.
// Probabilities are rounded to fp16 once and the row sums add the rounded values.
#include "attn_common.h"

namespace csa2 {
namespace {

typedef _Float16 w8_t __attribute__((ext_vector_type(8)));
typedef _Float16 w4_t __attribute__((ext_vector_type(4)));
typedef _Float16 w2_t __attribute__((ext_vector_type(2)));
typedef float wf4_t __attribute__((ext_vector_type(4)));
typedef short ws4_t __attribute__((ext_vector_type(4)));
typedef uint32_t wu4_t __attribute__((ext_vector_type(4)));

constexpr int kWideThreads = 512;  // eight waves: 4 head tiles x 2 key halves
constexpr int kWideHeads = 64;     // heads per workgroup, 16 per wave
constexpr int kWideMaxSel = 512;   // selection slots the kernel takes (staged in LDS)
constexpr int kPrefK = 6;          // K reads issued ahead of their MFMA
constexpr int kPrefV = 4;          // V read pairs issued ahead of their MFMA

// D(16x16, f32) += A(16x32, f16) * B(32x16, f16); lane l holds A row l%16 / B
// column l%16 with reduction elements 8(l/16) .. +7, and D rows 4(l/16)+i,
// column l%16 in element i.
CSA2_DEV wf4_t mfma16x16x32_f16(w8_t a, w8_t b, wf4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 8 bytes per lane from LDS, transposed inside each 16-lane group: lane j of the
// group receives element j%4 of what lanes 4e + j/4 (e = 0..3) addressed.
CSA2_DEV w4_t lds_read_tr(const uint8_t* p) {
  typedef __attribute__((address_space(3))) ws4_t lds_s4;
  return __builtin_bit_cast(w4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p)));
}
// exact conversions: the two E2M1 codes of byte SEL (low nibble first); two E4M3
// bytes (low or high half of the word)
template <int SEL>
CSA2_DEV w2_t e2m1_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
template <bool HI>
CSA2_DEV w2_t e4m3_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

template <int D>
__global__ __launch_bounds__(kWideThreads, 1) void sparse_attn_wide_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int rows, int head_groups,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int NS = D / 64;                   // S^T MFMA steps per tile (half the dims)
  constexpr int NO = D / 32;                   // output tiles of 16 dims in the wave's half
  constexpr int KSTB = 2 * D + 32;             // bytes per key row in LDS (second tile + 16)
  constexpr int KBUF = kKC * KSTB + 16;        // bytes per chunk buffer
  constexpr int VPT = kKC * D / kWideThreads;  // values each thread decodes per chunk
  constexpr int NU = VPT / 8;                  // 16-byte LDS units each thread writes
  constexpr int NCL = VPT >= 32 ? VPT / 32 : 1;  // 16-byte code loads of a selected entry
  constexpr int NSB = VPT / 16;                // its E4M3 block scales
  constexpr int NWL = VPT / 16;                // 16-byte loads of a window token
  constexpr int NLD = NCL + 1 > NWL ? NCL + 1 : NWL;
  static_assert((VPT == 16 || VPT == 32) && KSTB % 512 == 32, "decode split");
  // LDS: three chunk buffers, the exchanged partial tiles (parity, head tile, half,
  // key tile: 64 lanes x 16 bytes each)
  constexpr int KV_BYTES = 3 * KBUF;
  __shared__ __attribute__((aligned(16))) uint8_t kv[KV_BYTES];
  __shared__ __attribute__((aligned(16))) wf4_t xch[2][4][2][2][64];
  __shared__ int s_ent[kWideMaxSel];

  int row, hgrp;
  if (!xcd_map(blockIdx.x, rows, head_groups, row, hgrp)) return;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ht = wave & 3, kh = wave >> 2;  // head tile; half of the dims
  const int hc = lane & 15, g = lane >> 4;  // MFMA row / column and lane group
  const int head0 = hgrp * kWideHeads + ht * 16;

  // selection slots (ascending, -1 padded) rounded up to whole chunks; slots that
  // are not a valid entry are masked
  const int* srow = sel + (size_t)row * K;
  const int n_sel = N > 0 ? K : 0;
  const int nm = (n_sel + kKC - 1) / kKC;
  for (int i = tid; i < nm * kKC; i += kWideThreads) {
    const int v = i < n_sel ? srow[i] : -1;
    s_ent[i] = (v >= 0 && v < N) ? v : -1;
  }
  const WinRange win = window_of(q_pos, row, S, swa_pos0, n_win);
  const int n_swa = win.n;
  const int n_chunks = nm + (n_swa + kKC - 1) / kKC;
  __syncthreads();

  // ---- raw bytes of a chunk: thread = (key dkey, dims [dseg*VPT, +VPT)); both
  // kinds arrive through the same NLD 16-byte loads into the same registers
  const int dkey = tid & 31, dseg = tid >> 5;
  wu4_t raw[NLD];
  // raw buffers over this row's sequence (32-bit offsets; the launch checks the
  // extents fit)
  const __amdgpu_buffer_rsrc_t r_codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes) + (size_t)b * N * (D / 2), (short)0, N * (D / 2), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t r_scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(scales) + (size_t)b * N * (D / 16), (short)0, N * (D / 16), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t r_swa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(swa) + (size_t)b * S * D, (short)0, S * D, kRawBufferWord3);
  auto load_raw = [&](int c) {
    const bool mc = c < nm;
    const int e = mc ? max(s_ent[c * kKC + dkey], 0) : 0;  // padding reads entry 0, masked later
    const int t = (c - nm) * kKC + dkey;
    const int wo = window_slot(win, t >= 0 && t < n_swa ? t : 0, S) * D + dseg * VPT;
    const int co = e * (D / 2) + ((dseg * (VPT / 2)) & ~15);
    const int so = e * (D / 16) + ((dseg * NSB) & ~15);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const __amdgpu_buffer_rsrc_t r = mc ? (i < NCL ? r_codes : r_scales) : r_swa;
      const int off = mc ? (i < NCL ? co + 16 * i : so) : (i < NWL ? wo + 16 * i : wo);
      raw[i] = __builtin_bit_cast(wu4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
  };
  // ---- decode the raw registers into one LDS buffer (exact fp16)
  auto decode = [&](uint8_t* buf, bool main_chunk) {
    uint8_t* rp = buf + dkey * KSTB + (dkey & 16) + dseg * (2 * VPT);
    if (main_chunk) {
      const int so = (dseg * NSB) & 15;  // this thread's scale bytes inside the 16-byte block
      const wu4_t sv = raw[NCL];
      const uint32_t sw = ((so >> 2) == 0 ? sv[0] : (so >> 2) == 1 ? sv[1] : (so >> 2) == 2 ? sv[2] : sv[3]) >>
                          (8 * (so & 3));
      const w2_t s01 = e4m3_pair<false>(sw);
      const w2_t mm[2] = {w2_t{s01[0], s01[0]}, w2_t{s01[1], s01[1]}};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        // codes of dims 8u .. 8u+7 of the range (VPT = 16: half dseg%2 of the block)
        const uint32_t w = VPT >= 32 ? raw[u / 4][u % 4] : raw[0][2 * (dseg & 1) + u];
        const w2_t sc = mm[u / 2];  // their block scale
        const wu4_t pk = {__builtin_bit_cast(uint32_t, e2m1_pair<0>(w) * sc),
                          __builtin_bit_cast(uint32_t, e2m1_pair<1>(w) * sc),
                          __builtin_bit_cast(uint32_t, e2m1_pair<2>(w) * sc),
                          __builtin_bit_cast(uint32_t, e2m1_pair<3>(w) * sc)};
        *reinterpret_cast<wu4_t*>(rp + 16 * u) = pk;
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t w0 = raw[u / 2][2 * (u % 2)], w1 = raw[u / 2][2 * (u % 2) + 1];
        const wu4_t pk = {__builtin_bit_cast(uint32_t, e4m3_pair<false>(w0)),
                          __builtin_bit_cast(uint32_t, e4m3_pair<true>(w0)),
                          __builtin_bit_cast(uint32_t, e4m3_pair<false>(w1)),
                          __builtin_bit_cast(uint32_t, e4m3_pair<true>(w1))};
        *reinterpret_cast<wu4_t*>(rp + 16 * u) = pk;
      }
    }
  };
  // chunk c sits in buffer c mod 3; the three buffer addresses rotate each step (a
  // plain base per step lets every read take its offset as an immediate)
  uint8_t* buf_c = kv;                       // chunk c
  uint8_t* buf_n = kv + KBUF;                // chunk c+1
  uint8_t* buf_d = kv + 2 * KBUF;            // chunk c+2 (being decoded)

  if (n_chunks > 0) load_raw(0);

  // ---- the wave's query half (B operand of S^T): lane (head hc, group g) holds
  // dims D/2*kh + 32s + 8g .. +7, moved into fp16 by the head's power of two (from
  // the head's largest |q| over all dims, so both halves use the same one)
  w8_t qh[NS];
  float qs;  // logits of head hc = S^T * qs
  {
    const uint16_t* qr = q + ((size_t)row * H_q + head0 + hc) * D + 8 * g;
    float mx = 0.0f;
    wu4_t mineq[NS];
#pragma unroll
    for (int s = 0; s < 2 * NS; ++s) {
      const wu4_t r = *reinterpret_cast<const wu4_t*>(qr + 32 * s);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mx = fmaxf(mx, fabsf(__uint_as_float(r[k] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(r[k] & 0xFFFF0000u)));
      }
      if (s / NS == kh) mineq[s % NS] = r;
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    int e = 0;  // the head's largest |q| x 2^-e lands in [2^14, 2^15)
    if (mx > 0.0f) e = min(126, max(-126, (int)((__float_as_uint(mx) >> 23) & 255u) - 127 - 14));
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    qs = __uint_as_float((uint32_t)(127 + e) << 23);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qh[s][2 * k] = (_Float16)(__uint_as_float(mineq[s][k] << 16) * inv);
        qh[s][2 * k + 1] = (_Float16)(__uint_as_float(mineq[s][k] & 0xFFFF0000u) * inv);
      }
    }
  }

  // S^T A operand: MFMA row hc of tile t = key 16t + hc, dims D/2*kh + 32s + 8g
  const int qk_off = hc * KSTB + kh * D + 16 * g;
  constexpr int T1 = 16 * KSTB + 16;  // offset of key tile 1
  // partial S^T of chunk c's two tiles over this wave's dims, published for the partner
  auto partial = [&](const uint8_t* buf, int c, wf4_t (&pt)[2]) {
    const uint8_t* kb = buf + qk_off;
    pt[0] = pt[1] = wf4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const w8_t ka = *reinterpret_cast<const w8_t*>(kb + t * T1 + 64 * s);
        pt[t] = mfma16x16x32_f16(ka, qh[s], pt[t]);
      }
    }
    // schedule: the first reads well ahead, then one read per MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, kPrefK, 0);
#pragma unroll
    for (int k = 0; k < 2 * NS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (k + kPrefK < 2 * NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    xch[c & 1][ht][kh][0][lane] = pt[0];
    xch[c & 1][ht][kh][1][lane] = pt[1];
  };

  // ---- prologue: chunks 0 and 1 decoded, chunk 2 in flight, partials of chunk 0
  // published
  wf4_t mine[2] = {wf4_t{0.f, 0.f, 0.f, 0.f}, wf4_t{0.f, 0.f, 0.f, 0.f}};
  if (n_chunks > 0) {
    decode(buf_c, 0 < nm);
    if (1 < n_chunks) {
      load_raw(1);
      decode(buf_n, 1 < nm);
      if (2 < n_chunks) load_raw(2);
    }
    lds_barrier();
    partial(buf_c, 0, mine);
  }
  lds_barrier();

  wf4_t o[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = wf4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.0f;
  const float log2_swa = log2f(swa_scale), inv_swa = 1.0f / swa_scale;  // swa_scale > 0 here
  // transposing V read of tile t: lane 4e + q of group g addresses key 16t + 4g + e,
  // dims D/2*kh + 16n + 4q .. +3; it receives dim D/2*kh + 16n + hc of the keys of
  // S^T rows 4g .. 4g+3 (its P elements)
  const int pv_off = (4 * g + ((lane & 15) >> 2)) * KSTB + kh * D + 8 * (lane & 3);

  for (int c = 0; c < n_chunks; ++c) {
    const bool main_chunk = c < nm;
    // ---- logits of chunk c: the two halves' partial tiles added in dim order
    wf4_t st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const wf4_t other = xch[c & 1][ht][kh ^ 1][t][lane];
      st[t] = kh ? other + mine[t] : mine[t] + other;
    }
    // ---- partial logits of chunk c+1 (decoded in step c-1)
    if (c + 1 < n_chunks) partial(buf_n, c + 1, mine);
    // ---- validity of the chunk's 32 keys (bit r = key r)
    const int kr = lane & 31;
    const bool ok = main_chunk ? s_ent[c * kKC + kr] >= 0 : (c - nm) * kKC + kr < n_swa;
    const uint32_t vmask = (uint32_t)__ballot(ok);
    const float ks = main_chunk ? 1.0f : swa_scale;
    const float fs = ks * sm_log2 * qs;
    float lg[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = st[t][i] * fs;
        // the logit is rounded on its own (as the reference maximum is), so the
        // lazy bound below holds for the value exponentiated
        asm("" : "+v"(x));
        lg[4 * t + i] = x;
      }
    }
    if (vmask != 0xFFFFFFFFu) {  // a chunk with masked keys (most have none)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((vmask >> (16 * t + 4 * g + i)) & 1u)) lg[4 * t + i] = -INFINITY;
    }
    float lmax = lg[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) lmax = fmaxf(lmax, lg[k]);
    // Lazy reference maximum: it moves only when a logit exceeds it by more than
    // 2^kLazy; the head's four lanes then agree on the new value.
    const bool up_lane = lmax > m_ref + kLazy || (m_ref == -INFINITY && lmax != -INFINITY);
    if (__ballot(up_lane)) {
      float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const bool up = cmax > m_ref + kLazy || (m_ref == -INFINITY && cmax != -INFINITY);
      const float alpha = up ? (m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - cmax)) : 1.0f;
      m_ref = up ? cmax : m_ref;
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int n = 0; n < NO; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= al[i];
      }
    }
    // P times the key scale, in fp16: p * ks = exp2(lg - (m_ref - log2 ks)); the row
    // sum gains the rounded values divided by ks.  While no key has been seen
    // (m_ref = -inf) every lg is -inf and p = 0.
    const float mp = m_ref == -INFINITY ? 0.0f : m_ref - (main_chunk ? 0.0f : log2_swa);
    w8_t pa;  // A operand of P·V: reduction slots 8g .. 8g+7 = keys 4g .. 4g+3 of each tile
#pragma unroll
    for (int k = 0; k < 8; ++k) pa[k] = (_Float16)__builtin_amdgcn_exp2f(lg[k] - mp);
    // the row sum adds the rounded probabilities (exact products in the dot)
    float psum = 0.0f;
    const w2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 0, 1), one2, psum, false);
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 2, 3), one2, psum, false);
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 4, 5), one2, psum, false);
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 6, 7), one2, psum, false);
    l_run += main_chunk ? psum : psum * inv_swa;
    // ---- O += P·V over the wave's output tiles: one 16x16x32 MFMA per tile over
    // both key tiles (a 16x16x16 MFMA occupies the matrix unit as long as a
    // 16x16x32 one, so the wider reduction halves the matrix time)
    {
      const uint8_t* vb = buf_c + pv_off;
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        const w4_t lo = lds_read_tr(vb + 32 * n);
        const w4_t hi = lds_read_tr(vb + T1 + 32 * n);
        o[n] = mfma16x16x32_f16(pa, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), o[n]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPrefV, 0);
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (n + kPrefV < NO) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    // ---- decode chunk c+2 into the buffer chunk c-1 used (last read in step c-1),
    // load chunk c+3
    if (c + 2 < n_chunks) {
      decode(buf_d, c + 2 < nm);
      if (c + 3 < n_chunks) load_raw(c + 3);
    }
    uint8_t* const t = buf_c;
    buf_c = buf_n;
    buf_n = buf_d;
    buf_d = t;
    lds_barrier();
  }

  // ---- epilogue: O element i of lane l is head 4g + i, dim D/2*kh + 16n + hc
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float rl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = __shfl(l_tot, 4 * g + i);
    rl[i] = v > 0.0f ? 1.0f / v : 0.0f;
  }
  float* orow = out + ((size_t)row * H_q + head0) * D + kh * (D / 2) + hc;
#pragma unroll
  for (int n = 0; n < NO; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) orow[(size_t)(4 * g + i) * D + 16 * n] = o[n][i] * rl[i];
  }
  if (lse != nullptr && kh == 0 && g == 0)
    lse[(size_t)row * H_q + head0 + hc] =
        l_tot > 0.0f ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

bool attn_wide_supported(int H_q, int d, int K, int N, int S, float swa_scale) {
  // a sequence's codes and window must be addressable by 32-bit buffer offsets
  return H_q % kWideHeads == 0 && (d == 256 || d == 512) && K <= kWideMaxSel && swa_scale > 0.0f &&
         swa_scale <= 128.0f && (long long)N * (d / 2) < (1ll << 31) && (long long)S * d < (1ll << 31);
}

hipError_t launch_sparse_attn_wide(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                   int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                   int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                   int H_q, int d, float sm_log2, int rows, float* out, float* lse,
                                   hipStream_t st) {
  const int head_groups = H_q / kWideHeads;
  dim3 grid(xcd_grid(rows, head_groups));
  if (d == 512)
    hipLaunchKernelGGL((sparse_attn_wide_kernel<512>), grid, dim3(kWideThreads), 0, st, q, codes, scales,
                       N, sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq, H_q, sm_log2, rows,
                       head_groups, out, lse);
  else
    hipLaunchKernelGGL((sparse_attn_wide_kernel<256>), grid, dim3(kWideThreads), 0, st, q, codes, scales,
                       N, sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq, H_q, sm_log2, rows,
                       head_groups, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
