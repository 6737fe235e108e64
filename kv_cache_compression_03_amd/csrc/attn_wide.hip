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
// Work split: a workgroup owns one query row and 64 heads in four waves; two
// workgroups share a CU (one wave of each per SIMD, so their barriers and phases
// are independent).  Wave w owns heads 16w .. 16w+15 over all D dims: its query
// (B operand of S^T, fp16) and its output accumulators stay in registers, so no
// partial logits are exchanged and every softmax is computed once.
// The row's keys pass in 32-key chunks (selected entries first, then window
// tokens), each decoded once, exactly to fp16, into a key-major LDS buffer.  Two
// buffers and one barrier per step: step c attends chunk c while chunk c+1 is
// decoded into the other buffer.  Raw chunk bytes never occupy registers across a
// step: wave w stages the bytes of keys 8w .. 8w+7 (one half of the dims at a
// time) through its own 2 KB of LDS with 16-byte loads that write LDS directly,
// and decodes what it staged, so no other wave touches its staging.  The first
// half of chunk c+1 is decoded between the softmax and P·V of chunk c (loaded at
// the end of step c-1), the second half after P·V (loaded before it).
//   * S^T = K·Q^T on MFMA 16x16x32 f16: two 16-key tiles; A = keys read from LDS
//     (16 bytes per lane), B = the wave's fp16 query in registers;
//   * lazy online softmax in the S^T layout (lane = one head, 8 keys);
//   * O += P·V on MFMA 16x16x32 f16 over the D/16 output tiles: the 8
//     probabilities a lane holds (4 keys of each tile) are exactly its A operand,
//     and V comes from the same LDS rows through two transposing reads
//     (ds_read_b64_tr_b16), one per key tile.
// LDS layout of a chunk: key r at byte r(2D+32) + 16[r >= 16].  A 16-byte LDS
// access by a wave is served per 32-lane half and is conflict-free when each half
// hits distinct 4-byte banks out of 128 (measured): with a row stride of 32 mod 512
// bytes the K reads (16 keys x two 16-byte columns per half) are, and so are the
// transposing V reads (8 keys x 32 bytes per half).
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

constexpr int kWideThreads = 256;  // four waves of 16 heads
constexpr int kWideHeads = 64;     // heads per workgroup, 16 per wave
constexpr int kWideMaxSel = 512;   // selection slots the kernel takes (held in LDS)
constexpr int kPrefK = 6;          // K reads issued ahead of their MFMA
constexpr int kPrefV = 4;          // V read pairs issued ahead of their MFMA
constexpr int kStageBytes = 3072;  // LDS staging of raw chunk bytes per wave

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

// a value the compiler must treat as unknown where it is used (keeps lane-derived
// values from being hoisted out of the loop into registers that stay live)
CSA2_DEV int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The kernel body takes its LDS arrays as restrict pointers: the compiler then knows
// that the chunk buffers never alias the staging that 16-byte loads write straight
// into LDS, and waits for those loads only where the staged bytes are read.
template <int D>
__device__ __attribute__((always_inline)) void sparse_attn_wide_body(
    uint8_t* __restrict__ kv, uint8_t* __restrict__ stg_all, int* __restrict__ s_ent,
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int rows, int head_groups,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int NS = D / 32;                   // S^T MFMA steps per key tile (all dims)
  constexpr int NO = D / 16;                   // output tiles of 16 dims
  constexpr int KSTB = 2 * D + 32;             // bytes per key row in LDS (second tile + 16)
  constexpr int KBUF = kKC * KSTB;             // bytes per chunk buffer (row 31's shift fits its padding)
  static_assert(KSTB % 512 == 32, "LDS row stride");

  int row, hgrp;
  if (!xcd_map(blockIdx.x, rows, head_groups, row, hgrp)) return;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hc = lane & 15, g = lane >> 4;  // MFMA row / column and lane group
  const int head0 = hgrp * kWideHeads + wave * 16;

  // selection slots (ascending, -1 padded) rounded up to whole chunks, held as the
  // byte offset of the entry's codes (its scales sit at an eighth of it); slots
  // that are not a valid entry are -1 and masked
  const int* srow = sel + (size_t)row * K;
  const int n_sel = N > 0 ? K : 0;
  const int nm = (n_sel + kKC - 1) / kKC;
  for (int i = tid; i < nm * kKC; i += kWideThreads) {
    const int v = i < n_sel ? srow[i] : -1;
    s_ent[i] = (v >= 0 && v < N) ? v * (D / 2) : -1;
  }
  const WinRange win = window_of(q_pos, row, S, swa_pos0, n_win);
  const int n_swa = win.n;
  const int n_chunks = nm + (n_swa + kKC - 1) / kKC;
  __syncthreads();

  // ---- chunk bytes are staged per wave: wave w loads and decodes keys 8w .. 8w+7
  // of every chunk through its own 3 KB of LDS (16-byte loads that write LDS
  // directly: lane l's bytes land at base + 16 l).  A chunk of selected entries is
  // staged whole (codes of key k at k D/2, its block scales at 4 D + k D/16); a
  // window chunk one half of the dims at a time (key k's bytes at k D/2).
  constexpr int CUK = D / 32;  // 16-byte code units per key
  constexpr int SUK = D / 256; // 16-byte scale units per key
  constexpr int WU = D / 32;   // 16-byte window units per key and half
  constexpr int VPL = D / 16;  // values each lane decodes per half
  constexpr int SOFF = 4 * D;  // staged scales after the wave's 8 keys of codes
  constexpr int NCI = 8 * CUK / 64;        // load instructions of a chunk's codes
  constexpr int NWI = (8 * WU + 63) / 64;  // load instructions of a window half
  static_assert(8 * CUK % 64 == 0 && 8 * SUK <= 64 && SOFF + 8 * 16 * SUK <= kStageBytes &&
                    16 * 8 * WU <= kStageBytes, "staging split");
  uint8_t* const my_stg = stg_all + kStageBytes * wave;
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  // raw buffers over this row's sequence (32-bit offsets; the launch checks the
  // extents fit)
  const __amdgpu_buffer_rsrc_t r_codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes) + (size_t)b * N * (D / 2), (short)0, N * (D / 2), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t r_scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(scales) + (size_t)b * N * (D / 16), (short)0, N * (D / 16), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t r_swa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(swa) + (size_t)b * S * D, (short)0, S * D, kRawBufferWord3);
  // the loads of a whole chunk of selected entries (padding slots read entry 0,
  // masked later)
  auto stage_main = [&](int c) {
    const int ln = opaque(lane);
#pragma unroll
    for (int i = 0; i < NCI; ++i) {
      const int u = 64 * i + ln;
      const int eo = max(s_ent[c * kKC + 8 * wave + u / CUK], 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_codes, (lds_ptr_t)(my_stg + 1024 * i), 16,
                                               eo + 16 * (u % CUK), 0, 0, 0);
    }
    if (ln < 8 * SUK) {
      const int eo = max(s_ent[c * kKC + 8 * wave + ln / SUK], 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_scales, (lds_ptr_t)(my_stg + SOFF), 16,
                                               (eo >> 3) + 16 * (ln % SUK), 0, 0, 0);
    }
  };
  // the loads of half h of a window chunk (padding slots read the first visible
  // token, masked later)
  auto stage_win = [&](int c, int h) {
    const int ln = opaque(lane);
#pragma unroll
    for (int i = 0; i < NWI; ++i) {
      const int u = 64 * i + ln, k = u / WU;
      const int t = (c - nm) * kKC + 8 * wave + k;
      const int slot = window_slot(win, t < n_swa ? t : 0, S);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_swa, (lds_ptr_t)(my_stg + 1024 * i), 16,
                                               slot * D + (D / 2) * h + 16 * (u % WU), 0, 0, 0);
    }
  };
  // what is staged a step ahead of its decode: a whole chunk of entries, or the
  // first half of a window chunk
  auto stage_first = [&](int c) {
    if (c < nm) stage_main(c);
    else stage_win(c, 0);
  };
  // the wave's staged loads have landed in LDS / its staging reads have returned
  auto wait_staged = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  auto wait_lds = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  // ---- decode half h of the staged chunk into an LDS buffer (exact fp16): lane =
  // (key k = l % 8, dims D/2 h + VPL (l / 8) .. +VPL-1)
  auto decode_half = [&](uint8_t* buf, bool main_chunk, int h) {
    const int ln = opaque(lane), k = ln & 7, seg = ln >> 3;
    const int r = 8 * wave + k;
    uint8_t* rp = buf + r * KSTB + (r & 16) + (D / 2 * h + VPL * seg) * 2;
    if (main_chunk) {
      uint32_t cw[VPL / 8];  // 8 codes per word
      const uint8_t* cp = my_stg + k * (D / 2) + (D / 4) * h + (VPL / 2) * seg;
      if constexpr (VPL == 32) {
        const wu4_t v = *reinterpret_cast<const wu4_t*>(cp);
        cw[0] = v[0]; cw[1] = v[1]; cw[2] = v[2]; cw[3] = v[3];
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(cp);
        cw[0] = v.x; cw[1] = v.y;
      }
      const uint8_t* sp = my_stg + SOFF + k * (D / 16) + (D / 32) * h + (VPL / 16) * seg;
      const uint32_t sw = VPL == 32 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sp) : (uint32_t)*sp;
      const w2_t s01 = e4m3_pair<false>(sw);
      const w2_t mm[2] = {w2_t{s01[0], s01[0]}, w2_t{s01[1], s01[1]}};
#pragma unroll
      for (int u = 0; u < VPL / 8; ++u) {
        const uint32_t w = cw[u];
        const w2_t sc = mm[u / 2];  // dims 8u .. 8u+7 share the block scale u/2
        const wu4_t pk = {__builtin_bit_cast(uint32_t, e2m1_pair<0>(w) * sc),
                          __builtin_bit_cast(uint32_t, e2m1_pair<1>(w) * sc),
                          __builtin_bit_cast(uint32_t, e2m1_pair<2>(w) * sc),
                          __builtin_bit_cast(uint32_t, e2m1_pair<3>(w) * sc)};
        *reinterpret_cast<wu4_t*>(rp + 16 * u) = pk;
      }
    } else {
      const uint8_t* wp = my_stg + 16 * WU * k + VPL * seg;
#pragma unroll
      for (int j = 0; j < VPL / 16; ++j) {
        const wu4_t v = *reinterpret_cast<const wu4_t*>(wp + 16 * j);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t w0 = v[2 * q], w1 = v[2 * q + 1];
          const wu4_t pk = {__builtin_bit_cast(uint32_t, e4m3_pair<false>(w0)),
                            __builtin_bit_cast(uint32_t, e4m3_pair<true>(w0)),
                            __builtin_bit_cast(uint32_t, e4m3_pair<false>(w1)),
                            __builtin_bit_cast(uint32_t, e4m3_pair<true>(w1))};
          *reinterpret_cast<wu4_t*>(rp + 32 * j + 16 * q) = pk;
        }
      }
    }
  };
  // chunk c sits in buffer c mod 2; the two buffer addresses swap each step (a
  // plain base per step lets every read take its offset as an immediate)
  uint8_t* buf_c = kv;         // chunk c (attended)
  uint8_t* buf_n = kv + KBUF;  // chunk c+1 (being decoded)

  // ---- the wave's query (B operand of S^T): lane (head hc, group g) holds dims
  // 32s + 8g .. +7, moved into fp16 by the head's power of two
  w8_t qh[NS];
  float qs;  // logits of head hc = S^T * qs
  {
    const uint16_t* qr = q + ((size_t)row * H_q + head0 + hc) * D + 8 * g;
    float mx = 0.0f;
    wu4_t qr4[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qr4[s] = *reinterpret_cast<const wu4_t*>(qr + 32 * s);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mx = fmaxf(mx, fabsf(__uint_as_float(qr4[s][k] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(qr4[s][k] & 0xFFFF0000u)));
      }
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
        qh[s][2 * k] = (_Float16)(__uint_as_float(qr4[s][k] << 16) * inv);
        qh[s][2 * k + 1] = (_Float16)(__uint_as_float(qr4[s][k] & 0xFFFF0000u) * inv);
      }
    }
  }

  // ---- prologue: chunk 0 decoded, chunk 1 (or its first half) in flight
  if (n_chunks > 0) {
    stage_first(0);
    wait_staged();
    decode_half(buf_c, 0 < nm, 0);
    if (0 >= nm) {
      wait_lds();
      stage_win(0, 1);
      wait_staged();
    }
    decode_half(buf_c, 0 < nm, 1);
    if (1 < n_chunks) {
      wait_lds();
      stage_first(1);
    }
  }
  lds_barrier();

  // S^T A operand: MFMA row hc of tile t = key 16t + hc, dims 32s + 8g .. +7
  const int qk_off = hc * KSTB + 16 * g;
  constexpr int T1 = 16 * KSTB + 16;  // offset of key tile 1
  // transposing V read of tile t: lane 4e + q of group g addresses key 16t + 4g + e,
  // dims 16n + 4q .. +3; it receives dim 16n + hc of the keys of S^T rows
  // 4g .. 4g+3 (its P elements)
  const int pv_off = (4 * g + ((lane & 15) >> 2)) * KSTB + 8 * (lane & 3);

  wf4_t o[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = wf4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.0f;
  const float log2_swa = log2f(swa_scale), inv_swa = 1.0f / swa_scale;  // swa_scale > 0 here

  for (int c = 0; c < n_chunks; ++c) {
    const bool main_chunk = c < nm;
    // ---- S^T of chunk c over all dims: two 16-key tiles
    wf4_t st[2] = {wf4_t{0.f, 0.f, 0.f, 0.f}, wf4_t{0.f, 0.f, 0.f, 0.f}};
    {
      const uint8_t* kb = buf_c + qk_off;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const w8_t ka = *reinterpret_cast<const w8_t*>(kb + t * T1 + 64 * s);
          st[t] = mfma16x16x32_f16(ka, qh[s], st[t]);
        }
      }
      // schedule: the first reads well ahead, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, kPrefK, 0);
#pragma unroll
      for (int k = 0; k < 2 * NS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k + kPrefK < 2 * NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // ---- validity of the chunk's 32 keys (bit r = key r)
    const int kr = opaque(lane) & 31;
    const bool ok = main_chunk ? s_ent[c * kKC + kr] >= 0 : (c - nm) * kKC + kr < n_swa;
    const uint32_t vmask = (uint32_t)__ballot(ok);
    const float ks = main_chunk ? 1.0f : swa_scale;
    const float fs = ks * sm_log2 * qs;  // > 0: base-2 logit = S^T * fs
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * t + i] = st[t][i];
    if (vmask != 0xFFFFFFFFu) {  // a chunk with masked keys (most have none)
      // lane-derived values are formed here, not kept in registers over the loop
      const uint32_t vm = vmask >> opaque(4 * g);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((vm >> (16 * t + i)) & 1u)) sv[4 * t + i] = -INFINITY;
    }
    // the largest logit of the lane: the scale is positive, so it is the scaled
    // largest S^T value
    float smax = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) smax = fmaxf(smax, sv[k]);
    const float lmax = smax * fs;
    // Lazy reference maximum: it moves only when a logit exceeds it by more than
    // 2^kLazy; the head's four lanes then agree on the new value.
    const bool up_lane = lmax > m_ref + kLazy || (m_ref == -INFINITY && lmax != -INFINITY);
    if (__ballot(up_lane)) {
      const int ln = opaque(lane);  // shuffle addresses are formed here (rarely taken)
      float cmax = fmaxf(lmax, __shfl(lmax, ln ^ 16));
      cmax = fmaxf(cmax, __shfl(cmax, ln ^ 32));
      const bool up = cmax > m_ref + kLazy || (m_ref == -INFINITY && cmax != -INFINITY);
      const float alpha = up ? (m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - cmax)) : 1.0f;
      m_ref = up ? cmax : m_ref;
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * (ln >> 4) + i);
#pragma unroll
      for (int n = 0; n < NO; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= al[i];
      }
    }
    // P times the key scale, in fp16: p * ks = exp2(lg - (m_ref - log2 ks)); the row
    // sum gains the rounded values divided by ks.  While no key has been seen
    // (m_ref = -inf) every lg is -inf and p = 0.
    // The exponent is formed in one rounding (S^T * fs - mp); it stays within a few
    // units in the last place of the rounded logit minus mp, so p < 2^kLazy (1 + tiny).
    const float mp = m_ref == -INFINITY ? 0.0f : m_ref - (main_chunk ? 0.0f : log2_swa);
    w8_t pa;  // A operand of P·V: reduction slots 8g .. 8g+7 = keys 4g .. 4g+3 of each tile
#pragma unroll
    for (int k = 0; k < 8; ++k) pa[k] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sv[k], fs, -mp));
    // the row sum adds the rounded probabilities (exact products in the dot)
    float psum = 0.0f;
    const w2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 0, 1), one2, psum, false);
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 2, 3), one2, psum, false);
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 4, 5), one2, psum, false);
    psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 6, 7), one2, psum, false);
    l_run += main_chunk ? psum : psum * inv_swa;
    // ---- a window chunk c+1: decode its first half, stage the second
    if (c + 1 < n_chunks && c + 1 >= nm) {
      wait_staged();
      decode_half(buf_n, false, 0);
      wait_lds();
      stage_win(c + 1, 1);
    }
    // ---- O += P·V over the output tiles: one 16x16x32 MFMA per tile over both
    // key tiles (a 16x16x16 MFMA occupies the matrix unit as long as a 16x16x32
    // one, so the wider reduction halves the matrix time)
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
    // ---- the rest of chunk c+1 (its buffer was last read in step c-1): both
    // halves of a chunk of entries, the second half of a window chunk; then
    // chunk c+2 (or its first half) goes out
    if (c + 1 < n_chunks) {
      wait_staged();
      if (c + 1 < nm) decode_half(buf_n, true, 0);
      decode_half(buf_n, c + 1 < nm, 1);
      if (c + 2 < n_chunks) {
        wait_lds();
        stage_first(c + 2);
      }
    }
    uint8_t* const t = buf_c;
    buf_c = buf_n;
    buf_n = t;
    lds_barrier();
  }

  // ---- epilogue: O element i of lane l is head 4g + i, dim 16n + hc
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float rl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = __shfl(l_tot, 4 * g + i);
    rl[i] = v > 0.0f ? 1.0f / v : 0.0f;
  }
  // streaming (non-temporal) stores: the output is never read back here, and
  // keeping it out of the caches leaves them to the entries and window tokens the
  // other rows re-read (-3 % per layer measured)
  float* orow = out + ((size_t)row * H_q + head0) * D + hc;
#pragma unroll
  for (int n = 0; n < NO; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(o[n][i] * rl[i], &orow[(size_t)(4 * g + i) * D + 16 * n]);
  }
  if (lse != nullptr && g == 0)
    lse[(size_t)row * H_q + head0 + hc] =
        l_tot > 0.0f ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kWideThreads, 2) void sparse_attn_wide_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int rows, int head_groups,
    float* __restrict__ out, float* __restrict__ lse) {
  // LDS: two chunk buffers (the chunk being attended, the next being decoded), the
  // waves' staging of raw chunk bytes, the row's selection
  __shared__ __attribute__((aligned(16))) uint8_t kv[2 * kKC * (2 * D + 32)];
  __shared__ __attribute__((aligned(16))) uint8_t stg[kWideThreads / 64 * kStageBytes];
  __shared__ int s_ent[kWideMaxSel];
  sparse_attn_wide_body<D>(kv, stg, s_ent, q, codes, scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win,
                           q_pos, Tq, H_q, sm_log2, rows, head_groups, out, lse);
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
