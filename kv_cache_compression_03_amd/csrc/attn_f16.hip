// Sparse attention, fp16 MFMA kernel: main Q attends to (selected FP4 entries ++
// layer-local FP8 window).  Same function, same split plan and same partial
// results as the bf16 kernel in attn.hip, which remains for shapes this one does
// not take.
//
// [deep-dive §3.1] Main Q attends to the selected main KV plus the layer-local
// SWA KV; [digest 已确认] the selected entries are concatenated with the windowed
// KV; [reading §4.2] every layer has its own query and window.  Readings: K = V =
// the whole dequantised entry, shared by all query heads; one softmax over all
// keys; window tokens are E4M3 values times swa_scale.
//
// Why fp16.  An E2M1 value times its E4M3 block scale has at most 6 significant
// bits and lies in [2^-10, 2688]; an E4M3 value has at most 4 and lies in
// [2^-9, 448].  Both are exact fp16 numbers, so ONE fp16 copy of a chunk serves
// as K (for S = Q·K^T) and as V (for O += P·V): V fragments come straight out of
// the key-major copy through the transposing LDS read (ds_read_b64_tr_b16), and
// P is carried in fp16 (11 significant bits) by a single MFMA.  The bf16 query
// is moved into fp16 exactly by a power of two per head (from the head's largest
// |q|), which is undone on the logits.  Products are exact in both kernels and
// accumulate in fp32.
//
// Work split: a workgroup owns one query row, a contiguous range of 32-key
// chunks (split-K over the keys, merged by the combine kernel) and 32·HG2 heads.
// Its waves are (32-head group) x (quarter of the dims), MFMA 32x32x16 f16, so a
// wave holds 32 heads x D/4 dims of Q and of O (two waves fit per SIMD):
//   * S^T = K·Q^T: rows = the chunk's 32 keys, columns = the wave's 32 heads; a
//     wave reduces over its quarter of the dims and the four waves of a head
//     group add the partial logit tiles through LDS in one fixed order, so all
//     four hold bitwise identical logits;
//   * O += P·V: rows = heads, 32 dims per tile, 16 keys per MFMA.  In the S^T
//     output a lane holds one head's logits for 16 keys, which is directly the
//     P operand once the key order inside the reduction is matched in V.
// With 32 heads per wave every K and V byte in LDS is read by HG2 waves instead
// of one wave per 16 heads.  Chunks are double-buffered in LDS: while chunk c is
// multiplied, chunk c+1 (loaded into registers one chunk earlier) is decoded
// into the other buffer and chunk c+2 is loaded; two barriers per chunk.
#include "attn_common.h"

namespace csa2 {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// D(32x32, f32) += A(32x16, f16) * B(16x32, f16).  Lane l holds A row l%32 / B
// column l%32 with reduction elements 8*(l/32) .. +7, and D element i of lane l is
// row 8*(i/4) + 4*(l/32) + i%4, column l%32 (checked on the hardware).
CSA2_DEV f32x16_t mfma32x32x16_f16(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 bytes per lane from LDS, transposed inside each 16-lane group: lane j of the
// group receives element j%4 of what lanes 4e + j/4 (e = 0..3) addressed.
CSA2_DEV f16x4_t lds_read_tr(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// Exact conversions (checked exhaustively on the hardware): the two E2M1 codes of
// byte SEL (low nibble first) times pow2 = 2^E for E in [-9, 8]; two E4M3 bytes
// (low or high half of the word).
template <int SEL>
CSA2_DEV f16x2_t fp4x2_f16(uint32_t w, float pow2) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, SEL);
}
template <bool HI>
CSA2_DEV uint32_t fp8x2_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Key held by MFMA row m of a 32-key chunk: inside each 16-key half the 4x4
// grid (m/4, m%4) is transposed.  Any order works as long as K rows, the
// validity mask and the V slots agree; this one makes the four keys of each
// transposing V read sit 4 rows apart.
CSA2_DEV int key_of_row(int m) { return (m & 16) | ((m & 3) << 2) | ((m >> 2) & 3); }

template <int D, int HG2>
__global__ __launch_bounds__(HG2 * 256, 1) void sparse_attn_f16_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int chunks_per_split,
    int n_splits, int rows, int head_groups, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int DS = 4;              // dim quarters
  constexpr int NW = DS * HG2, NT = 64 * NW;
  constexpr int DH = D / DS;         // dims per wave
  constexpr int KSTB = 2 * D + 16;   // bytes per key row in LDS
  constexpr int VPT = kKC * D / NT;  // values each thread decodes per chunk
  constexpr int NU = VPT / 8;        // 16-byte LDS units each thread writes per chunk
  constexpr int NSB = VPT / 16;      // E4M3 block scales per thread
  static_assert(VPT >= 16 && VPT % 16 == 0 && NSB <= 4 && DH % 32 == 0, "decode split");
  // Key row k starts at k*KSTB bytes, i.e. in 16-byte bank slot k mod 16.  The
  // decode writes and the S^T operand reads touch one column of 16 keys per
  // instruction (16 distinct slots); with the row order of key_of_row() each
  // transposing V read touches 64 contiguous bytes of 4 keys whose slots are 4
  // apart.  No bank conflicts, and every per-step offset is a compile-time
  // immediate.  Three chunk buffers: chunk c is multiplied while c+1 is being
  // multiplied too (S^T) and c+2 is decoded.
  __shared__ __attribute__((aligned(16))) uint8_t kv[3][kKC * KSTB];
  __shared__ __attribute__((aligned(16))) float sx[NW * 4 * 64 * 4];     // partial logit tiles
  __shared__ __attribute__((aligned(16))) float sfin[HG2 * 4 * 64 * 4];  // summed tiles
  __shared__ int s_ent[kMaxSel];  // entry of each selection slot this split reads
  __shared__ float s_qmax[NW][32];  // per wave, largest |q| of each of its heads over its dims

  int row, split;
  if (!xcd_map(blockIdx.x, rows, n_splits * head_groups, row, split)) return;
  const int hgrp = split % head_groups;
  split /= head_groups;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane & 31, hh = lane >> 5;  // MFMA row/column and lane half
  const int head0 = (hgrp * HG2 + wave % HG2) * 32;
  const int dq = wave / HG2, dim0 = dq * DH;

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
  const int sl_lo = c_begin * kKC, sl_hi = min(c_end, nm) * kKC;
  for (int i = sl_lo + tid; i < sl_hi; i += NT) {
    const int v = i < n_sel ? srow[i] : -1;
    s_ent[i - sl_lo] = (v >= 0 && v < N) ? v : -1;
  }
  __syncthreads();

  // ---- raw bytes of a chunk: thread = (key dkey, dims [dseg*VPT, +VPT))
  const int dkey = tid & 31, dseg = tid >> 5;
  // Both kinds of chunk arrive through the same NLD 16-byte loads into the same
  // registers, with no branch: a selected entry as the aligned 16-byte blocks
  // holding this thread's VPT/2 code bytes plus the aligned 16-byte half of its
  // scale row holding this thread's NSB scale bytes, a window token as its VPT
  // bytes (slots past the data repeat a load).  With equal shapes the loads of
  // the chunk after next stay in flight across the loop.
  constexpr int NCL = VPT >= 32 ? VPT / 32 : 1;  // code loads
  constexpr int NLD = NCL + 1 > VPT / 16 ? NCL + 1 : VPT / 16;
  u32x4_t raw[NLD];
  auto load_raw = [&](u32x4_t (&raw)[NLD], int c) {
    const bool mc = c < nm;
    const int e = mc ? max(s_ent[c * kKC + dkey - sl_lo], 0) : 0;  // padding reads entry 0, masked later
    const size_t ent = (size_t)b * N + e;
    const uint8_t* cb = codes + ent * (D / 2) + ((dseg * (VPT / 2)) & ~15);
    const uint8_t* sb = scales + ent * (D / 16) + ((dseg * NSB) & ~15);
    const int t = (c - nm) * kKC + dkey;
    const uint8_t* wb = swa + ((size_t)b * S + window_slot(win, t >= 0 && t < n_swa ? t : 0, S)) * D + dseg * VPT;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const uint8_t* m = i < NCL ? cb + 16 * i : sb;
      const uint8_t* w = i < VPT / 16 ? wb + 16 * i : wb;
      raw[i] = *reinterpret_cast<const u32x4_t*>(mc ? m : w);
    }
  };
  // ---- decode the raw registers into one LDS buffer (exact fp16)
  auto decode = [&](const u32x4_t (&raw)[NLD], uint8_t* buf, bool main_chunk) {
    uint8_t* rp = buf + dkey * KSTB + dseg * NU * 16;
    if (main_chunk) {
      // this thread's scale bytes: offset (dseg*NSB) mod 16 of slot NCL
      const int so = (dseg * NSB) & 15;
      const u32x4_t sv = raw[NCL];
      const uint32_t sw = ((so >> 2) == 0 ? sv[0] : (so >> 2) == 1 ? sv[1] : (so >> 2) == 2 ? sv[2] : sv[3]) >>
                          (8 * (so & 3));
      // the E4M3 block scales as exact fp16 values (two per conversion); an E2M1
      // value times its scale has at most 6 significant bits, so the fp16 product
      // below is exact
      f16x2_t mm[NSB];
      {
        const f16x2_t s01 = __builtin_bit_cast(f16x2_t, fp8x2_f16<false>(sw));
        mm[0] = f16x2_t{s01[0], s01[0]};
        if constexpr (NSB >= 2) mm[1] = f16x2_t{s01[1], s01[1]};
        if constexpr (NSB >= 4) {
          const f16x2_t s23 = __builtin_bit_cast(f16x2_t, fp8x2_f16<true>(sw));
          mm[2] = f16x2_t{s23[0], s23[0]};
          mm[3] = f16x2_t{s23[1], s23[1]};
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        // codes of dims 8u .. 8u+7 of the range (VPT == 16: in half dseg%2 of slot 0)
        uint32_t w;
        if constexpr (VPT >= 32) w = raw[u / 4][u % 4];
        else w = (dseg & 1) ? raw[0][2 + u] : raw[0][u];
        const int j = u / 2;
        const u32x4_t pk = {__builtin_bit_cast(uint32_t, fp4x2_f16<0>(w, 1.0f) * mm[j]),
                            __builtin_bit_cast(uint32_t, fp4x2_f16<1>(w, 1.0f) * mm[j]),
                            __builtin_bit_cast(uint32_t, fp4x2_f16<2>(w, 1.0f) * mm[j]),
                            __builtin_bit_cast(uint32_t, fp4x2_f16<3>(w, 1.0f) * mm[j])};
        *reinterpret_cast<u32x4_t*>(rp + 16 * u) = pk;
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t w0 = raw[u / 2][2 * (u % 2)], w1 = raw[u / 2][2 * (u % 2) + 1];
        const u32x4_t pk = {fp8x2_f16<false>(w0), fp8x2_f16<true>(w0), fp8x2_f16<false>(w1),
                            fp8x2_f16<true>(w1)};
        *reinterpret_cast<u32x4_t*>(rp + 16 * u) = pk;
      }
    }
  };

  // the first two chunks' bytes are requested before the query, so the waits overlap
  u32x4_t raw2[NLD];
  if (c_begin < c_end) load_raw(raw, c_begin);
  if (c_begin + 1 < c_end) load_raw(raw2, c_begin + 1);

  // ---- this wave's query quarter (B operand of S^T), moved into fp16 exactly by
  // a power of two per head that the four dim-quarter waves share (so partial
  // logit tiles add without rescaling); the exponent needs every quarter's
  // largest |q|, which is exchanged at the prologue's barrier
  f16x8_t qh[DH / 16];
  float qs;  // logits of head hl = (sum of the partial tiles) * qs
  u32x4_t qraw[DH / 16];
  {
    const uint16_t* qr = q + ((size_t)row * H_q + head0 + hl) * D + dim0 + 8 * hh;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) qraw[s] = *reinterpret_cast<const u32x4_t*>(qr + 16 * s);
    float mx = 0.0f;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mx = fmaxf(mx, fabsf(__uint_as_float(qraw[s][k] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(qraw[s][k] & 0xFFFF0000u)));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (hh == 0) s_qmax[wave][hl] = mx;
  }
  auto convert_q = [&]() {
    const int hg = wave % HG2;
    float mx = s_qmax[hg][hl];
#pragma unroll
    for (int k = 1; k < DS; ++k) mx = fmaxf(mx, s_qmax[hg + HG2 * k][hl]);
    int e = 0;  // the head's largest |q| x 2^-e lands in [2^14, 2^15)
    if (mx > 0.0f) e = min(126, max(-126, (int)((__float_as_uint(mx) >> 23) & 255u) - 127 - 14));
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    qs = __uint_as_float((uint32_t)(127 + e) << 23);
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qh[s][2 * k] = (_Float16)(__uint_as_float(qraw[s][k] << 16) * inv);
        qh[s][2 * k + 1] = (_Float16)(__uint_as_float(qraw[s][k] & 0xFFFF0000u) * inv);
      }
    }
  };

  f32x16_t o[DH / 32];
#pragma unroll
  for (int n = 0; n < DH / 32; ++n) o[n] = f32x16_t{};
  float m_ref = -INFINITY, l_run = 0.0f;
  const float log2_swa = log2f(swa_scale), inv_swa = 1.0f / swa_scale;  // swa_scale > 0 here

  // S^T operand: MFMA row hl = key key_of_row(hl), dims dim0 + 16s + 8hh
  // (+32 bytes per step s)
  const int qk_off = key_of_row(hl) * KSTB + ((dim0 >> 3) + hh) * 16;
  // transposing V reads, k-step t, slots 0-3 / 4-7 = MFMA rows 16t + 4hh + e /
  // 16t + 8 + 4hh + e = keys 16t + 4e + hh / 16t + 4e + hh + 2; as a source lane
  // this lane addresses e = (lane%16)/4 and dims dim0 + 32n + vd .. +3
  const int vd = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int pv_off = (4 * ((lane & 15) >> 2) + hh) * KSTB + ((dim0 + vd) >> 3) * 16 + (((vd >> 2) & 1) << 3);

  auto qk = [&](const uint8_t* kb) {
    f32x16_t st = f32x16_t{};
    const uint8_t* kr = kb + qk_off;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s)
      st = mfma32x32x16_f16(*reinterpret_cast<const f16x8_t*>(kr + 32 * s), qh[s], st);
    return st;
  };
  // The head group's four partial logit tiles: each wave adds one quarter of the
  // tile (in dim-quarter order) and every wave reads the finished tile.  The
  // first barrier also orders everything before it against what follows (buffer
  // reuse), the second publishes the sum.
  auto exchange = [&](f32x16_t st) {
    float4* mine = reinterpret_cast<float4*>(sx + wave * 1024);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      mine[r * 64 + lane] = make_float4(st[4 * r], st[4 * r + 1], st[4 * r + 2], st[4 * r + 3]);
    lds_barrier();
    const int hg = wave % HG2;
    const float4* grp = reinterpret_cast<const float4*>(sx + hg * 1024) + dq * 64 + lane;
    const float4 a0 = grp[0], a1 = grp[HG2 * 256], a2 = grp[2 * HG2 * 256], a3 = grp[3 * HG2 * 256];
    reinterpret_cast<float4*>(sfin + hg * 1024)[dq * 64 + lane] =
        make_float4((a0.x + a1.x) + (a2.x + a3.x), (a0.y + a1.y) + (a2.y + a3.y),
                    (a0.z + a1.z) + (a2.z + a3.z), (a0.w + a1.w) + (a2.w + a3.w));
    lds_barrier();
    const float4* fin = reinterpret_cast<const float4*>(sfin + hg * 1024);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 v = fin[r * 64 + lane];
      st[4 * r] = v.x;
      st[4 * r + 1] = v.y;
      st[4 * r + 2] = v.z;
      st[4 * r + 3] = v.w;
    }
    return st;
  };

  // ---- prologue: chunks c_begin and c_begin+1 decoded, c_begin+2 in flight,
  // the logits of c_begin summed
  f32x16_t st = f32x16_t{};
  if (c_begin < c_end) {
    decode(raw, kv[0], c_begin < nm);
    if (c_begin + 1 < c_end) {
      decode(raw2, kv[1], c_begin + 1 < nm);
      if (c_begin + 2 < c_end) load_raw(raw, c_begin + 2);
    }
    lds_barrier();
    convert_q();
    st = exchange(qk(kv[0]));
  }
  for (int c = c_begin; c < c_end; ++c) {
    const int buf = (c - c_begin) % 3;
    const bool main_chunk = c < nm;
    // ---- S^T of the next chunk (its result is only needed after this chunk's
    // softmax and P·V, so the MFMAs overlap them); past the last chunk it reads
    // a stale buffer and is discarded
    const f32x16_t stn = qk(kv[buf == 2 ? 0 : buf + 1]);

    // ---- logits of chunk c: lane holds head hl, MFMA rows 8(i/4) + 4hh + i%4;
    // bit m of vmask = key key_of_row(m) is real
    const int kr = key_of_row(hl);
    const int slot = min(max(c * kKC + kr - sl_lo, 0), kMaxSel - 1);  // used for a selection chunk
    const bool sel_ok = s_ent[slot] >= 0, win_ok = (c - nm) * kKC + kr < n_swa;
    const uint32_t vmask = (uint32_t)__ballot(main_chunk ? sel_ok : win_ok);
    const float ks = main_chunk ? 1.0f : swa_scale;
    const float fs = ks * sm_log2 * qs;
    float lg[16];
    if (vmask == 0xFFFFFFFFu) {  // a full chunk (most of them): no per-key test
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = st[i] * fs;
        // the logit is rounded on its own (as the reference maximum is): a fused
        // multiply-subtract below could land an ulp above the reference, which at
        // extreme magnitudes is far more than the lazy margin
        asm("" : "+v"(x));
        lg[i] = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i / 4) + 4 * hh + (i % 4);
        lg[i] = ((vmask >> key) & 1u) ? st[i] * fs : -INFINITY;
      }
    }
    // Lazy reference maximum: it only moves (for both lanes of a head) when a
    // logit exceeds it by more than 2^kLazy; everything but the rare rescale of
    // O is branch-free, so this chunk's softmax and the next chunk's S^T MFMAs
    // form one block the scheduler can interleave.
    float lmax = lg[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) lmax = fmaxf(lmax, lg[i]);
    const float cmax = fmaxf(lmax, __shfl_xor(lmax, 32));
    const bool up = cmax > m_ref + kLazy || (m_ref == -INFINITY && cmax != -INFINITY);
    const float alpha = up ? (m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - cmax)) : 1.0f;
    m_ref = up ? cmax : m_ref;
    l_run *= alpha;
    // P times the key scale, in fp16 (A operand of k-step t = elements 8t .. 8t+7):
    // p * ks = exp2(lg - (m_ref - log2 ks)), and the row sum gains sum(p * ks) / ks.
    // The row sum adds the fp16-rounded values that P·V multiplies (exact products
    // in the dot), so numerator and denominator carry the same probabilities and a
    // key that takes all the weight is reproduced exactly.
    // While no key has been seen (m_ref = -inf) every lg is -inf and p = 0.
    const float mp = m_ref == -INFINITY ? 0.0f : m_ref - (main_chunk ? 0.0f : log2_swa);
    f16x8_t pa[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) pa[i / 8][i % 8] = (_Float16)__builtin_amdgcn_exp2f(lg[i] - mp);
    float psum = 0.0f;
    {
      const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa[t], pa[t], 0, 1), one2, psum, false);
        psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa[t], pa[t], 2, 3), one2, psum, false);
        psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa[t], pa[t], 4, 5), one2, psum, false);
        psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa[t], pa[t], 6, 7), one2, psum, false);
      }
    }
    l_run += main_chunk ? psum : psum * inv_swa;
    if (__ballot(up)) {
      float al[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) al[i] = __shfl(alpha, 8 * (i / 4) + 4 * hh + (i % 4));
#pragma unroll
      for (int n = 0; n < DH / 32; ++n) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[n][i] *= al[i];
      }
    }
    // ---- O += P·V: V slot s of k-step t = MFMA row 16t + 8(s/4) + 4hh + s%4, i.e.
    // key 16t + 4(s%4) + hh (+2 for s >= 4)
    {
      const uint8_t* vb = kv[buf] + pv_off;
#pragma unroll
      for (int n = 0; n < DH / 32; ++n) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f16x4_t lo = lds_read_tr(vb + 16 * t * KSTB + 64 * n);
          const f16x4_t hi = lds_read_tr(vb + (16 * t + 2) * KSTB + 64 * n);
          o[n] = mfma32x32x16_f16(pa[t], __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), o[n]);
        }
      }
    }
    // ---- decode chunk c+2 into the buffer chunk c-1 used, load chunk c+3
    if (c + 2 < c_end) {
      decode(raw, kv[buf == 0 ? 2 : buf - 1], c + 2 < nm);
      if (c + 3 < c_end) load_raw(raw, c + 3);
    }
    // ---- logits of chunk c+1
    if (c + 1 < c_end) st = exchange(stn);
  }

  // ---- epilogue: O element i of lane l is head 8(i/4) + 4hh + i%4, dim l%32
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  float rl[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) rl[i] = __shfl(l_tot, 8 * (i / 4) + 4 * hh + (i % 4));
  if (n_splits == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rl[i] = rl[i] > 0.0f ? 1.0f / rl[i] : 0.0f;
#pragma unroll
    for (int n = 0; n < DH / 32; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const size_t h = (size_t)row * H_q + head0 + 8 * (i / 4) + 4 * hh + (i % 4);
        out[h * D + dim0 + 32 * n + hl] = o[n][i] * rl[i];
      }
    }
    if (lse != nullptr && dq == 0 && hh == 0)
      lse[(size_t)row * H_q + head0 + hl] =
          l_tot > 0.0f ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  } else {
    const size_t base = ((size_t)row * n_splits + split) * H_q + head0;
#pragma unroll
    for (int n = 0; n < DH / 32; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        part_o[(base + 8 * (i / 4) + 4 * hh + (i % 4)) * D + dim0 + 32 * n + hl] = o[n][i];
    }
    if (dq == 0 && hh == 0) {
      part_ml[(base + hl) * 2 + 0] = m_ref;
      part_ml[(base + hl) * 2 + 1] = l_tot;
    }
  }
}

bool attn_f16_supported(int H_q, int d, float swa_scale) {
  return H_q % 32 == 0 && (d == 256 || d == 512) && swa_scale > 0.0f && swa_scale <= 128.0f;
}

hipError_t launch_sparse_attn_f16(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                  int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                  int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                  int H_q, int d, float sm_log2, const AttnPlan& p, int rows,
                                  int hg2, float* part_o, float* part_ml, float* out, float* lse,
                                  hipStream_t st) {
  const int head_groups = H_q / (32 * hg2);
  dim3 grid(xcd_grid(rows, p.n_splits * head_groups));
#define CSA2_ATTN16(D_, HG_)                                                                      \
  hipLaunchKernelGGL((sparse_attn_f16_kernel<D_, HG_>), grid, dim3(HG_ * 256), 0, st, q, codes,   \
                     scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq, H_q, sm_log2, \
                     p.chunks_per_split, p.n_splits, rows, head_groups, part_o, part_ml, out, lse)
  if (d == 512) {
    if (hg2 == 2) CSA2_ATTN16(512, 2);
    else CSA2_ATTN16(512, 1);
  } else {
    if (hg2 == 2) CSA2_ATTN16(256, 2);
    else CSA2_ATTN16(256, 1);
  }
#undef CSA2_ATTN16
  return hipGetLastError();
}

}  // namespace csa2
