// Sparse attention for few query rows (decode steps): main Q attends to
// (selected FP4 entries ++ layer-local FP8 window) with every key of a row handled
// inside one workgroup, so no split partials go through HBM and no combine
// launch follows.  Same function and readings as the split-K kernels of
// attn_f16.hip / attn.hip, which remain for many rows (prefill chunks, many
// queries per sequence).
//
// [deep-dive §3.1] Main Q attends to the selected main KV plus the layer-local
// SWA KV; [digest 已确认] the selected entries are concatenated with the windowed
// KV; [reading §4.2] every layer has its own query and window.  Readings: K = V =
// the whole dequantised entry, shared by all query heads; one softmax over all
// keys; window tokens are E4M3 values times swa_scale.
//
// Work split: a workgroup owns one query row, 16 heads and one part (D / DP) of
// the output dims.  Its NW waves take the row's 16-key tiles round robin (tile t
// to wave t mod NW; the selected entries first, then the window tokens); each
// wave keeps its own online softmax and needs no barrier inside its loop.  The
// waves' (O, m, l) are merged through LDS at the end, in wave order.
// Per tile and wave:
//   * S^T = K·Q^T on MFMA 16x16x32 f16: rows = the tile's 16 keys, columns = the
//     16 heads.  Lane (key r, group G) decodes dims [G·D/4, (G+1)·D/4) of its key
//     straight into the A operand, exactly in fp16 (an E2M1 value times its E4M3
//     block scale has at most 6 significant bits and lies in [2^-10, 2688]; an
//     E4M3 window value has at most 4 in [2^-9, 448]).  The reduction order is
//     permuted so each lane reads contiguous code bytes; Q is permuted alike.
//   * Lanes whose dims fall in the workgroup's output part also write them to
//     the wave's own key-major LDS tile; the V operand of O += P·V comes from it
//     through the transposing LDS read (ds_read_b64_tr_b16).
//   * In the S^T result a lane holds one head's logits for 4 keys, which is
//     directly the P operand of O += P·V on MFMA 16x16x16 f16 (rows = heads).
// The bf16 query is moved into fp16 exactly by a power of two per head (the
// head's largest |q| lands in [2^14, 2^15)), which is undone on the logits.
// Probabilities are rounded to fp16 once and the row sums add the rounded values,
// so a key that takes all the weight is reproduced exactly.
#include "attn_common.h"

namespace csa2 {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// D(16x16, f32) += A(16x32, f16) * B(32x16, f16); lane l holds A row l%16 / B
// column l%16 with 8 reduction elements of slot group l/16, and D rows 4(l/16)+i,
// column l%16 in element i.
CSA2_DEV f4_t mfma_qk(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// D(16x16, f32) += A(16x16, f16) * B(16x16, f16); reduction elements 4(l/16)..+3.
CSA2_DEV f4_t mfma_pv(h4_t a, h4_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// 8 bytes per lane from LDS, transposed inside each 16-lane group: lane j of the
// group receives element j%4 of what lanes 4e + j/4 (e = 0..3) addressed.
CSA2_DEV h4_t lds_read_tr4(const uint8_t* p) {
  typedef __attribute__((address_space(3))) s4_t lds_s4;
  return __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p)));
}
// exact conversions (checked exhaustively on the hardware): the two E2M1 codes of
// byte SEL (low nibble first); two E4M3 bytes (low or high half of the word)
template <int SEL>
CSA2_DEV h2_t e2m1x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
template <bool HI>
CSA2_DEV h2_t e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
CSA2_DEV h8_t cat8(h2_t a, h2_t b, h2_t c, h2_t d) {
  const h4_t lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const h4_t hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

constexpr int kRowsMaxSel = 512;  // selection slots the kernel takes
constexpr int kRowsMaxWin = 128;  // visible window tokens the kernel takes

template <int D, int DP, int NW>
struct RowsShape {
  static constexpr int NT = 64 * NW;
  static constexpr int DG = D / 4;            // dims of one lane group
  static constexpr int NS = D / 32;           // MFMA steps of S^T
  static constexpr int CB = DG / 2;           // code bytes of a lane per key
  static constexpr int SB = DG / 16;          // scale bytes of a lane per key
  static constexpr int DV = D / DP;           // output dims of the workgroup
  static constexpr int NJ = DV / 16;          // MFMAs of P·V per tile
  static constexpr int VROW = 2 * DV + 32;    // bytes per key row of a V tile
  static constexpr int QROW = 2 * D + 16;     // bytes per head row of the fp16 query
  static constexpr int OROW = DV + 4;         // floats per head row of a merge tile
  // the row's tiles are dealt round robin to the NW waves: a wave iterates JS
  // times over selection tiles, then JW times over window tiles, so the kind of
  // every iteration is fixed at compile time
  static constexpr int TPI = NW;
  static constexpr int JS = kRowsMaxSel / 16 / TPI;
  static constexpr int JW = (kRowsMaxWin / 16 + TPI - 1) / TPI;
  static constexpr int JMAX = JS + JW;
  static constexpr int RAW4 = (DG / 16 > CB / 16 + 1) ? DG / 16 : CB / 16 + 1;
  static constexpr int LDS_MAIN = 16 * QROW + 64 + NW * 2 * 16 * VROW;
  static constexpr int LDS_MERGE = NW * 16 * OROW * 4 + 2 * NW * 16 * 4;
  static constexpr int LDS = LDS_MAIN > LDS_MERGE ? LDS_MAIN : LDS_MERGE;
};

template <int D, int DP, int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_rows_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, int H_q, float sm_log2, int rows,
    float* __restrict__ out, float* __restrict__ lse) {
  using SH = RowsShape<D, DP, NW>;
  constexpr int NT = SH::NT, DG = SH::DG, NS = SH::NS, CB = SH::CB, SB = SH::SB;
  constexpr int DV = SH::DV, NJ = SH::NJ, VROW = SH::VROW, QROW = SH::QROW, OROW = SH::OROW;
  constexpr int JS = SH::JS, JMAX = SH::JMAX, RAW4 = SH::RAW4;
  constexpr int TPI = SH::TPI;
  static_assert(JS * TPI * 16 == kRowsMaxSel && JS >= 1, "tile slots");
  static_assert(SB == 4 || SB == 8, "scale bytes per lane");
  static_assert(CB % 16 == 0 && DG % 16 == 0 && DV % 16 == 0, "lane shapes");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SH::LDS];

  const int per_row = (H_q / 16) * DP;
  int row, unit;
  if (!xcd_map(blockIdx.x, rows, per_row, row, unit)) return;
  const int hg = unit / DP, dp = unit - hg * DP;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, G = lane >> 4;
  const int h0 = hg * 16;

  // ---- tiles: selection slots first (invalid slots masked), then the window
  const int n_sel = N > 0 ? K : 0;
  const int ts = (n_sel + 15) / 16;
  const WinRange win = window_of(q_pos, row, S, swa_pos0, n_win);
  // tile index (selection or window) and whether it exists, of iteration j
  auto tile_of = [&](int j) { return j < JS ? wave + j * TPI : wave + (j - JS) * TPI; };
  auto live_of = [&](int j) { return j < JS ? tile_of(j) < ts : 16 * tile_of(j) < win.n; };

  // entries of this wave's selection tiles (key r of each), requested first
  const int* srow = sel + (size_t)row * K;
  int ent[JS];
#pragma unroll
  for (int j = 0; j < JS; ++j) {
    const int slot = 16 * tile_of(j) + r;
    int e = -1;
    if (slot < n_sel) e = srow[slot];
    ent[j] = (e >= 0 && e < N) ? e : -1;
  }

  // the query slice this thread stages (requested before anything that waits)
  constexpr int TPH = NT / 16;  // threads per head (consecutive lanes of one wave)
  constexpr int VPT = D / TPH;  // query values per thread
  const int qh = tid / TPH, part = tid - qh * TPH;
  u4_t qv[VPT / 8];
  {
    const uint16_t* qr = q + ((size_t)row * H_q + h0 + qh) * D + part * VPT;
#pragma unroll
    for (int i = 0; i < VPT / 8; ++i) qv[i] = *reinterpret_cast<const u4_t*>(qr + 8 * i);
  }

  // ---- raw bytes of a tile, RAW4 16-byte loads for either kind: a selected
  // entry as the lane's CB code bytes and the aligned 16 bytes of its scale row
  // holding the lane's SB scales (the remaining loads repeat the scale row), a
  // window token as its DG bytes.  A selection slot past the list reads entry 0
  // and a window slot past the window reads its first token (both real cache
  // bytes, masked later); with no entries or no window at all the query row is
  // read instead (those iterations skip P·V, so its bytes never reach O).
  const size_t seq = (size_t)b * N;
  const uint8_t* qdummy = reinterpret_cast<const uint8_t*>(q + (size_t)row * H_q * D);
  struct Raw {
    u4_t v[RAW4];
  };
  auto load_tile = [&](int j) {
    Raw R;
    const int t = tile_of(j);
    if (j < JS) {
      const size_t e = seq + (size_t)max(ent[j], 0);
      const uint8_t* cb = codes + e * (D / 2) + G * CB;
      const uint8_t* sb = scales + e * (D / 16) + ((G * SB) & ~15);
#pragma unroll
      for (int i = 0; i < RAW4; ++i) {
        const uint8_t* p = i < CB / 16 ? cb + 16 * i : sb;
        R.v[i] = *reinterpret_cast<const u4_t*>(ts > 0 ? p : qdummy + 16 * i);
      }
    } else {
      const int wi = 16 * t + r;
      const uint8_t* wb = swa + ((size_t)b * S + window_slot(win, wi < win.n ? wi : 0, S)) * D + G * DG;
#pragma unroll
      for (int i = 0; i < RAW4; ++i) {
        const int u = i < DG / 16 ? i : 0;
        R.v[i] = *reinterpret_cast<const u4_t*>(win.n > 0 ? wb + 16 * u : qdummy + 16 * i);
      }
    }
    return R;
  };
  // the first two tiles' bytes are requested before the query is staged
  Raw rawA = load_tile(0), rawB = load_tile(1);

  // ---- query: the workgroup's 16 heads in fp16 in LDS, a power of two per head
  uint8_t* qlds = smem;
  float* s_qs = reinterpret_cast<float*>(smem + 16 * QROW);
  {
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT / 8; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mx = fmaxf(mx, fabsf(__uint_as_float(qv[i][k] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(qv[i][k] & 0xFFFF0000u)));
      }
    }
#pragma unroll
    for (int o = 1; o < TPH; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    int e = 0;  // the head's largest |q| x 2^-e lands in [2^14, 2^15)
    if (mx > 0.0f) e = min(126, max(-126, (int)((__float_as_uint(mx) >> 23) & 255u) - 127 - 14));
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    if (part == 0) s_qs[qh] = __uint_as_float((uint32_t)(127 + e) << 23);
    uint8_t* qw = qlds + qh * QROW + 2 * part * VPT;
#pragma unroll
    for (int i = 0; i < VPT / 8; ++i) {
      h8_t v;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = (_Float16)(__uint_as_float(qv[i][k] << 16) * inv);
        v[2 * k + 1] = (_Float16)(__uint_as_float(qv[i][k] & 0xFFFF0000u) * inv);
      }
      *reinterpret_cast<h8_t*>(qw + 16 * i) = v;
    }
  }
  lds_barrier();
  // B operand of S^T: head r, dims G·DG + 8s .. +7 at step s
  h8_t qb[NS];
  {
    const uint8_t* qrow = qlds + r * QROW + 2 * G * DG;
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[s] = *reinterpret_cast<const h8_t*>(qrow + 16 * s);
  }
  const float qsl = s_qs[r];

  // ---- the wave's tiles, software-pipelined: while tile j's softmax and P·V
  // run, tile j+1 is decoded and its S^T formed (two V buffers per wave), and
  // the bytes of tile j+2 are in flight
  uint8_t* vt0 = smem + 16 * QROW + 64 + wave * 2 * 16 * VROW;  // this wave's V tiles
  // lanes whose dims lie in this workgroup's output part write them to a V tile
  const bool vw = G * DG >= dp * DV && G * DG < dp * DV + DV;
  const int vwr = r * VROW + 2 * (G * DG - dp * DV);
  // transposing V read: this lane addresses key row 4G + (lane%16)/4, dims 4(lane%4)
  const int vrd = (4 * G + ((lane & 15) >> 2)) * VROW + 8 * (lane & 3);
  const float log2_swa = log2f(swa_scale), inv_swa = 1.0f / swa_scale;
  f4_t o[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) o[jj] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY, l_run = 0.0f;

  // S^T of a selection tile (decoding it into V tile vb): two MFMA chains
  auto qk_sel = [&](const Raw& R, uint8_t* vb) {
    const u4_t* raw = R.v;
    _Float16 scl[SB];  // the lane's block scales as exact fp16 values (16 dims each)
    // the lane's SB scale bytes start at byte (G * SB) mod 16 of the scale load
    const int sw0 = ((G * SB) & 15) >> 2;
#pragma unroll
    for (int k = 0; k < SB / 4; ++k) {
      const int wi = sw0 + k;
      const uint32_t w = wi == 0 ? raw[CB / 16][0] : wi == 1 ? raw[CB / 16][1] : wi == 2 ? raw[CB / 16][2] : raw[CB / 16][3];
      const h2_t a = e4m3x2<false>(w), c = e4m3x2<true>(w);
      scl[4 * k] = a[0];
      scl[4 * k + 1] = a[1];
      scl[4 * k + 2] = c[0];
      scl[4 * k + 3] = c[1];
    }
    f4_t s0 = f4_t{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t w = raw[s / 4][s % 4];
      const h2_t m2 = h2_t{scl[s / 2], scl[s / 2]};
      const h8_t a = cat8(e2m1x2<0>(w) * m2, e2m1x2<1>(w) * m2, e2m1x2<2>(w) * m2, e2m1x2<3>(w) * m2);
      if (s & 1) s1 = mfma_qk(a, qb[s], s1);
      else s0 = mfma_qk(a, qb[s], s0);
      if (vw) *reinterpret_cast<h8_t*>(vb + vwr + 16 * s) = a;
    }
    return s0 + s1;
  };
  // S^T of a window tile
  auto qk_win = [&](const Raw& R, uint8_t* vb) {
    const u4_t* raw = R.v;
    f4_t s0 = f4_t{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t w0 = raw[(2 * s) / 4][(2 * s) % 4], w1 = raw[(2 * s + 1) / 4][(2 * s + 1) % 4];
      const h8_t a = cat8(e4m3x2<false>(w0), e4m3x2<true>(w0), e4m3x2<false>(w1), e4m3x2<true>(w1));
      if (s & 1) s1 = mfma_qk(a, qb[s], s1);
      else s0 = mfma_qk(a, qb[s], s0);
      if (vw) *reinterpret_cast<h8_t*>(vb + vwr + 16 * s) = a;
    }
    return s0 + s1;
  };
  // O += P·V from V tile vb
  auto pv = [&](const h4_t pa, const uint8_t* vb) {
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) o[jj] = mfma_pv(pa, lds_read_tr4(vb + vrd + 32 * jj), o[jj]);
  };

  f4_t st = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  st = JS > 0 ? qk_sel(rawA, vt0) : qk_win(rawA, vt0);

#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    const int t = tile_of(j);
    const bool mt = j < JS, live = live_of(j);
    // bytes of tile j+2 into the registers tile j came in (decoded one step ago)
    if (j + 2 < JMAX) {
      if (j & 1) rawB = load_tile(j + 2);
      else rawA = load_tile(j + 2);
    }
    // logits of tile j: lane holds head r, keys 4G + i; bit k of vmask = key k is real
    uint32_t vmask;
    if (mt) {
      vmask = (uint32_t)__ballot(ent[j] >= 0) & 0xFFFFu;  // lane k (< 16) holds key k's entry
    } else {
      const int nv = win.n - 16 * t;
      vmask = nv >= 16 ? 0xFFFFu : (nv > 0 ? (1u << nv) - 1u : 0u);
    }
    const float fs = (mt ? 1.0f : swa_scale) * sm_log2 * qsl;
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = st[i] * fs;
      // rounded on its own, like the reference maximum taken from it
      asm volatile("" : "+v"(x));
      lg[i] = ((vmask >> (4 * G + i)) & 1u) ? x : -INFINITY;
    }
    // lazy reference maximum (moves only when a logit exceeds it by > kLazy);
    // the four lanes of a head always share it
    const float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__ballot(lmax > m_ref + kLazy || (m_ref == -INFINITY && lmax != -INFINITY))) {
      float cm = fmaxf(lmax, __shfl_xor(lmax, 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      const bool up = cm > m_ref + kLazy || (m_ref == -INFINITY && cm != -INFINITY);
      const float alpha = up ? (m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - cm)) : 1.0f;
      m_ref = up ? cm : m_ref;
      l_run *= alpha;
      // O rows are heads 4G + i, whose alpha lane 4G + i holds
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * G + i);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[jj][i] *= al[i];
      }
    }
    // P (times the key scale for window tokens) in fp16: the A operand of P·V;
    // the row sum adds the rounded values
    const float mp = m_ref == -INFINITY ? 0.0f : m_ref - (mt ? 0.0f : log2_swa);
    h4_t pa;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(lg[i] - mp);
      pa[i] = ph;
      psum += (float)ph;
    }
    l_run += mt ? psum : psum * inv_swa;
    // tile j+1's S^T beside tile j's P·V, both in one block (so the two streams
    // interleave); a tile that does not exist skips P·V (its V tile may hold
    // bytes that are not cache values)
    const uint8_t* vcur = vt0 + (j & 1) * 16 * VROW;
    uint8_t* vnext = vt0 + ((j + 1) & 1) * 16 * VROW;
    const Raw& rn = (j & 1) ? rawA : rawB;
    if (j + 1 < JMAX) {
      if (live) {
        const f4_t sn = j + 1 < JS ? qk_sel(rn, vnext) : qk_win(rn, vnext);
        pv(pa, vcur);
        st = sn;
      } else {
        st = j + 1 < JS ? qk_sel(rn, vnext) : qk_win(rn, vnext);
      }
    } else if (live) {
      pv(pa, vcur);
    }
  }

  // ---- merge the waves: (O, m, l) per wave through LDS, summed in wave order
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  lds_barrier();  // every wave is done with the query and V tiles
  float* po = reinterpret_cast<float*>(smem);  // [NW][16][OROW]
  float* pm = po + NW * 16 * OROW;             // [NW][16]
  float* pl = pm + NW * 16;                    // [NW][16]
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
#pragma unroll
    for (int i = 0; i < 4; ++i) po[(wave * 16 + 4 * G + i) * OROW + 16 * jj + r] = o[jj][i];
  }
  if (G == 0) {
    pm[wave * 16 + r] = m_ref;
    pl[wave * 16 + r] = lt;
  }
  lds_barrier();
  {
    constexpr int TPH = NT / 16, OPT = DV / TPH;  // threads per head, outputs per thread
    static_assert(OPT % 4 == 0, "merge shape");
    const int h = tid / TPH, c0 = (tid - h * TPH) * OPT;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, pm[w * 16 + h]);
    float a[NW], L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = pm[w * 16 + h];
      a[w] = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      L += a[w] * pl[w * 16 + h];
    }
    float4 acc[OPT / 4];
#pragma unroll
    for (int c = 0; c < OPT; c += 4) {
      float4 v4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4 v = *reinterpret_cast<const float4*>(po + (w * 16 + h) * OROW + c0 + c);
        v4.x += a[w] * v.x;
        v4.y += a[w] * v.y;
        v4.z += a[w] * v.z;
        v4.w += a[w] * v.w;
      }
      acc[c / 4] = v4;
    }
    float* orow = out + ((size_t)row * H_q + h0 + h) * D + dp * DV + c0;
    {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
      for (int c = 0; c < OPT; c += 4) {
        const float4 v = acc[c / 4];
        *reinterpret_cast<float4*>(orow + c) = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
      }
      if (lse != nullptr && dp == 0 && c0 == 0)
        lse[(size_t)row * H_q + h0 + h] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

}  // namespace

bool attn_rows_supported(int H_q, int d, int K, int S, int n_win, bool with_pos, float swa_scale) {
  const int vis = with_pos ? (S < n_win ? S : n_win) : S;  // window tokens a query can see
  return H_q % 16 == 0 && (d == 256 || d == 512) && K <= kRowsMaxSel && vis <= kRowsMaxWin &&
         swa_scale > 0.0f && swa_scale <= 128.0f;
}

hipError_t launch_sparse_attn_rows(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                   int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                   int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                   int H_q, int d, float sm_log2, int rows, int dp, float* out,
                                   float* lse, hipStream_t st) {
#define CSA2_ROWS(D_, DP_, NW_)                                                                    \
  hipLaunchKernelGGL((sparse_attn_rows_kernel<D_, DP_, NW_>),                                      \
                     dim3(xcd_grid(rows, (H_q / 16) * DP_)), dim3(64 * NW_), 0, st, q, codes,      \
                     scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq, H_q, sm_log2, \
                     rows, out, lse)
  if (d == 512) {
    if (dp == 4) CSA2_ROWS(512, 4, 8);
    else if (dp == 2) CSA2_ROWS(512, 2, 8);
    else CSA2_ROWS(512, 1, 4);
  } else {
    if (dp == 2) CSA2_ROWS(256, 2, 8);
    else CSA2_ROWS(256, 1, 4);
  }
#undef CSA2_ROWS
  return hipGetLastError();
}

}  // namespace csa2
