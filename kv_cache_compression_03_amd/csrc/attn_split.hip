// Sparse attention for few query rows in two launches: every key of a row is
// decoded and scored once, for all 64 heads, and the output dims are spread over
// many workgroups afterwards.
//
// [deep-dive §3.1] Main Q attends to the selected main KV plus the layer-local
// SWA KV; [digest 已确认] the selected entries are concatenated with the windowed
// KV; [reading §4.2] every layer has its own query and window.  Readings: K = V =
// the whole dequantised entry, shared by all query heads; one softmax over all
// keys; window tokens are E4M3 values times swa_scale.
//
// A decode step has few rows (8 at 8 sequences), each with up to 640 keys of 512
// dims.  Scoring a key needs all 512 dims of it and of each head's query, while
// P·V needs only the dims of the output part being formed.  Splitting rows over
// (head group, output part) workgroups, as the one-launch kernel does, decodes
// and scores every key once per workgroup; here the two halves run apart:
//   1. attn_split_logits_kernel: a workgroup per (row, 32-key chunk).  The chunk
//      is decoded once (exact fp16) into LDS; each of the four waves forms S^T
//      for 16 heads (MFMA 16x16x32 f16, the query in registers scaled into fp16
//      by a power of two per head), takes the chunk's maximum per head and writes
//        P   = fp16(exp2(logit - chunk max))            (x swa_scale for window
//              keys, whose value scale folds into P as in the other kernels),
//        m, l = the chunk maximum and the sum of the rounded P (/ swa_scale for
//              window keys),
//      and the decoded chunk again as V, already in the B-operand order of the
//      P·V MFMA (read back from LDS with the transposing read), 1 KB per 16 dims.
//   2. attn_split_pv_kernel: a workgroup per (row, 16 heads, 64 dims).  From the
//      chunks' (m, l) it forms the row maximum M, the weights a_c = exp2(m_c - M)
//      and L = sum a_c l_c; its four waves take the chunks round robin and add
//      a_c · (P_c · V_c) (one MFMA per 16 dims per chunk); the waves' sums are
//      added through LDS and divided by L.
// The numerator and the denominator add the same rounded probabilities, so a key
// that takes all the weight is reproduced exactly, as in the other kernels.
// A window chunk past the visible window writes P = 0, V = 0 and m = -inf without
// reading anything; every other chunk reads real cache bytes for all its keys
// (a masked selection slot reads entry 0, a masked window slot the first visible
// token) so V is always finite where P is 0.
#include "attn_common.h"

namespace csa2 {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kSD = 512;                 // dims
constexpr int kSHeads = 64;              // query heads (four 16-head waves)
constexpr int kSThreads = 256;
constexpr int kSMaxSel = 512;            // selection slots
constexpr int kSMaxWin = 128;            // visible window tokens
constexpr int kSMaxChunks = kSMaxSel / kKC + kSMaxWin / kKC;
constexpr int kSBlocks = kSD / 16;       // 16-dim blocks of V
constexpr int kSSlice = 4;               // blocks per P·V workgroup
constexpr int kSSlices = kSBlocks / kSSlice;
constexpr int kSKRow = 2 * kSD + 16;     // LDS bytes per decoded key row
constexpr int kSOperand = 64 * 16;       // bytes of one MFMA operand of a wave

// D(16x16, f32) += A(16x32, f16) * B(32x16, f16); lane l holds A row l%16 / B
// column l%16 with 8 reduction elements of slot group l/16, and D rows 4(l/16)+i,
// column l%16 in element i.
CSA2_DEV f4_t mfma32(h8_t a, h8_t b, f4_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
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

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// Workspace of a launch: P [row][chunk][wave][lane] 16 B, (m, l) [row][chunk][head],
// V [row][chunk][16-dim block][lane] 16 B.
inline size_t split_p_bytes(size_t rows, int C) { return align256(rows * C * 4 * kSOperand); }
inline size_t split_ml_bytes(size_t rows, int C) { return align256(rows * C * kSHeads * sizeof(float2)); }
inline size_t split_v_bytes(size_t rows, int C) { return align256(rows * C * kSBlocks * kSOperand); }

__global__ __launch_bounds__(kSThreads) void attn_split_logits_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int N, const int* __restrict__ sel, int K,
    const uint8_t* __restrict__ swa, float swa_scale, int S, long long swa_pos0, int n_win,
    const int* __restrict__ q_pos, int Tq, float sm_log2, int rows, int CS, int C,
    uint8_t* __restrict__ pbuf, float2* __restrict__ mlbuf, uint8_t* __restrict__ vbuf) {
  constexpr int D = kSD, DG = D / 4, NS = D / 32;
  __shared__ __attribute__((aligned(16))) uint8_t kt[kKC * kSKRow];
  __shared__ __attribute__((aligned(16))) uint8_t s_valid[kKC];

  int row, c;
  if (!xcd_map(blockIdx.x, rows, C, row, c)) return;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, G = lane >> 4;
  const int h = wave * 16 + r;  // this lane's head (S^T column)
  const size_t unit = (size_t)row * C + c;
  uint8_t* const pdst = pbuf + (unit * 4 + wave) * kSOperand + lane * 16;
  uint8_t* const vdst = vbuf + unit * kSBlocks * kSOperand + lane * 16;

  const WinRange win = window_of(q_pos, row, S, swa_pos0, n_win);
  const bool mainc = c < CS;
  const int wbase = kKC * (c - CS);  // a window chunk's first visible token
  if (!mainc && wbase >= win.n) {
    // nothing visible in this chunk: no weight, zero values
    *reinterpret_cast<u4_t*>(pdst) = u4_t{0u, 0u, 0u, 0u};
    if (G == 0) mlbuf[unit * kSHeads + h] = make_float2(-INFINITY, 0.0f);
#pragma unroll
    for (int k = 0; k < kSBlocks / 4; ++k)
      *reinterpret_cast<u4_t*>(vdst + (size_t)(wave + 4 * k) * kSOperand) = u4_t{0u, 0u, 0u, 0u};
    return;
  }

  // ---- raw bytes: thread (key kk, part p) holds dims 64p .. 64p+63 of key kk
  // (a selected entry's 32 code bytes and 4 scale bytes, or a window token's 64
  // bytes); the loads go out before the query's
  const int kk = tid & (kKC - 1), p = tid >> 5;
  u4_t raw[4];
  bool kval;
  if (mainc) {
    const int slot = kKC * c + kk;
    const int e = slot < K ? sel[(size_t)row * K + slot] : -1;
    kval = e >= 0 && e < N;
    const size_t ent = (size_t)b * N + (kval ? e : 0);
    const uint8_t* cb = codes + ent * (D / 2) + 32 * p;
    raw[0] = *reinterpret_cast<const u4_t*>(cb);
    raw[1] = *reinterpret_cast<const u4_t*>(cb + 16);
    raw[2] = u4_t{*reinterpret_cast<const uint32_t*>(scales + ent * (D / 16) + 4 * p), 0u, 0u, 0u};
    raw[3] = raw[2];
  } else {
    const int wi = wbase + kk;
    kval = wi < win.n;
    const uint8_t* wb = swa + ((size_t)b * S + window_slot(win, kval ? wi : 0, S)) * D + 64 * p;
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = *reinterpret_cast<const u4_t*>(wb + 16 * i);
  }
  // ---- query of head h: dims G·DG + 8s .. +7 at step s (the B operand of S^T)
  u4_t qv[NS];
  {
    const uint16_t* qr = q + ((size_t)row * kSHeads + h) * D + G * DG;
#pragma unroll
    for (int s = 0; s < NS; ++s) qv[s] = *reinterpret_cast<const u4_t*>(qr + 8 * s);
  }

  // ---- decode into the chunk's key-major fp16 rows
  {
    uint8_t* krow = kt + kk * kSKRow + 2 * 64 * p;
    if (mainc) {
      const h2_t s01 = e4m3x2<false>(raw[2][0]), s23 = e4m3x2<true>(raw[2][0]);
      const _Float16 scl[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
      for (int wi = 0; wi < 8; ++wi) {
        const uint32_t w = raw[wi / 4][wi % 4];
        const h2_t m2 = h2_t{scl[wi / 2], scl[wi / 2]};
        *reinterpret_cast<h8_t*>(krow + 16 * wi) =
            cat8(e2m1x2<0>(w) * m2, e2m1x2<1>(w) * m2, e2m1x2<2>(w) * m2, e2m1x2<3>(w) * m2);
      }
    } else {
#pragma unroll
      for (int wi = 0; wi < 8; ++wi) {
        const uint32_t w0 = raw[(2 * wi) / 4][(2 * wi) % 4], w1 = raw[(2 * wi + 1) / 4][(2 * wi + 1) % 4];
        *reinterpret_cast<h8_t*>(krow + 16 * wi) =
            cat8(e4m3x2<false>(w0), e4m3x2<true>(w0), e4m3x2<false>(w1), e4m3x2<true>(w1));
      }
    }
    if (p == 0) s_valid[kk] = kval ? 1 : 0;
  }

  // ---- the query in fp16: the head's largest |q| x 2^-e lands in [2^14, 2^15)
  h8_t qb[NS];
  float qsl;
  {
    float mx = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mx = fmaxf(mx, fabsf(__uint_as_float(qv[s][k] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(qv[s][k] & 0xFFFF0000u)));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    int e = 0;
    if (mx > 0.0f) e = min(126, max(-126, (int)((__float_as_uint(mx) >> 23) & 255u) - 127 - 14));
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    qsl = __uint_as_float((uint32_t)(127 + e) << 23);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qb[s][2 * k] = (_Float16)(__uint_as_float(qv[s][k] << 16) * inv);
        qb[s][2 * k + 1] = (_Float16)(__uint_as_float(qv[s][k] & 0xFFFF0000u) * inv);
      }
    }
  }
  lds_barrier();

  // ---- S^T of the chunk's two 16-key tiles: lane (head r, group G) receives keys
  // 16u + 4G + i of tile u
  f4_t acc0 = f4_t{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  {
    const uint8_t* a0 = kt + r * kSKRow + 2 * G * DG;
    const uint8_t* a1 = a0 + 16 * kSKRow;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc0 = mfma32(*reinterpret_cast<const h8_t*>(a0 + 16 * s), qb[s], acc0);
      acc1 = mfma32(*reinterpret_cast<const h8_t*>(a1 + 16 * s), qb[s], acc1);
    }
  }
  // ---- V in the B-operand order of P·V: lane (dim j, group G) of block jb holds
  // dim 16jb + j of keys 4G .. 4G+3 of both tiles, which is the key order of the
  // P operand below (reduction slot 8G + 4u + i = key 16u + 4G + i)
  {
    const uint8_t* vr = kt + (4 * G + (r >> 2)) * kSKRow + 8 * (r & 3);
#pragma unroll
    for (int k = 0; k < kSBlocks / 4; ++k) {
      const int jb = wave + 4 * k;
      const h4_t lo = lds_read_tr4(vr + 32 * jb);
      const h4_t hi = lds_read_tr4(vr + 16 * kSKRow + 32 * jb);
      *reinterpret_cast<h8_t*>(vdst + (size_t)jb * kSOperand) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  // ---- softmax pieces of the chunk for head h
  const float log2_swa = log2f(swa_scale), inv_swa = 1.0f / swa_scale;
  const float fs = (mainc ? 1.0f : swa_scale) * sm_log2 * qsl;
  const uint32_t v0 = *reinterpret_cast<const uint32_t*>(s_valid + 4 * G);
  const uint32_t v1 = *reinterpret_cast<const uint32_t*>(s_valid + 16 + 4 * G);
  float lg[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = acc0[i] * fs, x1 = acc1[i] * fs;
    // rounded on their own, like the maximum taken from them
    asm volatile("" : "+v"(x0), "+v"(x1));
    lg[i] = ((v0 >> (8 * i)) & 1u) ? x0 : -INFINITY;
    lg[4 + i] = ((v1 >> (8 * i)) & 1u) ? x1 : -INFINITY;
  }
  float m = lg[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) m = fmaxf(m, lg[k]);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float mp = m == -INFINITY ? 0.0f : m - (mainc ? 0.0f : log2_swa);
  h8_t pa;
#pragma unroll
  for (int k = 0; k < 8; ++k) pa[k] = (_Float16)__builtin_amdgcn_exp2f(lg[k] - mp);
  // the sum adds the rounded probabilities (exact products in the dot)
  float psum = 0.0f;
  const h2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
  psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 0, 1), one2, psum, false);
  psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 2, 3), one2, psum, false);
  psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 4, 5), one2, psum, false);
  psum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pa, pa, 6, 7), one2, psum, false);
  psum += __shfl_xor(psum, 16);
  psum += __shfl_xor(psum, 32);
  *reinterpret_cast<h8_t*>(pdst) = pa;
  if (G == 0) mlbuf[unit * kSHeads + h] = make_float2(m, mainc ? psum : psum * inv_swa);
}

__global__ __launch_bounds__(kSThreads) void attn_split_pv_kernel(
    const uint8_t* __restrict__ pbuf, const float2* __restrict__ mlbuf,
    const uint8_t* __restrict__ vbuf, int rows, int C, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int OROW = 16 * kSSlice + 4;  // floats per head row of the merge tile
  __shared__ __attribute__((aligned(16))) float s_a[kSMaxChunks * 16];
  __shared__ float s_m[16], s_l[16];
  __shared__ __attribute__((aligned(16))) float s_o[4 * 16 * OROW];

  int row, unit;
  if (!xcd_map(blockIdx.x, rows, 4 * kSSlices, row, unit)) return;
  const int hg = unit / kSSlices, sl = unit - hg * kSSlices;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, G = lane >> 4;
  constexpr int CPW = (kSMaxChunks + 3) / 4;  // chunks per wave at most

  // ---- this wave's chunks (c = wave + 4j): P of the head group, V of the slice
  h8_t pc[CPW], vc[CPW][kSSlice];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = wave + 4 * j;
    if (c < C) {
      const size_t u = (size_t)row * C + c;
      pc[j] = *reinterpret_cast<const h8_t*>(pbuf + (u * 4 + hg) * kSOperand + lane * 16);
#pragma unroll
      for (int n = 0; n < kSSlice; ++n)
        vc[j][n] = *reinterpret_cast<const h8_t*>(vbuf + (u * kSBlocks + sl * kSSlice + n) * kSOperand + lane * 16);
    }
  }
  // ---- row maximum, chunk weights and the row sum, per head of the group
  // (wave 0; lane (head r, group G) reads chunks G, G+4, ...)
  if (wave == 0) {
    float2 ml[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int c = G + 4 * j;
      ml[j] = c < C ? mlbuf[((size_t)row * C + c) * kSHeads + hg * 16 + r] : make_float2(-INFINITY, 0.0f);
    }
    float M = ml[0].x;
#pragma unroll
    for (int j = 1; j < CPW; ++j) M = fmaxf(M, ml[j].x);
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    float L = 0.0f;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int c = G + 4 * j;
      const float a = ml[j].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[j].x - M);
      if (c < C) s_a[c * 16 + r] = a;
      L = fmaf(a, ml[j].y, L);
    }
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (G == 0) {
      s_m[r] = M;
      s_l[r] = L;
    }
  }
  __syncthreads();

  // ---- O (heads 4G + i, dim j of each block) += a_c · (P_c · V_c)
  f4_t o[kSSlice];
#pragma unroll
  for (int n = 0; n < kSSlice; ++n) o[n] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = wave + 4 * j;
    if (c < C) {
      const f4_t a = *reinterpret_cast<const f4_t*>(s_a + c * 16 + 4 * G);
#pragma unroll
      for (int n = 0; n < kSSlice; ++n) {
        const f4_t t = mfma32(pc[j], vc[j][n], f4_t{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] = fmaf(a[i], t[i], o[n][i]);
      }
    }
  }
  // ---- the four waves' sums, added in wave order, divided by L
#pragma unroll
  for (int n = 0; n < kSSlice; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(wave * 16 + 4 * G + i) * OROW + 16 * n + r] = o[n][i];
  }
  __syncthreads();
  {
    const int hh = tid >> 4, c4 = (tid & 15) * 4;
    f4_t v = *reinterpret_cast<const f4_t*>(s_o + hh * OROW + c4);
#pragma unroll
    for (int w = 1; w < 4; ++w) v += *reinterpret_cast<const f4_t*>(s_o + (w * 16 + hh) * OROW + c4);
    const float L = s_l[hh];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float* orow = out + ((size_t)row * kSHeads + hg * 16 + hh) * kSD + sl * 16 * kSSlice + c4;
    *reinterpret_cast<float4*>(orow) = make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    if (lse != nullptr && sl == 0 && (tid & 15) == 0)
      lse[(size_t)row * kSHeads + hg * 16 + hh] = L > 0.0f ? (s_m[hh] + log2f(L)) * 0.69314718055994531f : -INFINITY;
  }
}

// chunks of a row: selection chunks (none without entries), then window chunks
inline int split_sel_chunks(int N, int K) { return (N > 0 && K > 0) ? (K + kKC - 1) / kKC : 0; }
inline int split_win_chunks(int vis) { return (vis + kKC - 1) / kKC; }

}  // namespace

bool attn_split_supported(int H_q, int d, int K, int S, int n_win, bool with_pos, float swa_scale) {
  const int vis = with_pos ? (S < n_win ? S : n_win) : S;  // window tokens a query can see
  return H_q == kSHeads && d == kSD && K <= kSMaxSel && vis <= kSMaxWin && swa_scale > 0.0f &&
         swa_scale <= 128.0f;
}

size_t attn_split_ws_bytes(int rows, int K, int S) {
  // every chunk the launch may use: all selection slots, up to kSMaxWin window tokens
  const int C = (K + kKC - 1) / kKC + split_win_chunks(S < kSMaxWin ? S : kSMaxWin);
  return split_p_bytes(rows, C) + split_ml_bytes(rows, C) + split_v_bytes(rows, C);
}

hipError_t launch_sparse_attn_split(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                    int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                    int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                    float sm_log2, int rows, void* ws, float* out, float* lse,
                                    hipStream_t st) {
  const int vis = q_pos != nullptr ? (S < n_win ? S : n_win) : S;
  const int CS = split_sel_chunks(N, K), C = CS + split_win_chunks(vis);
  char* base = static_cast<char*>(ws);
  uint8_t* pbuf = reinterpret_cast<uint8_t*>(base);
  float2* mlbuf = reinterpret_cast<float2*>(base + split_p_bytes(rows, C));
  uint8_t* vbuf = reinterpret_cast<uint8_t*>(base + split_p_bytes(rows, C) + split_ml_bytes(rows, C));
  // with no keys at all only the second launch runs: zero output, -inf log-sum-exp
  if (C > 0) {
    hipLaunchKernelGGL(attn_split_logits_kernel, dim3(xcd_grid(rows, C)), dim3(kSThreads), 0, st, q,
                       codes, scales, N, sel, K, swa, swa_scale, S, swa_pos0, n_win, q_pos, Tq,
                       sm_log2, rows, CS, C, pbuf, mlbuf, vbuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_split_pv_kernel, dim3(xcd_grid(rows, 4 * kSSlices)), dim3(kSThreads), 0, st,
                     pbuf, mlbuf, vbuf, rows, C, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
