// Indexer scores of many queries at once (prefill): a causal bf16 contraction on
// MFMA.  s_{t,j} = sum_h w_{t,h} * max(0, q_{t,h} · k_j) for every entry j visible
// to query t (p_j <= t), -inf for the others.
//
// [deep-dive §3.1, §3.3] the indexer scores every visible entry of every query;
// with thousands of queries the scores form a dense [Tq*h_i, d_i] x [d_i, N]
// product (rows = (query, head) pairs), so this is MFMA work.
//
// A workgroup owns 256 rows (256 / h_i queries) and a range of keys.  Each of
// its four waves keeps its 64 rows of Q in registers (the A operands) for the
// whole range; the keys pass through LDS in tiles of 64, double-buffered, each
// staged once and read by all four waves as B operands.  Per tile a wave runs
// 4 row tiles x 4 key tiles x d_i/32 MFMA 16x16x32 steps.  Rows are assigned
// so that a group of h_i/4 row tiles holds 4 queries: row 4q + i of the group's
// tile u is head 4u + i of query q.  An MFMA output lane (lane group g, key
// column c) then holds, across the group's tiles, every head of query g for
// key c, and applies ReLU, the head weights, the head sum and the causal mask
// on its own before storing the score.
// Key tiles that no query of the workgroup can see are filled with -inf
// without any MFMA.
#include "common.h"
#include "internal.h"

namespace csa2 {

// cache-policy operand of a buffer store on gfx950: non-temporal (streaming)
constexpr int kStoreNonTemporal = 2;

constexpr int kPfWaves = 4;
constexpr int kPfRows = 256;  // (query, head) rows per workgroup, 64 per wave
constexpr int kPfKeys = 64;   // keys per staged tile
constexpr int kOutOfRange = 0x7FFFFFF0;      // a byte offset past any score buffer of this kernel
#ifndef CSA2_PF_SPLIT
#define CSA2_PF_SPLIT 4096    // keys per workgroup
#endif

// max(x, 0) in one integer instruction: a float with the sign bit set is a
// negative int32 (that includes -0), any other float keeps its bits.  (fmaxf
// would first quiet a NaN input, one more instruction per element.)
CSA2_DEV float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int HI, int DI>
__global__ __launch_bounds__(kPfWaves * 64, 2) void index_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, const int* __restrict__ q_pos, int m, int Tq, int N,
    float* __restrict__ scores) {
  constexpr int QPW = kPfRows / HI;         // queries per workgroup
  constexpr int TPG = HI / 4;               // row tiles per group of 4 queries
  constexpr int KS = DI / 32;               // MFMA reduction steps
  constexpr int RT = 4;                     // 16-row tiles per wave
  constexpr int CT = kPfKeys / 16;          // 16-key tiles per staged tile
  constexpr int KP = DI + 8;                // staged key pitch (bf16): 16 B pad, conflict-free reads
  constexpr int CPK = DI / 8;               // 16-byte chunks per key
  constexpr int CPT = kPfKeys * CPK / (kPfWaves * 64);  // chunks each thread stages
  constexpr int NG = RT / TPG;              // query groups per wave
  static_assert(TPG >= 1 && TPG <= 4 && RT % TPG == 0, "h_i must be 4, 8 or 16");
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kPfKeys * KP];
  __shared__ int s_vmax[kPfWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, g = lane >> 4;
  const int b = blockIdx.z;
  const int qb0 = blockIdx.y * QPW;
  const int key_lo = blockIdx.x * CSA2_PF_SPLIT;
  const int key_hi = min(N, key_lo + CSA2_PF_SPLIT);

  // ---- A operands: row r of row tile rt (rt = group * TPG + u) is head 4u + r%4 of
  // query 64*wave/HI + 4*group + r/4; the reduction slots of step s, lane group
  // g are dims 32s + 8g .. 32s + 8g + 7
  const int wq0 = qb0 + (64 * wave) / HI;  // first query of this wave
  bf16x8_t qa[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int t = wq0 + 4 * (rt / TPG) + col / 4;
    const int h = 4 * (rt % TPG) + col % 4;
    const uint4* qr =
        reinterpret_cast<const uint4*>(q_idx + (((size_t)b * Tq + min(t, Tq - 1)) * HI + h) * DI);
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[rt][s] = as_bf16x8(t < Tq ? qr[4 * s + g] : make_uint4(0, 0, 0, 0));
  }
  // Wait for Q here, once: otherwise the wait for it lands inside the key loop,
  // where it would also wait for that loop's score stores.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(qa[rt][s]));
  // ---- output side: in group n, lane group g holds query wq0 + 4n + g; element i of
  // its tile u is head 4u + i
  float wv[NG][TPG][4];
  int nv[NG];
  int vmax = 0;
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    const int t = wq0 + 4 * n + g;
    const bool live = t < Tq;
    const size_t qrow = (size_t)b * Tq + (live ? t : 0);
#pragma unroll
    for (int u = 0; u < TPG; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[n][u][i] = live ? w[qrow * HI + 4 * u + i] : 0.0f;
    int c = 0;
    if (live) {
      if (q_pos != nullptr) {
        const long long v = ((long long)q_pos[qrow] + 1) / m;  // entries with p_j <= t
        c = (int)(v < 0 ? 0 : (v > N ? N : v));
      } else {
        c = N;
      }
    }
    nv[n] = c;
    vmax = max(vmax, c);
  }
  // the same for the head weights and visible counts (loaded before the loop)
#pragma unroll
  for (int n = 0; n < NG; ++n) {
#pragma unroll
    for (int u = 0; u < TPG; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(wv[n][u][i]));
    asm volatile("" : "+v"(nv[n]));
  }
  int vmin = N;  // the fewest entries any of the wave's queries sees (rows past Tq: all N)
#pragma unroll
  for (int n = 0; n < NG; ++n) vmin = min(vmin, wq0 + 4 * n + g < Tq ? nv[n] : N);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    vmax = max(vmax, __shfl_xor(vmax, o));
    vmin = min(vmin, __shfl_xor(vmin, o));
  }
  vmin = __builtin_amdgcn_readfirstlane(vmin);
  if (lane == 0) s_vmax[wave] = vmax;
  // The workgroup's score rows as one raw buffer: a store whose offset falls
  // outside it is dropped by the hardware range check, so masked lanes (keys
  // past N, rows past Tq) are given an out-of-range offset and no store sits
  // behind a branch.
  const int rows_here = min(QPW, Tq - qb0);
  const __amdgpu_buffer_rsrc_t srsc = __builtin_amdgcn_make_buffer_rsrc(
      scores + ((size_t)b * Tq + qb0) * N, (short)0, rows_here * N * (int)sizeof(float), kRawBufferWord3);
  int roff[NG];  // byte offset of this lane's query row in the buffer, per group
#pragma unroll
  for (int n = 0; n < NG; ++n) roff[n] = (wq0 - qb0 + 4 * n + g) * N * (int)sizeof(float);

  // staging of key tile `tile`: thread tid moves 16-byte chunks tid + u*256
  // (key c / CPK, dims (c % CPK)*8 ..) through registers into LDS.  The keys are
  // read through a buffer descriptor over the sequence's keys: the per-thread byte
  // offset is fixed, the tile's offset is one uniform value, and keys past N read
  // as zeros (their scores are masked).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 stg[CPT];
  const __amdgpu_buffer_rsrc_t krsc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(k_idx) + (size_t)b * N * DI, (short)0, N * DI * (int)sizeof(uint16_t), kRawBufferWord3);
#define CSA2_PF_FETCH(tile_)                                                                   \
  _Pragma("unroll") for (int u = 0; u < CPT; ++u) {                                            \
    const int c = tid + u * (kPfWaves * 64);                                                   \
    stg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(                  \
        krsc, ((c / CPK) * DI + (c % CPK) * 8) * (int)sizeof(uint16_t),                        \
        (key_lo + (tile_) * kPfKeys) * DI * (int)sizeof(uint16_t), 0));                        \
  }
#define CSA2_PF_STASH(buf_)                                                                    \
  _Pragma("unroll") for (int u = 0; u < CPT; ++u) {                                            \
    const int c = tid + u * (kPfWaves * 64);                                                   \
    *reinterpret_cast<u32x4*>(&kt[(buf_)][(c / CPK) * KP + (c % CPK) * 8]) = stg[u];           \
  }

  __syncthreads();  // s_vmax
  const int vis = min(key_hi, max(max(s_vmax[0], s_vmax[1]), max(s_vmax[2], s_vmax[3])));
  const int n_comp = vis > key_lo ? (vis - key_lo + kPfKeys - 1) / kPfKeys : 0;

  // Pipeline: tile t is multiplied from LDS buffer t&1; at the end of the pass tile
  // t+1 (whose loads were issued at the end of the previous pass) is stashed into
  // the other buffer and tile t+2's loads are issued, to fly during the next pass.
  // Stash and fetch run on every pass, clamped to the last tile, and every path
  // into the stash has the same loads and score stores before it, so its wait
  // covers the loads only.
  if (n_comp > 0) {
    CSA2_PF_FETCH(0)
    CSA2_PF_STASH(0)
    CSA2_PF_FETCH(min(1, n_comp - 1))
  }
  lds_barrier();
  for (int tile = 0; tile < n_comp; ++tile) {
    const int buf = tile & 1;
    f32x4_t acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the B operands of key tile ct+1 are read from LDS while the MFMAs of key tile
    // ct run (the schedule below holds them in that order)
    const uint16_t* kbase = &kt[buf][col * KP + 8 * g];
    bf16x8_t kb[2][KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) kb[0][s] = *reinterpret_cast<const bf16x8_t*>(kbase + 32 * s);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (ct + 1 < CT) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          kb[(ct + 1) & 1][s] = *reinterpret_cast<const bf16x8_t*>(kbase + 16 * (ct + 1) * KP + 32 * s);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][ct] = mfma16x16x32(qa[rt][s], kb[ct & 1][s], acc[rt][ct]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // LDS reads of key tile 0
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (ct + 1 < CT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one read ahead
        __builtin_amdgcn_sched_group_barrier(0x008, RT, 0);                  // RT MFMAs
      }
    // ---- epilogue: ReLU, head weights, head sum, causal mask (all within the lane);
    // the stores follow the branch, so every path issues the same number of them
    const int key0 = key_lo + tile * kPfKeys;
    float pv[NG][CT];
    int of[NG][CT];
#pragma unroll
    for (int n = 0; n < NG; ++n)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float p = 0.0f;
#pragma unroll
        for (int u = 0; u < TPG; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) p = fmaf(wv[n][u][i], relu(acc[n * TPG + u][ct][i]), p);
        pv[n][ct] = p;
      }
    if (key0 + kPfKeys <= vmin) {
      // every key of the tile is visible to every query of the wave (and below N)
#pragma unroll
      for (int n = 0; n < NG; ++n) {
        const int base = roff[n] + (key0 + col) * (int)sizeof(float);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) of[n][ct] = base + 64 * ct;
      }
    } else {
#pragma unroll
      for (int n = 0; n < NG; ++n)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int j = key0 + 16 * ct + col;
          of[n][ct] = j < N ? roff[n] + j * (int)sizeof(float) : kOutOfRange;
          if (j >= nv[n]) pv[n][ct] = -INFINITY;
        }
    }
    // streaming stores (non-temporal): the scores of a chunk are far larger than
    // the caches, and keeping them out leaves L2 to the keys every query block
    // re-reads (-2.5 % per launch measured)
#pragma unroll
    for (int n = 0; n < NG; ++n)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pv[n][ct]), srsc, of[n][ct], 0, kStoreNonTemporal);
    __builtin_amdgcn_sched_barrier(0);  // stash after the stores
    // buffer buf^1 was last read in pass tile-1, before that pass's barrier
    CSA2_PF_STASH(buf ^ 1)
    CSA2_PF_FETCH(min(tile + 2, n_comp - 1))
    lds_barrier();
  }
#undef CSA2_PF_FETCH
#undef CSA2_PF_STASH
  // ---- key tiles no query of this workgroup can see
  const int tail = key_lo + n_comp * kPfKeys;
  if (tail < key_hi) {
    for (int qq = 0; qq < QPW; ++qq) {
      const int t = qb0 + qq;
      if (t >= Tq) break;
      float* r = scores + ((size_t)b * Tq + t) * N;
      for (int j = tail + tid; j < key_hi; j += kPfWaves * 64) r[j] = -INFINITY;
    }
  }
}

bool index_prefill_supported(int Tq, int N, int h_i, int d_i, const int* gather) {
  // a workgroup's score rows (at most 64 of N floats) must fit one raw buffer below
  // kOutOfRange, and a sequence's keys one buffer descriptor
  return gather == nullptr && (long long)Tq * h_i >= kPfRows && (h_i == 4 || h_i == 8 || h_i == 16) &&
         (d_i == 64 || d_i == 128) && (long long)(kPfRows / 4) * N * sizeof(float) < kOutOfRange &&
         (long long)N * d_i * 2 < (1ll << 31);
}

hipError_t launch_index_prefill(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                const int* q_pos, int m, int B, int Tq, int N, int h_i, int d_i,
                                float* scores, hipStream_t st) {
  if (B == 0 || Tq == 0 || N == 0) return hipSuccess;
  const int qpw = kPfRows / h_i;
  dim3 grid((unsigned)((N + CSA2_PF_SPLIT - 1) / CSA2_PF_SPLIT), (unsigned)((Tq + qpw - 1) / qpw),
            (unsigned)B),
      block(kPfWaves * 64);
#define CSA2_PF(HI_, DI_)                                                                      \
  hipLaunchKernelGGL((index_prefill_kernel<HI_, DI_>), grid, block, 0, st, q_idx, w, k_idx, q_pos, \
                     m, Tq, N, scores)
  if (h_i == 8 && d_i == 128) CSA2_PF(8, 128);
  else if (h_i == 8 && d_i == 64) CSA2_PF(8, 64);
  else if (h_i == 4 && d_i == 128) CSA2_PF(4, 128);
  else if (h_i == 4 && d_i == 64) CSA2_PF(4, 64);
  else if (h_i == 16 && d_i == 128) CSA2_PF(16, 128);
  else CSA2_PF(16, 64);
#undef CSA2_PF
  return hipGetLastError();
}

}  // namespace csa2
