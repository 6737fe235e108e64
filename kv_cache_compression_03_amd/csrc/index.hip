// Indexer scores: s_j = sum_h w_h * max(0, q_h · k_j)  (Full and Reindex modes).
//
// [deep-dive §3.1, §3.2] Indexer Q x Indexer K -> score -> Top-K; Reindex rescores
// only the shared pool [deep-dive §3.3].  Reading: ReLU per head, weighted sum.
//
// The contraction per entry is [h_i x d_i]·[d_i], 16 bf16 flops per byte of key,
// so a decode step is bound by streaming the keys from HBM.  One MFMA
// 16x16x32 bf16 handles 16 entries: A = the query heads (16 rows: 16/h_i
// queries of h_i heads, rows past Tq are zero), B = 16 keys.  Each wave keeps
// its queries in registers for its whole entry range and streams keys straight
// from global memory into the B operand.  The reduction axis is permuted so
// that in MFMA step s the four lane groups of entry e read 64 contiguous bytes
// of key e (16 B each); the queries use the same permutation, so the dot
// products are unchanged.  The ReLU / head-weight / head-sum epilogue runs on the MFMA
// output: a lane holds 4 heads of one query for one entry, and one or two
// cross-lane adds finish the head sum.
//
// Scores leave through non-temporal stores.  They are few beside the keys (4 B
// per query against 256 B per entry) but cost far more than their share: the
// writes, spread thinly through a saturated read stream, made the 8 x 1M scan
// about 12 % slower than the same kernel with its stores removed, and whether a
// wave writes one or two lines per batch made no difference.  The non-temporal
// hint takes 1 % of that back at one query per sequence and 2.5-3 % at three to
// six queries.
#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kScanWaves = 4;
#ifndef CSA2_SCAN_BATCH
#define CSA2_SCAN_BATCH 2
#endif
#ifndef CSA2_SCAN_TARGET_WGS
#define CSA2_SCAN_TARGET_WGS 65536
#endif
constexpr int kScanBatch = CSA2_SCAN_BATCH;  // entry tiles whose keys are in flight together
static_assert(kScanBatch * 16 == kTmaxSpan, "one score maximum per batch of tiles");

// QG query tiles per wave; the launcher uses it with QG = 1 (one query tile per
// sequence row group) and index_scores_mq_kernel below for more.
// TM: also write the maximum of every 16-entry tile of each score row.
template <int HI, int DI, int QG, bool TM>
__global__ __launch_bounds__(kScanWaves * 64, QG == 1 ? 7 : 1) void index_scores_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, const int* __restrict__ gather,
    const int* __restrict__ gather_len, const int* __restrict__ q_pos, int m, int Tq, int N, int L,
    int tiles_per_wave, float* __restrict__ scores, float* __restrict__ tmax) {
  constexpr int QPT = 16 / HI;     // queries per A tile
  constexpr int KS = DI / 32;      // MFMA reduction steps
  // the wave index is uniform: keep it (and the entry range) in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int b = blockIdx.z;
  const int tw0 = blockIdx.y * QG * QPT;   // first query of this workgroup

  // ---- queries (A operands) and head weights, kept for the whole range
  bf16x8_t qa[QG][KS];
  float wr[QG][4];
  int nvis_row[QG];   // entries visible to this lane's query (decode: all)
  bool writer[QG];
  float* srow[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int t0 = tw0 + qg * QPT;
    {
      const int t = t0 + col / HI, h = col % HI;
      const uint4* qrow = reinterpret_cast<const uint4*>(q_idx + (((size_t)b * Tq + t) * HI + h) * DI);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < Tq) v = qrow[s * 4 + g];
        qa[qg][s] = as_bf16x8(v);
      }
    }
    const int myq = t0 + (4 * g) / HI;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i, t = t0 + r / HI;
      wr[qg][i] = t < Tq ? w[((size_t)b * Tq + t) * HI + (r % HI)] : 0.0f;
    }
    nvis_row[qg] = L;
    if (q_pos != nullptr && myq < Tq) {
      long long p = q_pos[(size_t)b * Tq + myq];
      long long nv = (p + 1) / m;
      nvis_row[qg] = (int)(nv < 0 ? 0 : (nv > L ? L : nv));
    }
    writer[qg] = (g % (HI / 4 >= 1 ? HI / 4 : 1)) == 0 && myq < Tq;
    srow[qg] = scores + ((size_t)b * Tq + (myq < Tq ? myq : 0)) * L;
  }
  int Lb = L;
  if (gather_len != nullptr) Lb = min(L, gather_len[b]);

  const long long wave_first = ((long long)blockIdx.x * kScanWaves + wave) * tiles_per_wave * 16;
  const uint16_t* kb = k_idx + (size_t)b * N * DI;
  const int* gb = gather ? gather + (size_t)b * L : nullptr;

  for (int tile = 0; tile < tiles_per_wave; tile += kScanBatch) {
    uint4 kv[kScanBatch][KS];
    int ent[kScanBatch];
    bool ent_ok[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const long long e = wave_first + (long long)(tile + u) * 16 + col;
      ent[u] = (int)e;
      bool live = (tile + u) < tiles_per_wave && e < Lb;
      long long row = e;
      if (live && gb) {
        row = gb[e];
        live = row >= 0 && row < N;  // an entry outside the cache scores -inf
      }
      ent_ok[u] = live;
#pragma unroll
      for (int s = 0; s < KS; ++s) kv[u][s] = make_uint4(0, 0, 0, 0);
      if (live) {
        const uint4* kr = reinterpret_cast<const uint4*>(kb + (size_t)row * DI);
#pragma unroll
        for (int s = 0; s < KS; ++s) kv[u][s] = kr[s * 4 + g];
      }
    }
    float bm[QG];  // TM: this lane's maximum over the batch's tiles, per query tile
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) bm[qg] = -INFINITY;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      if (tile + u >= tiles_per_wave) break;
      const int e = ent[u];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma16x16x32(qa[qg][s], as_bf16x8(kv[u][s]), acc);
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wr[qg][i], fmaxf(acc[i], 0.0f), v);
        if (HI >= 8) v += __shfl_xor(v, 16);
        if (HI >= 16) v += __shfl_xor(v, 32);
        const float sv = (ent_ok[u] && e < nvis_row[qg]) ? v : -INFINITY;
        if (writer[qg] && e < L) __builtin_nontemporal_store(sv, &srow[qg][e]);
        if constexpr (TM) bm[qg] = fmaxf(bm[qg], e < L ? sv : -INFINITY);
      }
    }
    if constexpr (TM) {
      // the maximum of the batch's 32 entries for each query row: the 16 columns
      // of a query are one 16-lane row of the wave
      const int nmt = (L + kTmaxSpan - 1) / kTmaxSpan;
      const int mt = (int)((wave_first + (long long)tile * 16) / kTmaxSpan);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const float tv = row16_max(bm[qg]);
        // query row qi of the tile sits in lane row qi * HI / 4: its maximum is taken
        // to a scalar and stored by lane 0 (uniform addresses, few vector registers)
#pragma unroll
        for (int qi = 0; qi < QPT; ++qi) {
          const int t = tw0 + qg * QPT + qi;
          const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tv), 16 * qi * (HI / 4 >= 1 ? HI / 4 : 1)));
          if (lane == 0 && t < Tq && mt < nmt) tmax[((size_t)b * Tq + t) * nmt + mt] = v;
        }
      }
    }
  }
}

// Waves per SIMD the register budget is sized for (every variant without scratch).
constexpr int scan_occupancy(int HI, int QG, bool TM) {
  return !TM ? (QG == 2 ? 7 : 6) : (QG == 2 ? 5 : (HI == 4 ? 4 : 5));
}

// Several query tiles per wave (QG >= 2: several queries per sequence, e.g.
// drafted positions): each key tile is loaded once and multiplied by all of them.
// The A operands (and head weights) are the same for every wave of the workgroup,
// so they are staged once in LDS instead of each wave holding QG tiles of them in
// registers.  Each wave keeps two key batches in registers (four waves per SIMD):
// the next batch's keys are in flight while the current one is scored.  Key loads
// are issued from clamped addresses and masked after (the only branches around
// them are uniform: whether a wave has a next batch), and the first batch's key
// loads go out before the staging barrier.
// TM: also write the maximum of every 32-entry span of each score row.
template <int HI, int DI, int QG, bool TM>
__global__ __launch_bounds__(kScanWaves * 64, 4) void index_scores_mq_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, const int* __restrict__ gather,
    const int* __restrict__ gather_len, const int* __restrict__ q_pos, int m, int Tq, int N, int L,
    int tiles_per_wave, float* __restrict__ scores, float* __restrict__ tmax) {
  constexpr int QPT = 16 / HI;     // queries per A tile
  constexpr int KS = DI / 32;      // MFMA reduction steps
  static_assert(QG >= 2, "one query tile takes index_scores_kernel");
  constexpr bool QL = true;  // A operands staged in LDS (lane-indexed, 16 bytes per lane and step)
  __shared__ __attribute__((aligned(16))) uint4 s_qa[QL ? QG * KS * 64 : 1];
  __shared__ __attribute__((aligned(16))) float4 s_w[QL ? QG * 64 : 1];  // head weights per lane
  // the wave index is uniform: keep it (and the entry range) in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int b = blockIdx.z;
  const int tw0 = blockIdx.y * QG * QPT;   // first query of this workgroup

  // A operand of query tile qg, step s for lane l: row l%16 of the tile (query
  // t0 + row/HI, head row%HI), reduction slots of group l/16 (16 bytes)
  // (loads are issued unconditionally from a clamped row and masked after, so the
  // staging loads of a thread are all in flight together)
  auto load_qa = [&](int qg, int s, int l) {
    const int t = tw0 + qg * QPT + (l & 15) / HI, h = (l & 15) % HI;
    const uint4 v =
        reinterpret_cast<const uint4*>(q_idx + (((size_t)b * Tq + min(t, Tq - 1)) * HI + h) * DI)[s * 4 + (l >> 4)];
    return t < Tq ? v : make_uint4(0, 0, 0, 0);
  };
  bf16x8_t qa[QL ? 1 : QG][KS];
  if constexpr (QL) {
    constexpr int NQ = (QG * KS * 64 + kScanWaves * 64 - 1) / (kScanWaves * 64);
    uint4 qv[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int i = min((int)threadIdx.x + j * kScanWaves * 64, QG * KS * 64 - 1);
      qv[j] = load_qa(i / (KS * 64), (i / 64) % KS, i % 64);
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int i = threadIdx.x + j * kScanWaves * 64;
      if (i < QG * KS * 64) s_qa[i] = qv[j];
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[0][s] = as_bf16x8(load_qa(0, s, lane));
  }
  // ---- head weights (lane l, element i: row 4(l/16) + i of the tile), visibility
  // and output rows, kept for the whole range (the weights in LDS with the queries
  // when there are several query tiles)
  auto load_w = [&](int qg, int l) {
    float4 v;
    float* vp = reinterpret_cast<float*>(&v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * (l >> 4) + i, t = tw0 + qg * QPT + r / HI;
      const float x = w[((size_t)b * Tq + min(t, Tq - 1)) * HI + (r % HI)];
      vp[i] = t < Tq ? x : 0.0f;
    }
    return v;
  };
  float4 wr[QL ? 1 : QG];
  if constexpr (QL) {
    constexpr int NW = (QG * 64 + kScanWaves * 64 - 1) / (kScanWaves * 64);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int i = threadIdx.x + j * kScanWaves * 64;
      const float4 v = load_w(min(i, QG * 64 - 1) / 64, i % 64);
      if (i < QG * 64) s_w[i] = v;
    }
  } else {
    wr[0] = load_w(0, lane);
  }
  int nvis_row[QG];   // entries visible to this lane's query (decode: all)
  bool writer[QG];
  const int myq0 = tw0 + (4 * g) / HI;  // this lane's query in tile 0; tile qg adds qg*QPT
  float* const srow0 = scores + ((size_t)b * Tq + myq0) * L;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int myq = myq0 + qg * QPT;
    nvis_row[qg] = L;
    if (q_pos != nullptr && myq < Tq) {
      long long p = q_pos[(size_t)b * Tq + myq];
      long long nv = (p + 1) / m;
      nvis_row[qg] = (int)(nv < 0 ? 0 : (nv > L ? L : nv));
    }
    writer[qg] = (g % (HI / 4 >= 1 ? HI / 4 : 1)) == 0 && myq < Tq;
  }
  int Lb = L;
  if (gather_len != nullptr) Lb = min(L, gather_len[b]);

  const long long wave_first = ((long long)blockIdx.x * kScanWaves + wave) * tiles_per_wave * 16;
  const uint16_t* kb = k_idx + (size_t)b * N * DI;
  const int* gb = gather ? gather + (size_t)b * L : nullptr;

  // the keys of a batch (two 16-entry tiles): dead entries read row 0 (their
  // scores are masked), so every path issues the same loads
  struct KeyBatch {
    uint4 kv[kScanBatch][KS];
    bool ok[kScanBatch];
  };
  auto load_batch = [&](int tile, KeyBatch& kt) {
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const long long e = wave_first + (long long)(tile + u) * 16 + col;
      bool live = (tile + u) < tiles_per_wave && e < Lb;
      long long row = e;
      if (gb) {  // uniform: the gathered row of every slot is read, masked after
        row = gb[min(e, (long long)L - 1)];
        live = live && row >= 0 && row < N;  // an entry outside the cache scores -inf
      }
      kt.ok[u] = live;
      const uint4* kr = reinterpret_cast<const uint4*>(kb + (size_t)(live ? row : 0) * DI);
#pragma unroll
      for (int s = 0; s < KS; ++s) kt.kv[u][s] = kr[s * 4 + g];
    }
  };
  auto score_batch = [&](int tile, const KeyBatch& kt) {
    // TM: the maximum of the batch's 32 entries for each query row goes out per
    // query tile (the 16 columns of a query are one 16-lane row of the wave)
    const int nmt = (L + kTmaxSpan - 1) / kTmaxSpan;
    const int mt = (int)((wave_first + (long long)tile * 16) / kTmaxSpan);
    // the staged A operands are re-read every batch (an opaque index keeps the
    // compiler from hoisting all of them into registers)
    int qli = lane;
    asm volatile("" : "+v"(qli));
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      // both tiles of the batch against query tile qg: each A operand read once
      f32x4_t acc[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t a = QL ? as_bf16x8(s_qa[(qg * KS + s) * 64 + qli]) : qa[0][s];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) acc[u] = mfma16x16x32(a, as_bf16x8(kt.kv[u][s]), acc[u]);
      }
      const float4 wq = QL ? s_w[qg * 64 + qli] : wr[0];
      const float wv[4] = {wq.x, wq.y, wq.z, wq.w};
      float bm = -INFINITY;  // TM: this lane's maximum over the batch's tiles
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (tile + u >= tiles_per_wave) break;
        const int e = (int)(wave_first + (long long)(tile + u) * 16 + col);
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wv[i], fmaxf(acc[u][i], 0.0f), v);
        if (HI >= 8) v += __shfl_xor(v, 16);
        if (HI >= 16) v += __shfl_xor(v, 32);
        const float sv = (kt.ok[u] && e < nvis_row[qg]) ? v : -INFINITY;
        if (writer[qg] && e < L) __builtin_nontemporal_store(sv, &srow0[(size_t)qg * QPT * L + e]);
        if constexpr (TM) bm = fmaxf(bm, e < L ? sv : -INFINITY);
      }
      if constexpr (TM) {
        const float tv = row16_max(bm);
        // query row qi of the tile sits in lane row qi * HI / 4: its maximum is taken
        // to a scalar and stored by lane 0 (uniform addresses, few vector registers)
#pragma unroll
        for (int qi = 0; qi < QPT; ++qi) {
          const int t = tw0 + qg * QPT + qi;
          const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tv), 16 * qi * (HI / 4 >= 1 ? HI / 4 : 1)));
          if (lane == 0 && t < Tq && mt < nmt) tmax[((size_t)b * Tq + t) * nmt + mt] = v;
        }
      }
    }
  };
  // two batches in registers: the next one's keys are in flight while the current
  // one is scored (the trip count is the same for every wave)
  KeyBatch b0, b1;
  load_batch(0, b0);
  // the staged queries are complete once every wave has passed here; the first
  // batch's key loads are already in flight
  if constexpr (QL) __syncthreads();
  for (int tile = 0; tile < tiles_per_wave; tile += 2 * kScanBatch) {
    const bool has1 = tile + kScanBatch < tiles_per_wave;
    if (has1) load_batch(tile + kScanBatch, b1);
    score_batch(tile, b0);
    if (tile + 2 * kScanBatch < tiles_per_wave) load_batch(tile + 2 * kScanBatch, b0);
    if (has1) score_batch(tile + kScanBatch, b1);
  }
}


// One query per sequence over long rows (at least kPersMinL entries): one
// workgroup per CU holds the scores it computes in LDS while its keys stream in
// and writes them in one burst at the end.  Score writes spread thinly through
// the key stream cost far more than their bytes (about 12 % of the 8 x 1M scan);
// written at the end they cost about their bytes, and the scores the selection
// kernels read next are still in the memory-side cache.  The 32-entry batches are
// dealt round robin over the whole grid (batch F to workgroup F mod G), so all
// CUs move through the keys together, as the one-shot waves of the other scan do
// (a contiguous share per workgroup, 256 streams at once, was 7 % slower).  Each
// wave prefetches its next batch while it scores the current one; its batches
// change sequence only every L/32/G of them, and the query is reloaded then.
// Measured against index_scores_kernel: 8 x 1M 346 vs 350-385 us, equal at 512K
// and 256K per row, 4 % slower at 128K and below (the query reloads), hence
// kPersMinL.
constexpr int kPersThreads = 1024;
constexpr int kPersWaves = kPersThreads / 64;
constexpr int kPersMaxBatches = 1152;   // 32-entry batches a workgroup holds (144 KB of LDS)
constexpr int kPersMinL = 1 << 19;

template <int HI, int DI, bool TM>
__global__ __launch_bounds__(kPersThreads, 1) void index_scores_persist_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, const int* __restrict__ q_pos, int m, int N, int L,
    int nbat, float* __restrict__ scores, float* __restrict__ tmax) {
  static_assert(kScanBatch == 2 && kTmaxSpan == 32, "32-entry batches of two 16-key tiles");
  constexpr int KS = DI / 32;
  __shared__ __attribute__((aligned(16))) float s_sc[kPersMaxBatches * 32];
  __shared__ float s_tm[kPersMaxBatches];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int G = gridDim.x, wg = blockIdx.x;
  const int bpr = L / 32;                       // batches per sequence
  const int nloc = (nbat - wg + G - 1) / G;     // local slots: batch wg + G t, t < nloc
  // lane group 0 holds query 0's score of each key after the head sum
  const bool writer = g == 0;

  // the query of the current sequence: A row col = head col (rows past h_i zero)
  int bq = -1, nvis = L;
  bf16x8_t qa[KS];
  float wq[4];
  auto set_seq = [&](int b) {
    const uint4* qrow = reinterpret_cast<const uint4*>(q_idx + ((size_t)b * HI + (col < HI ? col : 0)) * DI);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = qrow[s * 4 + g];
      qa[s] = as_bf16x8(col < HI ? v : make_uint4(0, 0, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const float x = w[(size_t)b * HI + (r < HI ? r : 0)];
      wq[i] = r < HI ? x : 0.0f;
    }
    nvis = L;
    if (q_pos != nullptr) {
      const long long p = q_pos[b];
      const long long nv = (p + 1) / m;
      nvis = (int)(nv < 0 ? 0 : (nv > L ? L : nv));
    }
    bq = b;
  };
  struct Batch {
    uint4 kv[kScanBatch][KS];
  };
  // keys of local slot t (past the last slot: the last one again, masked later)
  auto load = [&](int t, Batch& bt) {
    const int F = wg + G * min(t, nloc - 1);
    const int b = F / bpr, e = (F - b * bpr) * 32;
    const uint16_t* kb = k_idx + (size_t)b * N * DI;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const uint4* kr = reinterpret_cast<const uint4*>(kb + (size_t)(e + 16 * u + col) * DI);
#pragma unroll
      for (int s = 0; s < KS; ++s) bt.kv[u][s] = kr[s * 4 + g];
    }
  };
  auto score = [&](int t, const Batch& bt) {
    const bool live = t < nloc;
    const int F = wg + G * min(t, nloc - 1);
    const int b = F / bpr, e = (F - b * bpr) * 32;
    if (b != bq) set_seq(b);  // uniform
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma16x16x32(qa[s], as_bf16x8(bt.kv[u][s]), acc);
      float v = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaf(wq[i], fmaxf(acc[i], 0.0f), v);
      if (HI >= 8) v += __shfl_xor(v, 16);
      if (HI >= 16) v += __shfl_xor(v, 32);
      const float sv = (e + 16 * u + col < nvis) ? v : -INFINITY;
      if (writer && live) s_sc[32 * t + 16 * u + col] = sv;
      if constexpr (TM) bm = fmaxf(bm, sv);
    }
    if constexpr (TM) {
      const float tv = row16_max(bm);  // query 0's maximum sits in lane 0
      if (lane == 0 && live) s_tm[t] = tv;
    }
  };

  Batch b0, b1;
  load(wave, b0);
  for (int t = wave; t < nloc; t += 2 * kPersWaves) {
    load(t + kPersWaves, b1);
    score(t, b0);
    load(t + 2 * kPersWaves, b0);
    score(t + kPersWaves, b1);
  }
  __syncthreads();
  // slot t holds batch F = wg + G t, whose 32 scores sit at F * 32 (Tq = 1)
  for (int i = threadIdx.x; i < nloc * 8; i += kPersThreads) {
    const int t = i >> 3, k = (i & 7) * 4;
    const size_t F = (size_t)wg + (size_t)G * t;
    *reinterpret_cast<float4*>(scores + F * 32 + k) = *reinterpret_cast<const float4*>(s_sc + 32 * t + k);
  }
  if constexpr (TM) {
    for (int t = threadIdx.x; t < nloc; t += kPersThreads) tmax[(size_t)wg + (size_t)G * t] = s_tm[t];
  }
}

// compute units of the current device (looked up once per device)
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_index_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                               const int* gather, const int* gather_len, const int* q_pos, int m,
                               int B, int Tq, int N, int L, int h_i, int d_i, float* scores,
                               hipStream_t st, float* tmax) {
  if (B == 0 || Tq == 0 || L == 0) return hipSuccess;
  if (tmax == nullptr && L == N && index_prefill_supported(Tq, N, h_i, d_i, gather))
    return launch_index_prefill(q_idx, w, k_idx, q_pos, m, B, Tq, N, h_i, d_i, scores, st);
  // one query per sequence over long rows: the LDS-held scan
  const int cus = device_cus();
  const long long nbat = (long long)B * (L / 32);
  if (Tq == 1 && gather == nullptr && L == N && L % 32 == 0 && L >= kPersMinL && cus > 0 &&
      nbat >= cus && nbat <= (long long)cus * kPersMaxBatches &&
      (reinterpret_cast<uintptr_t>(scores) & 15) == 0) {
#define CSA2_PERS(HI_, DI_)                                                                        \
  do {                                                                                             \
    if (tmax)                                                                                      \
      hipLaunchKernelGGL((index_scores_persist_kernel<HI_, DI_, true>), dim3(cus), dim3(kPersThreads), \
                         0, st, q_idx, w, k_idx, q_pos, m, N, L, (int)nbat, scores, tmax);          \
    else                                                                                           \
      hipLaunchKernelGGL((index_scores_persist_kernel<HI_, DI_, false>), dim3(cus), dim3(kPersThreads), \
                         0, st, q_idx, w, k_idx, q_pos, m, N, L, (int)nbat, scores, tmax);          \
  } while (0)
    if (h_i == 8 && d_i == 128) CSA2_PERS(8, 128);
    else if (h_i == 8 && d_i == 64) CSA2_PERS(8, 64);
    else if (h_i == 4 && d_i == 128) CSA2_PERS(4, 128);
    else if (h_i == 4 && d_i == 64) CSA2_PERS(4, 64);
    else if (h_i == 16 && d_i == 128) CSA2_PERS(16, 128);
    else CSA2_PERS(16, 64);
#undef CSA2_PERS
    return hipGetLastError();
  }
  const int qpt = 16 / h_i;
  const int qtiles = (Tq + qpt - 1) / qpt;
  // query tiles per wave: every key tile is read once for up to four of them
  const int qg = qtiles >= 4 ? 4 : qtiles;
  const int qgroups = (qtiles + qg - 1) / qg;
  const long long tiles = ((long long)L + 15) / 16;
  // aim for about CSA2_SCAN_TARGET_WGS workgroups, at most 32 tiles (512 entries) per wave
#ifndef CSA2_MQ_TARGET_DIV
#define CSA2_MQ_TARGET_DIV 4
#endif
  const long long target = qg >= 2 ? CSA2_SCAN_TARGET_WGS / CSA2_MQ_TARGET_DIV : CSA2_SCAN_TARGET_WGS;
  long long per_wave = ((long long)tiles * B * qgroups + target * kScanWaves - 1) / (target * kScanWaves);
  int tpw = (int)(per_wave < 1 ? 1 : (per_wave > 32 ? 32 : per_wave));
  tpw = (tpw + kScanBatch - 1) / kScanBatch * kScanBatch;
  const long long bx = (tiles + (long long)tpw * kScanWaves - 1) / ((long long)tpw * kScanWaves);
  dim3 grid((unsigned)bx, (unsigned)qgroups, (unsigned)B), block(kScanWaves * 64);
#define CSA2_SCAN_K(KERN_, HI_, DI_, QG_)                                                                \
  do {                                                                                                  \
    if (tmax)                                                                                           \
      hipLaunchKernelGGL((KERN_<HI_, DI_, QG_, true>), grid, block, 0, st, q_idx, w, k_idx, gather,    \
                         gather_len, q_pos, m, Tq, N, L, tpw, scores, tmax);                            \
    else                                                                                                \
      hipLaunchKernelGGL((KERN_<HI_, DI_, QG_, false>), grid, block, 0, st, q_idx, w, k_idx, gather,   \
                         gather_len, q_pos, m, Tq, N, L, tpw, scores, tmax);                            \
  } while (0)
#define CSA2_SCAN(HI_, DI_)                                           \
  do {                                                                \
    if (qg == 1) CSA2_SCAN_K(index_scores_kernel, HI_, DI_, 1);       \
    else if (qg == 2) CSA2_SCAN_K(index_scores_mq_kernel, HI_, DI_, 2); \
    else if (qg == 3) CSA2_SCAN_K(index_scores_mq_kernel, HI_, DI_, 3); \
    else CSA2_SCAN_K(index_scores_mq_kernel, HI_, DI_, 4);            \
  } while (0)
  if (h_i == 8 && d_i == 128) CSA2_SCAN(8, 128);
  else if (h_i == 8 && d_i == 64) CSA2_SCAN(8, 64);
  else if (h_i == 4 && d_i == 128) CSA2_SCAN(4, 128);
  else if (h_i == 4 && d_i == 64) CSA2_SCAN(4, 64);
  else if (h_i == 16 && d_i == 128) CSA2_SCAN(16, 128);
  else CSA2_SCAN(16, 64);
#undef CSA2_SCAN
#undef CSA2_SCAN_K
  return hipGetLastError();
}

}  // namespace csa2
