// Top-K selection and the shared candidate pool.
//
// [deep-dive §3.3] the first Full indexer scans the whole visible range, keeps
// the best positions of each block and a Top-512; the pool of 2,048 blocks x 8
// positions is shared by later Reindex layers.  Readings: rank by (score desc,
// index asc), output ascending and -1 padded; a block is G consecutive entries
// scored by its maximum; the PB best blocks (ties: lower block) give their PE
// best entries (ties: lower index).
//
// Every ordering is decided on one 64-bit key, (order-preserving bits of the
// score) << 32 | (0xFFFFFFFF - index): keys are unique, larger is better, and
// the score ties break to the lower index.
//
// Rows with at most kTopkCap visible entries are selected whole in LDS (one
// 1024-thread workgroup per row: radix select of the K-th key, then ranks).  Rows
// of up to kRowCap entries are thinned to candidates inside that same workgroup
// (below).  Longer rows (decode over 64K-1M entries, a handful of rows) first go
// through two wide passes:
//   chunkmax: split the row into C >= K chunks and take each chunk's maximum;
//   filter:   T = min of the chunk maxima.  Those C maxima are C distinct entries
//             scoring >= T, so the K-th best score is >= T and every entry below
//             T can be dropped; entries >= T are appended to a candidate list.
// For continuous scores about K*ln(K) (~3.2K for K = 512) entries survive.  If
// more than kTopkCap survive (heavy ties), the row falls back to an exact radix
// select over the whole row in one workgroup (slow, correct).
#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kSelThreads = 1024;

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Calls whose rows hold at most kRowCap entries run the one-pass row kernel
// (no workspace); longer rows take the two wide passes first.
constexpr int kRowCap = 16384;

size_t topk_ws_bytes(int R, int N, int K) {
  if (N <= kRowCap) return 0;
  size_t b = 0;
  b += align256((size_t)R * 2 * K * sizeof(float));
  b += align256((size_t)R * sizeof(int));
  b += align256((size_t)R * kTopkCap * sizeof(float));
  b += align256((size_t)R * kTopkCap * sizeof(int));
  return b;
}

TopkWs topk_ws_carve(void* ws, int R, int K) {
  char* p = static_cast<char*>(ws);
  TopkWs w;
  w.cmax = reinterpret_cast<float*>(p);
  p += align256((size_t)R * 2 * K * sizeof(float));
  w.cnt = reinterpret_cast<int*>(p);
  p += align256((size_t)R * sizeof(int));
  w.cscore = reinterpret_cast<float*>(p);
  p += align256((size_t)R * kTopkCap * sizeof(float));
  w.cidx = reinterpret_cast<int*>(p);
  return w;
}

CSA2_DEV int row_len(const int* valid_len, int r, int N) {
  if (!valid_len) return N;
  int v = valid_len[r];
  return v < 0 ? 0 : (v > N ? N : v);
}

CSA2_DEV unsigned long long make_key(float s, int idx) {
  return ((unsigned long long)mono_key(s) << 32) | (0xFFFFFFFFu - (uint32_t)idx);
}
CSA2_DEV int key_index(unsigned long long k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

// ---------------------------------------------------------------- wide passes

constexpr int kChunksPerWave = 4;

// Short chunks (<= 128 entries): one wave per kChunksPerWave consecutive chunks,
// every load requested together.  Long chunks: one wave per chunk, 8 loads per
// lane in flight.
__global__ __launch_bounds__(256) void topk_chunkmax_kernel(const float* __restrict__ scores, int N,
                                                            const int* __restrict__ valid_len, int K,
                                                            int cpw, float* __restrict__ cmax,
                                                            int* __restrict__ cnt) {
  const int r = blockIdx.y;
  const int n = row_len(valid_len, r, N);
  if (n <= kTopkCap) return;
  if (blockIdx.x == 0 && threadIdx.x == 0) cnt[r] = 0;
  const int clen = n / K;  // >= 4 because n > kTopkCap >= 4K
  const int C = (n + clen - 1) / clen;
  const int c0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * cpw;
  if (c0 >= C) return;
  const int lane = threadIdx.x & 63;
  const float* row = scores + (size_t)r * N;
  if (cpw == 1) {
    const int lo = c0 * clen, hi = min(lo + clen, n);
    float mx = -INFINITY;
#pragma unroll 8
    for (int i = lo + lane; i < hi; i += 64) mx = fmaxf(mx, row[i]);
    mx = wave_max(mx);
    if (lane == 0) cmax[(size_t)r * 2 * K + c0] = mx;
    return;
  }
  float v[kChunksPerWave][2];
#pragma unroll
  for (int j = 0; j < kChunksPerWave; ++j) {
    const int lo = (c0 + j) * clen, hi = min(lo + clen, n);
    v[j][0] = c0 + j < C && lo + lane < hi ? row[lo + lane] : -INFINITY;
    v[j][1] = c0 + j < C && lo + 64 + lane < hi ? row[lo + 64 + lane] : -INFINITY;
  }
#pragma unroll
  for (int j = 0; j < kChunksPerWave; ++j) {
    if (c0 + j >= C) break;
    const int lo = (c0 + j) * clen, hi = min(lo + clen, n);
    float mx = fmaxf(v[j][0], v[j][1]);
    for (int i = lo + 128 + lane; i < hi; i += 64) mx = fmaxf(mx, row[i]);
    mx = wave_max(mx);
    if (lane == 0) cmax[(size_t)r * 2 * K + c0 + j] = mx;
  }
}

// Entries per filter thread: more for long rows, so fewer workgroups contend for
// a row's candidate counter.
template <int PER>
__global__ __launch_bounds__(256) void topk_filter_kernel(const float* __restrict__ scores, int N,
                                                          const int* __restrict__ valid_len, int K,
                                                          const float* __restrict__ cmax,
                                                          int* __restrict__ cnt,
                                                          float* __restrict__ cscore,
                                                          int* __restrict__ cidx) {
  const int r = blockIdx.y;
  const int n = row_len(valid_len, r, N);
  if (n <= kTopkCap) return;
  const long long e0 = (long long)blockIdx.x * 256 * PER;
  if (e0 >= n) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int clen = n / K;
  const int C = (n + clen - 1) / clen;
  __shared__ float red[4];
  __shared__ int wsum[4];
  __shared__ int base;
  // this thread's scores and (C <= 2K <= 4096) chunk maxima, all requested at once
  const float* row = scores + (size_t)r * N;
  float sv[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const long long e = e0 + it * 256 + tid;
    sv[it] = e < n ? row[e] : 0.0f;
  }
  float mn = INFINITY;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int c = tid + 256 * u;
    if (c < C) mn = fminf(mn, cmax[(size_t)r * 2 * K + c]);
  }
  mn = wave_min(mn);
  if (lane == 0) red[wave] = mn;
  __syncthreads();
  const uint32_t tk = mono_key(fminf(fminf(red[0], red[1]), fminf(red[2], red[3])));
  uint64_t take = 0;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const long long e = e0 + it * 256 + tid;
    take |= (e < n && mono_key(sv[it]) >= tk) ? (1ull << it) : 0ull;
  }
  // workgroup prefix of the per-thread candidate counts, then one atomic per workgroup
  const int mine = __popcll(take);
  int x = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (tid == 0) base = atomicAdd(&cnt[r], wsum[0] + wsum[1] + wsum[2] + wsum[3]);
  __syncthreads();
  int pos = base + x - mine;
  for (int w2 = 0; w2 < wave; ++w2) pos += wsum[w2];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    if (take & (1ull << it)) {
      if (pos < kTopkCap) {
        cscore[(size_t)r * kTopkCap + pos] = sv[it];
        cidx[(size_t)r * kTopkCap + pos] = (int)(e0 + it * 256 + tid);
      }
      ++pos;
    }
  }
}

// ---------------------------------------------------------------- per-row select




// Exact selection over a whole row in global memory (rows whose candidate list
// overflowed).  Radix select on the 32-bit score key finds the K-th score T;
// every entry above T is taken, and entries equal to T are taken in index order
// until K are chosen.  Writes the chosen indices (unsorted) to sel[0..k).
CSA2_DEV void radix_select_row(const float* __restrict__ row, int n, int k, int* sel, uint32_t* hist,
                               int* misc) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t key = mono_key(row[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, dsel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (acc + (int)hist[dg] >= need) {
          dsel = dg;
          break;
        }
        acc += (int)hist[dg];
      }
      misc[0] = dsel;
      misc[1] = need - acc;
    }
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    pmask |= 255u << shift;
    need = misc[1];
    __syncthreads();
  }
  // prefix = key of the K-th score; `need` entries equal to it are taken
  const int n_gt = k - need;
  if (tid == 0) {
    misc[2] = 0;  // gt slots used
    misc[3] = 0;  // equal entries seen so far
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  int* wcount = misc + 8;  // [16]
  for (int base = 0; base < n; base += kSelThreads) {
    const int i = base + tid;
    uint32_t key = 0;
    if (i < n) key = mono_key(row[i]);
    const bool gt = i < n && key > prefix;
    const bool eq = i < n && key == prefix;
    if (gt) sel[atomicAdd(&misc[2], 1)] = i;
    const unsigned long long m = __ballot(eq);
    if (lane == 0) wcount[wave] = __popcll(m);
    __syncthreads();
    int before = misc[3];
    for (int w2 = 0; w2 < wave; ++w2) before += wcount[w2];
    const int rank = before + __popcll(m & ((1ull << lane) - 1ull));
    if (eq && rank < need) sel[n_gt + rank] = i;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w2 = 0; w2 < kSelThreads / 64; ++w2) tot += wcount[w2];
      misc[3] += tot;
    }
    __syncthreads();
  }
}

// The k-th largest of `total` unique 64-bit keys in LDS, by 8-bit digits; the bits
// every key shares (scores of one magnitude share their top bits) are skipped, so
// the first digit already spreads the keys.  Stops early once a digit's bucket is
// taken whole.  Returns T such that exactly k keys are >= T.  hist holds two
// 256-bucket histograms and bcast eight slots: pass p counts into histogram p%2
// and publishes in slots 3(p%2) .. +2 while the other histogram is cleared for
// the next pass, so a pass needs two barriers.
CSA2_DEV unsigned long long radix_kth_u64(const unsigned long long* keys, int total, int k,
                                          uint32_t* hist, unsigned long long* bcast) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 256) hist[tid] = 0u;
  if (tid == 0) {
    bcast[6] = 0ull;
    bcast[7] = ~0ull;
  }
  __syncthreads();
  // common high bits: OR and AND of all keys agree exactly where every key agrees
  unsigned long long kor = 0ull, kand = ~0ull;
  for (int i = tid; i < total; i += kSelThreads) {
    kor |= keys[i];
    kand &= keys[i];
  }
  {
    auto bor = [](int x, int y) { return x | y; };
    auto band = [](int x, int y) { return x & y; };
    const uint32_t oh = (uint32_t)wave_reduce_i32((int)(kor >> 32), bor);
    const uint32_t ol = (uint32_t)wave_reduce_i32((int)(uint32_t)kor, bor);
    const uint32_t ah = (uint32_t)wave_reduce_i32((int)(kand >> 32), band);
    const uint32_t al = (uint32_t)wave_reduce_i32((int)(uint32_t)kand, band);
    if (lane == 0) {
      atomicOr(&bcast[6], ((unsigned long long)oh << 32) | ol);
      atomicAnd(&bcast[7], ((unsigned long long)ah << 32) | al);
    }
  }
  __syncthreads();
  const unsigned long long diff = bcast[6] ^ bcast[7];
  const int top = diff ? 63 - __clzll(diff) : 0;  // highest bit where keys differ
  unsigned long long mask = diff ? ~0ull << (top + 1) : ~0ull;
  if (top == 63) mask = 0ull;
  unsigned long long prefix = bcast[7] & mask;
  int need = k;
  int pass = 0;
  for (int shift = top - 7; shift > -8; shift -= 8, ++pass) {
    if (shift < 0) shift = 0;
    uint32_t* h = hist + 256 * (pass & 1);
    if (tid < 256) hist[256 * ((pass + 1) & 1) + tid] = 0u;  // the next pass's histogram
    for (int i = tid; i < total; i += kSelThreads) {
      const unsigned long long key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&h[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    unsigned long long* bc = bcast + 3 * (pass & 1);
    if (tid < 64) {
      // lane l owns buckets 4l..4l+3; find the bucket where the count from the top reaches need
      uint32_t hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = h[4 * lane + q];
      const int c = (int)(hv[0] + hv[1] + hv[2] + hv[3]);
      int suf = c;  // inclusive suffix over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(suf, o);
        if (lane + o < 64) suf += y;
      }
      int run = suf - c;  // keys in buckets above this lane's
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (run < need && run + (int)hv[q] >= need) {
          bc[0] = (unsigned long long)(4 * lane + q);
          bc[1] = (unsigned long long)(need - run);
          bc[2] = (unsigned long long)hv[q];
        }
        run += (int)hv[q];
      }
    }
    __syncthreads();
    const unsigned long long dsel = bc[0];
    const int need2 = (int)bc[1], bucket = (int)bc[2];
    prefix = (prefix & ~(255ull << shift)) | (dsel << shift);
    mask |= 255ull << shift;
    need = need2;
    if (bucket == need || shift == 0) break;  // the whole bucket is taken: keys >= prefix are exactly k
  }
  return prefix;
}

// Inclusive prefix sum over a kSelThreads workgroup (one value per thread); wsum:
// kSelThreads / 64 ints of LDS; *total = the sum.
CSA2_DEV int block_scan_sel(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w2 = 0; w2 < kSelThreads / 64; ++w2) {
    const int c = wsum[w2];
    before += w2 < wave ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + x;
}

// ---------------------------------------------------------------- histogram select
//
// Exact choice of the k best of a row's values (thread t holds the M values
// t + kSelThreads * u; key order = value desc, index asc) in few barriers:
//   1. min and max of the values;
//   2. a histogram of kHistBuckets buckets of [min, max] under a monotone map
//      (value_bucket: equal values share a bucket, a larger value never falls in
//      a lower one);
//   3. the bucket b* where the count from the top reaches k: every value in a
//      higher bucket is chosen, and only the values in b* need ranking;
//   4. the b* values are ranked exactly: by comparing each with all the others
//      when they are few, else by the radix select on unique 64-bit keys, else
//      (more than kTopkCap in one bucket: a row of equal or tightly packed
//      values) by the exact whole-row select.
// Marks the k chosen indices in the bitmap (bit i & 31 of word i >> 5; all words
// are written).  LDS: keys holds kTopkCap keys (its first 8 KB also serve as the
// histogram).
constexpr int kHistBuckets = 2 * kSelThreads;
constexpr int kRankDirect = 256;   // boundary values ranked by direct comparison

CSA2_DEV int value_bucket(float v, float lo, float scale) {
  // the barrier on the input keeps the compiler from holding the differences of
  // the histogram pass until the placement pass (it would spill them)
  asm volatile("" : "+v"(v));
  float d = v - lo;
  asm volatile("" : "+v"(d));   // the difference and the product are rounded on their own
  float x = d * scale;
  asm volatile("" : "+v"(x));
  // x >= 0 or NaN (an infinite value against an infinite range, or 0 times an
  // infinite scale): NaN goes to bucket 0, which keeps the map monotone (every
  // value then shares bucket 0, or only the row minimum sits below the rest)
  return x >= 0.0f ? (int)fminf(x, (float)(kHistBuckets - 1)) : 0;
}

struct HistSelLds {
  unsigned long long* keys;  // [kTopkCap]
  uint32_t* bitmap;          // [M * kSelThreads / 32]
  uint32_t* rhist;           // [512] radix histograms
  unsigned long long* bcast; // [8]
  int* wsum;                 // [kSelThreads / 64]
  float* red;                // [2 * kSelThreads / 64]
  int* misc;                 // [32]
};

// Value u of thread t is element t + u * kSelThreads of the row (present when that
// is below `total`).
template <int M>
CSA2_DEV void hist_select(const float (&v)[M], int total, int k,
                          const float* __restrict__ row, int n, const HistSelLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kSelThreads / 64;
  // ---- 1. range of the values
  auto ok = [&](int u) { return tid + u * kSelThreads < total; };
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < M; ++u) {
    if (ok(u)) {
      mn = fminf(mn, v[u]);
      mx = fmaxf(mx, v[u]);
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    L.red[wave] = mn;
    L.red[NW + wave] = mx;
  }
  uint32_t* hist = reinterpret_cast<uint32_t*>(L.keys);
  hist[tid] = 0u;
  hist[tid + kSelThreads] = 0u;
  if (tid < 8) L.misc[tid] = 0;
  __syncthreads();
  float lo = L.red[0], hi = L.red[NW];
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) {
    lo = fminf(lo, L.red[w2]);
    hi = fmaxf(hi, L.red[NW + w2]);
  }
  const float span = hi - lo;
  const float scale = (span > 0.0f && span < INFINITY) ? (float)kHistBuckets / span : 0.0f;
  // ---- 2. histogram
#pragma unroll
  for (int u = 0; u < M; ++u)
    if (ok(u)) atomicAdd(&hist[value_bucket(v[u], lo, scale)], 1u);
  __syncthreads();
  // ---- 3. boundary bucket (thread t owns buckets 2t and 2t + 1)
  const uint32_t c0 = hist[2 * tid], c1 = hist[2 * tid + 1];
  int tot;
  const int incl = block_scan_sel((int)(c0 + c1), L.wsum, &tot);
  const int above = tot - incl;  // values in buckets above 2t + 1
  if (above < k && above + (int)c1 >= k) {
    L.misc[0] = 2 * tid + 1;
    L.misc[1] = k - above;
    L.misc[2] = (int)c1;
  } else if (above + (int)c1 < k && above + (int)(c0 + c1) >= k) {
    L.misc[0] = 2 * tid;
    L.misc[1] = k - above - (int)c1;
    L.misc[2] = (int)c0;
  }
  __syncthreads();
  const int bstar = L.misc[0], need = L.misc[1], nbnd = L.misc[2];
  // ---- 4. values above b* are chosen; b*'s values are chosen too when all of
  // them are needed, else their keys are staged for ranking.  Step u of wave w
  // covers indices kSelThreads * u + 64 w .. + 63: the wave's ballot of the chosen
  // ones is that 64-bit stretch of the bitmap, stored whole by one lane
  const bool all_bnd = nbnd == need;
  const unsigned long long below = (1ull << lane) - 1ull;
  unsigned long long* bm64 = reinterpret_cast<unsigned long long*>(L.bitmap);
#pragma unroll
  for (int u = 0; u < M; ++u) {
    const int bb = ok(u) ? value_bucket(v[u], lo, scale) : -1;
    const unsigned long long mt = __ballot(bb > bstar || (all_bnd && bb == bstar));
    if (lane == 0) bm64[u * NW + wave] = mt;
    const bool stage = !all_bnd && bb == bstar;
    const unsigned long long ms = __ballot(stage);
    if (ms) {  // the same for the whole wave; most steps stage nothing
      int bs = 0;
      if (lane == 0) bs = atomicAdd(&L.misc[4], __popcll(ms));
      bs = __builtin_amdgcn_readfirstlane(bs);
      const int ps = bs + __popcll(ms & below);
      if (stage && ps < kTopkCap) L.keys[ps] = make_key(v[u], tid + u * kSelThreads);
    }
  }
  __syncthreads();
  if (all_bnd) return;
  auto mark = [&](int i) { atomicOr(&L.bitmap[i >> 5], 1u << (i & 31)); };
  if (nbnd <= kRankDirect) {
    if (tid < nbnd) {
      const unsigned long long key = L.keys[tid];
      int rank = 0;
      for (int j = 0; j < nbnd; ++j) rank += L.keys[j] > key ? 1 : 0;
      if (rank < need) mark(key_index(key));
    }
  } else if (nbnd <= kTopkCap) {
    const unsigned long long T = radix_kth_u64(L.keys, nbnd, need, L.rhist, L.bcast);
    for (int i = tid; i < nbnd; i += kSelThreads) {
      const unsigned long long key = L.keys[i];
      if (key >= T) mark(key_index(key));
    }
  } else {
    int* sel = reinterpret_cast<int*>(L.keys + 1024);
    radix_select_row(row, n, k, sel, reinterpret_cast<uint32_t*>(L.keys), L.misc);
    for (int w = tid; w < M * kSelThreads / 32; w += kSelThreads) L.bitmap[w] = 0u;
    __syncthreads();
    for (int i = tid; i < k; i += kSelThreads) mark(sel[i]);
  }
  __syncthreads();
}

// Writes the k chosen indices of a row in ascending order (rank = number of
// chosen indices below), -1 in slots k..K-1.  chosen[k .. 4*ceil(k/4)) must hold
// INT_MAX; the count reads four chosen indices per LDS access.
CSA2_DEV void write_ranked(const int* chosen, int k, int K, int* orow, const int* cmap_row) {
  const int4* c4 = reinterpret_cast<const int4*>(chosen);
  const int k4 = (k + 3) / 4;
  for (int i = threadIdx.x; i < K; i += kSelThreads) {
    if (i < k) {
      const int v = chosen[i];
      int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll 4
      for (int j = 0; j < k4; ++j) {
        const int4 c = c4[j];
        r0 += c.x < v;
        r1 += c.y < v;
        r2 += c.z < v;
        r3 += c.w < v;
      }
      orow[r0 + r1 + r2 + r3] = cmap_row ? cmap_row[v] : v;
    } else {
      orow[i] = -1;
    }
  }
}

CSA2_DEV void pad_chosen(int* chosen, int k) {
  const int k4 = 4 * ((k + 3) / 4);
  if ((int)threadIdx.x < k4 - k) chosen[k + threadIdx.x] = 0x7FFFFFFF;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const float* __restrict__ scores, int N, const int* __restrict__ valid_len,
    const int* __restrict__ cand_map, int K, int* __restrict__ out, const int* __restrict__ cnt,
    int cnt_stride, const float* __restrict__ cscore, const int* __restrict__ cidx) {
  extern __shared__ unsigned long long keys[];  // kTopkCap keys (64 KB)
  __shared__ __attribute__((aligned(16))) int chosen[2048];
  __shared__ uint32_t hist[512];
  __shared__ unsigned long long bcast[8];
  __shared__ int misc[32];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = row_len(valid_len, r, N);
  const bool direct = n <= kTopkCap;
  const int total = direct ? n : cnt[(size_t)r * cnt_stride];
  const int k = min(K, n);
  const float* row = scores + (size_t)r * N;
  if (!direct && (total > kTopkCap || total < k)) {
    int* sel = reinterpret_cast<int*>(keys + 1024);
    radix_select_row(row, n, k, sel, reinterpret_cast<uint32_t*>(keys), misc);
    for (int i = tid; i < k; i += kSelThreads) chosen[i] = sel[i];
    __syncthreads();
  } else {
    // all of a thread's loads first, then the LDS writes (one memory round trip)
    constexpr int kPer = kTopkCap / kSelThreads;
    float sv[kPer];
    int iv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      sv[u] = i < total ? (direct ? row[i] : cscore[(size_t)r * kTopkCap + i]) : 0.0f;
      iv[u] = i < total ? (direct ? i : cidx[(size_t)r * kTopkCap + i]) : 0;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < total) keys[i] = make_key(sv[u], iv[u]);
    }
    if (tid == 0) misc[0] = 0;
    __syncthreads();
    const unsigned long long T = k > 0 ? radix_kth_u64(keys, total, k, hist, bcast) : ~0ull;
    for (int i = tid; i < total; i += kSelThreads) {
      const unsigned long long key = keys[i];
      if (key >= T) chosen[atomicAdd(&misc[0], 1)] = key_index(key);
    }
    __syncthreads();
  }
  // output in ascending index order
  pad_chosen(chosen, k);
  __syncthreads();
  write_ranked(chosen, k, K, out + (size_t)r * K, cand_map ? cand_map + (size_t)r * N : nullptr);
}

// A key T with at least k of the workgroup's keys >= T (NPT keys per thread; key 0
// marks an empty slot and ranks below every real key).  Radix select by 8-bit
// digits from the highest bit where the keys differ; with `passes` >= 4 (or when
// a digit's bucket is taken whole) T is exactly the k-th largest key, otherwise
// it is the k-th largest key with its remaining low bits cleared (a lower bound).
// hist: 256 uint32 of LDS; bc: 4 uint32 of LDS.  k >= 1.
template <int NPT>
CSA2_DEV uint32_t block_kth_u32(const uint32_t (&key)[NPT], int k, int passes, uint32_t* hist,
                                uint32_t* bc) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t kor = 0u, kand = ~0u;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    kor |= key[i];
    kand &= key[i] ? key[i] : ~0u;
  }
  if (tid == 0) {
    bc[0] = 0u;
    bc[1] = ~0u;
  }
  __syncthreads();
  {
    const uint32_t o = (uint32_t)wave_reduce_i32((int)kor, [](int x, int y) { return x | y; });
    const uint32_t a = (uint32_t)wave_reduce_i32((int)kand, [](int x, int y) { return x & y; });
    if (lane == 0) {
      atomicOr(&bc[0], o);
      atomicAnd(&bc[1], a);
    }
  }
  __syncthreads();
  const uint32_t diff = bc[0] ^ bc[1];
  __syncthreads();
  int top = diff ? 31 - __clz((int)diff) : 0;  // highest bit where (non-empty) keys differ
  uint32_t mask = top >= 31 ? 0u : ~0u << (top + 1);
  uint32_t prefix = bc[1] & mask;
  int need = k;
  for (int pass = 0, shift = top - 7; shift > -8; shift -= 8, ++pass) {
    if (shift < 0) shift = 0;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if ((key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      uint32_t hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = hist[4 * lane + q];
      const int c = (int)(hv[0] + hv[1] + hv[2] + hv[3]);
      int suf = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(suf, o);
        if (lane + o < 64) suf += y;
      }
      int run = suf - c;  // keys in buckets above this lane's
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (run < need && run + (int)hv[q] >= need) {  // one bucket of one lane
          bc[2] = (uint32_t)(4 * lane + q);
          bc[3] = (uint32_t)(need - run) | ((uint32_t)hv[q] << 16);
        }
        run += (int)hv[q];
      }
      // fewer keys than k under the prefix (the first pass, when k exceeds the
      // number of non-empty keys): every key is taken, T = 0
      if (lane == 0 && suf < need) bc[2] = 0xFFFFFFFFu;
    }
    __syncthreads();
    const uint32_t dsel = bc[2], nb = bc[3];
    __syncthreads();
    if (dsel == 0xFFFFFFFFu) return 0u;
    prefix |= dsel << shift;
    mask |= 255u << shift;
    const int need2 = (int)(nb & 0xFFFFu), bucket = (int)(nb >> 16);
    need = need2;
    if (bucket == need || shift == 0 || pass + 1 >= passes) break;
  }
  return prefix;
}

// Rows of at most kRowCap entries (prefill: thousands of rows of 12K-16K visible
// entries; Reindex pools of 16,384) in one pass, one workgroup per row: the row
// stays in registers and the histogram select above picks its K best (the
// values above the boundary bucket directly, the boundary bucket's few values
// by exact ranking).  Against the earlier chunk-maxima bound + radix select on
// all candidates: 16.2 -> 13.0 us for 8 rows of 16,384, 333 -> 245 us for
// 8,192 prefill rows.

// Two rows per CU (eight waves per SIMD) are part of the design, and the bound
// keeps the register budget there: without it the compiler used 85 scalar
// registers and the GPU then held only one row per CU (prefill rows 1.8x
// slower); with it a few scalar registers spill to vector lanes.
__global__ __launch_bounds__(kSelThreads, 8) void topk_row_kernel(
    const float* __restrict__ scores, int N, const int* __restrict__ valid_len,
    const int* __restrict__ cand_map, int K, int* __restrict__ out) {
  __shared__ unsigned long long keys[kTopkCap];   // 64 KB
  __shared__ __attribute__((aligned(16))) int chosen[2048];
  __shared__ uint32_t hist[512];
  __shared__ unsigned long long bcast[8];
  __shared__ int misc[32];
  __shared__ __attribute__((aligned(8))) uint32_t bitmap[kRowCap / 32];
  __shared__ int wsum[kSelThreads / 64];
  __shared__ float red[2 * kSelThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = row_len(valid_len, r, N);
  const int k = min(K, n);
  const float* row = scores + (size_t)r * N;
  // every load of a thread is requested before the first is used: the row arrives
  // in one memory round trip and stays in registers (thread t holds entries
  // t + 1024u)
  constexpr int kPer = kRowCap / kSelThreads;
  float rv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * kSelThreads;
    rv[u] = i < n ? row[i] : 0.0f;
  }
  // the chosen indices (all < kRowCap) as a bitmap; for the output in ascending
  // index order, word w's set bits go to slots from the number of bits in words < w
  if (k > 0) {
    const HistSelLds L{keys, bitmap, hist, bcast, wsum, red, misc};
    hist_select<kPer>(rv, n, k, row, n, L);
  } else {
    for (int w2 = tid; w2 < kRowCap / 32; w2 += kSelThreads) bitmap[w2] = 0u;
    __syncthreads();
  }
  constexpr int kWords = kRowCap / 32;  // one word per thread (kWords <= kSelThreads)
  const uint32_t word = tid < kWords ? bitmap[tid] : 0u;
  const int cnt = __popc(word);
  int x = cnt;  // inclusive prefix within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int slot = x - cnt;
  for (int w2 = 0; w2 < wave; ++w2) slot += wsum[w2];
  // the chosen indices in ascending order, in LDS, then one parallel pass maps
  // them through the candidate
  // map and stores them: one memory round trip, not one per chosen index
  for (uint32_t m = word; m; m &= m - 1u) chosen[slot++] = 32 * tid + __ffs(m) - 1;
  __syncthreads();
  int* orow = out + (size_t)r * K;
  const int* cmap_row = cand_map ? cand_map + (size_t)r * N : nullptr;
  for (int i = tid; i < K; i += kSelThreads) {
    const int v = i < k ? chosen[i] : -1;
    orow[i] = (cmap_row != nullptr && v >= 0) ? cmap_row[v] : v;
  }
}

hipError_t launch_topk(const float* scores, int R, int N, const int* valid_len, const int* cand_map,
                       int K, int* out_idx, const TopkWs& ws, hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (N <= kRowCap) {
    hipLaunchKernelGGL(topk_row_kernel, dim3(R), dim3(kSelThreads), 0, st, scores, N, valid_len,
                       cand_map, K, out_idx);
    return hipGetLastError();
  }
  {
    const int cpw = N / K <= 128 ? kChunksPerWave : 1;  // chunk length <= N / K
    hipLaunchKernelGGL(topk_chunkmax_kernel, dim3((2 * K + 4 * cpw - 1) / (4 * cpw), R), dim3(256), 0,
                       st, scores, N, valid_len, K, cpw, ws.cmax, ws.cnt);
    if (N >= (1 << 18)) {
      const int fx = (N + 256 * 64 - 1) / (256 * 64);
      hipLaunchKernelGGL(topk_filter_kernel<64>, dim3(fx, R), dim3(256), 0, st, scores, N, valid_len, K,
                         ws.cmax, ws.cnt, ws.cscore, ws.cidx);
    } else {
      const int fx = (N + 256 * 16 - 1) / (256 * 16);
      hipLaunchKernelGGL(topk_filter_kernel<16>, dim3(fx, R), dim3(256), 0, st, scores, N, valid_len, K,
                         ws.cmax, ws.cnt, ws.cscore, ws.cidx);
    }
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3(R), dim3(kSelThreads),
                     kTopkCap * sizeof(unsigned long long), st, scores, N, valid_len, cand_map, K,
                     out_idx, ws.cnt, 1, ws.cscore, ws.cidx);
  return hipGetLastError();
}

// ---------------------------------------------------------------- candidate pool

static inline int pool_nblk(int N, int G) { return (N + G - 1) / G; }


size_t pool_ws_bytes(int R, int N, int G, int PB) {
  const int nb = pool_nblk(N, G);
  size_t b = 0;
  b += align256((size_t)R * nb * sizeof(float));  // block maxima
  b += align256((size_t)R * sizeof(int));         // blocks per row
  b += align256((size_t)R * PB * sizeof(int));    // chosen blocks
  b += topk_ws_bytes(R, nb, PB);
  return b;
}

CSA2_DEV int visible(const int* q_pos, int m, int r, int N) {
  if (!q_pos) return N;
  long long v = ((long long)q_pos[r] + 1) / m;
  return (int)(v < 0 ? 0 : (v > N ? N : v));
}

constexpr int kBlocksPerWave = 4;

// Block maxima: one wave per kBlocksPerWave consecutive blocks, the first 128
// entries of each block requested together (blocks are G <= 256 entries).
__global__ __launch_bounds__(256) void pool_blockmax_kernel(const float* __restrict__ scores, int N,
                                                            const int* __restrict__ q_pos, int m,
                                                            int G, int nblk_max,
                                                            float* __restrict__ bmax,
                                                            int* __restrict__ nblk_out) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int b0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kBlocksPerWave;
  if (b0 >= nblk_max) return;
  const int n = visible(q_pos, m, r, N);
  const int nblk = (n + G - 1) / G;
  if (b0 == 0 && lane == 0) nblk_out[r] = nblk;
  const float* row = scores + (size_t)r * N;
  float v[kBlocksPerWave][2];
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    const int lo = (b0 + j) * G, hi = min(lo + G, n);
    const bool live = b0 + j < nblk;
    v[j][0] = live && lo + lane < hi ? row[lo + lane] : -INFINITY;
    v[j][1] = live && lo + 64 + lane < hi ? row[lo + 64 + lane] : -INFINITY;
  }
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    const int blk = b0 + j;
    if (blk >= nblk_max) break;
    float mx = -INFINITY;
    if (blk < nblk) {
      const int lo = blk * G, hi = min(lo + G, n);
      mx = fmaxf(v[j][0], v[j][1]);
      for (int i = lo + 128 + lane; i < hi; i += 64) mx = fmaxf(mx, row[i]);
      mx = wave_max(mx);
    }
    if (lane == 0) bmax[(size_t)r * nblk_max + blk] = mx;
  }
}


// The PE best entries (score, then lower index) of row[lo, lo + len), len <= 64 *
// KPL, written in ascending index order to out[0 .. min(PE, len)) and -1 to the
// rest of out[0 .. PE).  One wave; each pick is an arg-max over the wave: the
// 32-bit score key is reduced first, the full (score, index) key only when
// several lanes tie on the score.
template <int KPL>
CSA2_DEV void block_top_pe(const float* __restrict__ row, int lo, int len, int PE, int* out) {
  const int lane = threadIdx.x & 63;
  unsigned long long key[KPL];  // 0 = no entry (a real key is never 0)
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int j = lane + 64 * q;
    key[q] = j < len ? make_key(row[lo + j], lo + j) : 0ull;
  }
  const int cntb = min(PE, len);  // PE <= 16
  int mine = 0x7FFFFFFF;          // lane p keeps the p-th pick
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    if (p < cntb) {
      unsigned long long best = key[0];
#pragma unroll
      for (int q = 1; q < KPL; ++q) best = key[q] > best ? key[q] : best;
      const uint32_t hi = (uint32_t)(best >> 32);
      const uint32_t hmax = wave_max_u32(hi);
      const unsigned long long tied = __ballot(hi == hmax);
      unsigned long long win;
      if (__popcll(tied) == 1) {
        const int wl = __ffsll((long long)tied) - 1;
        win = ((unsigned long long)hmax << 32) |
              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, wl);
      } else {
        win = wave_max_u64(hi == hmax ? best : 0ull);
      }
      if (lane == p) mine = key_index(win);
#pragma unroll
      for (int q = 0; q < KPL; ++q)
        if (key[q] == win) key[q] = 0ull;
    }
  }
  // ascending order of the picks: rank = number of smaller picks
  int rank = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int v = __builtin_amdgcn_readlane(mine, q);
    rank += (q < cntb && v < mine) ? 1 : 0;
  }
  if (lane < cntb) out[rank] = mine;
  else if (lane < PE) out[lane] = -1;
}

// Per selected block, its PE best entries (score, then lower index) in ascending
// index order.  One wave per block, KPL = ceil(G/64) keys per lane; each pick is
// an arg-max over the wave: the 32-bit score key is reduced first, and the full
// (score, index) key only when several lanes tie on the score.
template <int KPL>
__global__ __launch_bounds__(256) void pool_gather_kernel(const float* __restrict__ scores, int N,
                                                          const int* __restrict__ q_pos, int m, int G,
                                                          int PB, int PE,
                                                          const int* __restrict__ selblk,
                                                          int* __restrict__ pool,
                                                          int* __restrict__ pool_len) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slot >= PB) return;
  const int n = visible(q_pos, m, r, N);
  const int nblk = (n + G - 1) / G;
  const int nsel = min(PB, nblk);
  int* prow = pool + (size_t)r * PB * PE;
  if (slot >= nsel) {
    for (int i = lane; i < PE; i += 64) prow[(size_t)slot * PE + i] = -1;
    if (slot == 0 && lane == 0) pool_len[r] = 0;
    return;
  }
  const int blk = selblk[(size_t)r * PB + slot];
  const int lo = blk * G;
  const int len = min(G, n - lo);
  block_top_pe<KPL>(scores + (size_t)r * N, lo, len, PE, prow + (size_t)slot * PE);
  if (slot == nsel - 1 && threadIdx.x % 64 == 0) pool_len[r] = slot * PE + min(PE, len);
}

hipError_t launch_pool(const float* scores, int R, int N, const int* q_pos, int m, int G, int PB,
                       int PE, int* pool, int* pool_len, void* ws, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int nb = pool_nblk(N, G);
  char* p = static_cast<char*>(ws);
  float* bmax = reinterpret_cast<float*>(p);
  p += align256((size_t)R * nb * sizeof(float));
  int* nblk = reinterpret_cast<int*>(p);
  p += align256((size_t)R * sizeof(int));
  int* selblk = reinterpret_cast<int*>(p);
  p += align256((size_t)R * PB * sizeof(int));
  TopkWs tws = topk_ws_carve(p, R, PB);
  hipLaunchKernelGGL(pool_blockmax_kernel, dim3((nb + 4 * kBlocksPerWave - 1) / (4 * kBlocksPerWave), R),
                     dim3(256), 0, st, scores, N, q_pos,
                     m, G, nb, bmax, nblk);
  hipError_t e = launch_topk(bmax, R, nb, nblk, nullptr, PB, selblk, tws, st);
  if (e != hipSuccess) return e;
  const dim3 ggrid((PB + 3) / 4, R);
  if (G <= 64)
    hipLaunchKernelGGL(pool_gather_kernel<1>, ggrid, dim3(256), 0, st, scores, N, q_pos, m, G, PB, PE,
                       selblk, pool, pool_len);
  else if (G <= 128)
    hipLaunchKernelGGL(pool_gather_kernel<2>, ggrid, dim3(256), 0, st, scores, N, q_pos, m, G, PB, PE,
                       selblk, pool, pool_len);
  else
    hipLaunchKernelGGL(pool_gather_kernel<4>, ggrid, dim3(256), 0, st, scores, N, q_pos, m, G, PB, PE,
                       selblk, pool, pool_len);
  return hipGetLastError();
}


// ---------------------------------------------------------------- Full-layer selection from tile maxima
//
// The decode scan writes, with the scores, the maximum of every 32-entry span of
// each row.  From those maxima alone one workgroup per row (the plan kernel)
// finds, for the whole visible range:
//   * block maxima of the G = 128-entry pool blocks (4 spans each) and the PB
//     best blocks by (maximum desc, block asc) -- the pool's blocks;
//   * a threshold T for the Top-K: T is at most the K-th largest maximum of
//     C >= K disjoint groups of spans; those K group maxima are K distinct entries
//     scoring >= T, so the K-th best score is >= T, and every entry of the K best
//     lies in a span whose maximum is >= T (the candidate spans).
// A gather kernel then reads only the pool blocks (their PE best entries) and the
// candidate spans (entries scoring >= T, appended to a candidate list), and the
// exact select above finishes the Top-K from the candidates.  With 4,096 groups
// per row the threshold keeps about K entries of a million.

constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxBlocks = 8;  // pool blocks per thread: rows of up to 1,048,576 entries
constexpr int kPlanGroups = 4;     // threshold groups per thread
constexpr int kCntStride = 64;     // candidate counters one 256-byte line apart (per row)

struct PlanWs {
  uint32_t* thr;   // [R] threshold key (mono_key of T)
  int* npb;        // [R] pool blocks chosen
  int* nct;        // [R] candidate spans
  int* vlen;       // [R] visible entries
  int* selblk;     // [R, PB] pool blocks, ascending
  int* candtile;   // [R, spans] candidate spans
};

// Inclusive prefix sum over the workgroup (kPlanThreads threads, one value each).
// wsum: kPlanThreads / 64 ints of LDS.  Returns the inclusive prefix; *total the sum.
CSA2_DEV int block_scan_incl(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w2 = 0; w2 < kPlanThreads / 64; ++w2) {
    const int c = wsum[w2];
    before += w2 < wave ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + x;
}

// Two radix selections over the workgroup's keys at once (they share every
// barrier): for each, a key T with at least k keys >= T (key 0 marks an empty
// slot and ranks below every real key), found digit by digit (8 bits) from the
// highest bit where the non-empty keys differ.  Selection s stops after
// passes[s] digits (T = the k-th largest key with its lower bits cleared: a lower
// bound) or when its digit's bucket is taken whole; with 4 passes T is exact.
// k[s] = 0 skips selection s (T = 0).  hist: 1024 uint32 of LDS (two halves used in
// turn); bc: 16 uint32.
template <int NA, int NB>
CSA2_DEV void block_kth2_u32(const uint32_t (&ka)[NA], const uint32_t (&kb)[NB], const int (&k)[2],
                             const int (&passes)[2], uint32_t (&T)[2], uint32_t* hist, uint32_t* bc) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t kor[2] = {0u, 0u}, kand[2] = {~0u, ~0u};
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    kor[0] |= ka[i];
    kand[0] &= ka[i] ? ka[i] : ~0u;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    kor[1] |= kb[i];
    kand[1] &= kb[i] ? kb[i] : ~0u;
  }
  if (tid < 2) {
    bc[2 * tid] = 0u;
    bc[2 * tid + 1] = ~0u;
  }
  if (tid < 512) hist[tid] = 0u;  // the first pass's half of the histogram
  __syncthreads();
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const uint32_t o = (uint32_t)wave_reduce_i32((int)kor[s2], [](int x, int y) { return x | y; });
    const uint32_t a = (uint32_t)wave_reduce_i32((int)kand[s2], [](int x, int y) { return x & y; });
    if (lane == 0) {
      atomicOr(&bc[2 * s2], o);
      atomicAnd(&bc[2 * s2 + 1], a);
    }
  }
  __syncthreads();
  uint32_t prefix[2], mask[2];
  int shift[2], need[2];
  bool live[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const uint32_t diff = bc[2 * s2] ^ bc[2 * s2 + 1];
    const int top = diff ? 31 - __clz((int)diff) : 0;
    mask[s2] = top >= 31 ? 0u : ~0u << (top + 1);
    prefix[s2] = bc[2 * s2 + 1] & mask[s2];
    shift[s2] = top - 7;
    need[s2] = k[s2];
    live[s2] = k[s2] > 0;
    T[s2] = 0u;
  }
  __syncthreads();
  for (int pass = 0; live[0] || live[1]; ++pass) {
    int sh[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) sh[s2] = shift[s2] < 0 ? 0 : shift[s2];
    // two halves of hist alternate: pass p counts into half p mod 2 and clears the
    // other for pass p + 1 (its last reader, the scan of pass p - 1, finished
    // before that pass's second barrier)
    uint32_t* hc = hist + 512 * (pass & 1);
    if (tid < 512) hist[512 * ((pass + 1) & 1) + tid] = 0u;
    if (live[0]) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        if ((ka[i] & mask[0]) == prefix[0]) atomicAdd(&hc[(ka[i] >> sh[0]) & 255u], 1u);
    }
    if (live[1]) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if ((kb[i] & mask[1]) == prefix[1]) atomicAdd(&hc[256 + ((kb[i] >> sh[1]) & 255u)], 1u);
    }
    __syncthreads();
    if (tid < 128) {  // wave s2 finds selection s2's bucket
      const int s2 = tid >> 6;
      if (live[s2]) {
        const uint32_t* h = hc + 256 * s2;
        uint32_t hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = h[4 * lane + q];
        const int c = (int)(hv[0] + hv[1] + hv[2] + hv[3]);
        int suf = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_down(suf, o);
          if (lane + o < 64) suf += y;
        }
        int run = suf - c;  // keys in buckets above this lane's
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (run < need[s2] && run + (int)hv[q] >= need[s2]) {  // one bucket of one lane
            bc[8 + 2 * s2] = (uint32_t)(4 * lane + q);
            bc[9 + 2 * s2] = (uint32_t)(need[s2] - run) | ((uint32_t)hv[q] << 16);
          }
          run += (int)hv[q];
        }
        // fewer keys than k under the prefix (first pass, k above the number of
        // non-empty keys): every key is taken, T = 0
        if (lane == 0 && suf < need[s2]) bc[8 + 2 * s2] = 0xFFFFFFFFu;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (!live[s2]) continue;
      const uint32_t dsel = bc[8 + 2 * s2], nb = bc[9 + 2 * s2];
      if (dsel == 0xFFFFFFFFu) {
        T[s2] = 0u;
        live[s2] = false;
        continue;
      }
      prefix[s2] |= dsel << sh[s2];
      mask[s2] |= 255u << sh[s2];
      need[s2] = (int)(nb & 0xFFFFu);
      const int bucket = (int)(nb >> 16);
      T[s2] = prefix[s2];
      if (bucket == need[s2] || sh[s2] == 0 || pass + 1 >= passes[s2]) live[s2] = false;
      shift[s2] -= 8;
    }
    // no barrier here: the next pass writes bc only after its first barrier, which
    // every thread reaches after reading bc above
  }
}

// Span maxima (kTmaxSpan = 32 entries each) of a row are read as float4 f =
// j * kPlanThreads + t, j < F: every load instruction is coalesced, and float4 f
// holds the four spans of pool block f (128 entries), so each thread owns F
// blocks.
template <int F>
CSA2_DEV void plan_load(const float* __restrict__ trow, int ns, float4 (&v)[F]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const int f = j * kPlanThreads + t, sp = 4 * f;
    if (sp + 3 < ns) {
      v[j] = reinterpret_cast<const float4*>(trow)[f];
    } else {
      v[j].x = sp < ns ? trow[sp] : -INFINITY;
      v[j].y = sp + 1 < ns ? trow[sp + 1] : -INFINITY;
      v[j].z = sp + 2 < ns ? trow[sp + 2] : -INFINITY;
      v[j].w = sp + 3 < ns ? trow[sp + 3] : -INFINITY;
    }
  }
}

template <int F>
__global__ __launch_bounds__(kPlanThreads) void select_plan_kernel(
    const float* __restrict__ tmax, int L, const int* __restrict__ q_pos, int m, int K, int PB,
    PlanWs pw, int* __restrict__ cnt) {
  constexpr int NG = kPlanGroups;                      // threshold groups per thread
  constexpr int GSP = 4 * F / NG;                      // spans per group
  constexpr int kBlkWords = kPlanThreads * F / 32;     // bitmap words of all blocks
  static_assert(kBlkWords <= kPlanThreads && GSP >= 1, "plan shape");
  __shared__ uint32_t hist[1024];  // two alternating 512-bucket halves
  __shared__ uint32_t bc[16];
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ __attribute__((aligned(8))) uint32_t bitmap[2 * kBlkWords];  // above V, equal to V
  const int r = blockIdx.x, tid = threadIdx.x;
  const int ns_cap = (L + kTmaxSpan - 1) / kTmaxSpan;
  const int n = visible(q_pos, m, r, L);
  const int ns = (n + kTmaxSpan - 1) / kTmaxSpan, nblk = (n + 127) / 128;
  const float* trow = tmax + (size_t)r * ns_cap;
  uint32_t gk[NG], bk[F];  // keys of threshold groups and pool blocks; 0 = empty
  float4 v[F];             // the span maxima, held for the candidate pass
  {
    plan_load<F>(trow, ns, v);
    float sm[4 * F];  // span maxima, local span l = 4j + c
#pragma unroll
    for (int j = 0; j < F; ++j) {
      sm[4 * j] = v[j].x;
      sm[4 * j + 1] = v[j].y;
      sm[4 * j + 2] = v[j].z;
      sm[4 * j + 3] = v[j].w;
      const float bm = fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w));
      bk[j] = j * kPlanThreads + tid < nblk ? mono_key(bm) : 0u;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float gm = -INFINITY;
      bool any = false;
#pragma unroll
      for (int u = 0; u < GSP; ++u) {
        const int l = g * GSP + u;
        gm = fmaxf(gm, sm[l]);
        any = any || 4 * ((l >> 2) * kPlanThreads + tid) + (l & 3) < ns;
      }
      gk[g] = any ? mono_key(gm) : 0u;
    }
  }
  if (tid == 0) {
    pw.vlen[r] = n;
    if (cnt != nullptr) cnt[(size_t)r * kCntStride] = 0;
  }
  const int take = PB > 0 ? min(PB, nblk) : 0;
  uint32_t T[2];
  {
    const int kk[2] = {K > 0 ? K : 0, take};
    const int ps[2] = {2, 4};  // Top-K: a lower bound after two digits; pool: exact
    block_kth2_u32<NG, F>(gk, bk, kk, ps, T, hist, bc);
  }
  const uint32_t thr = T[0], V = T[1];
  // ---- candidate spans (maximum >= T), from the span maxima still in registers
  unsigned long long cmask = 0ull;  // bit 4j + c: span 4(j*1024 + t) + c is a candidate
  if (K > 0) {
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int sp = 4 * (j * kPlanThreads + tid) + c;
        if (sp < ns && mono_key(e[c]) >= thr) cmask |= 1ull << (4 * j + c);
      }
    }
  }
  const int ncand = __popcll(cmask);
  int tot1;
  const int pos0 = block_scan_incl(ncand, wsum, &tot1) - ncand;
  {
    int pos = pos0;
    for (unsigned long long mm = cmask; mm; mm &= mm - 1ull) {
      const int b = __ffsll((long long)mm) - 1;
      pw.candtile[(size_t)r * ns_cap + pos++] = 4 * ((b >> 2) * kPlanThreads + tid) + (b & 3);
    }
  }
  if (tid == 0) {
    pw.thr[r] = thr;
    pw.nct[r] = K > 0 ? tot1 : 0;
    pw.npb[r] = take;
  }
  // ---- pool blocks: above V all, equal to V in block order until `take`.  Block
  // j * kPlanThreads + t sits in thread t, so for each j the 64 lanes of a wave
  // hold 64 consecutive blocks: the wave's ballots are 64-bit stretches of the
  // bitmaps of blocks above V and equal to V, stored whole by one lane.  One block
  // scan of both counts per 32-block word (equal low, above high; each below
  // 2^16) then gives every word its first output slot.
  if (take > 0) {
    const int lane = tid & 63, wave = tid >> 6;
    unsigned long long* gt64 = reinterpret_cast<unsigned long long*>(bitmap);
    unsigned long long* eq64 = reinterpret_cast<unsigned long long*>(bitmap + kBlkWords);
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const unsigned long long mg = __ballot(bk[j] != 0u && bk[j] > V);
      const unsigned long long me = __ballot(bk[j] != 0u && bk[j] == V);
      if (lane == 0) {
        gt64[j * (kPlanThreads / 64) + wave] = mg;
        eq64[j * (kPlanThreads / 64) + wave] = me;
      }
    }
    __syncthreads();
    const uint32_t gw = tid < kBlkWords ? bitmap[tid] : 0u;
    const uint32_t ew = tid < kBlkWords ? bitmap[kBlkWords + tid] : 0u;
    const int packed = __popc(ew) | (__popc(gw) << 16);
    int ptot;
    const int before = block_scan_incl(packed, wsum, &ptot) - packed;
    const int need_eq = max(take - (ptot >> 16), 0);  // equal blocks still to take
    const int eq_before = before & 0xFFFF;
    uint32_t chosen = gw;
    int erank = eq_before;
    for (uint32_t mm = ew; mm && erank < need_eq; mm &= mm - 1u, ++erank) chosen |= mm & (0u - mm);
    int p = (before >> 16) + min(eq_before, need_eq);
    for (uint32_t mm = chosen; mm; mm &= mm - 1u) pw.selblk[(size_t)r * PB + p++] = 32 * tid + __ffs(mm) - 1;
  }
}

// Pool role: wave s of a row takes pool block s (its PE best entries to pool
// slots s*PE ..).  Candidate role: the workgroup takes 8 candidate spans per
// round (a lane per entry, two spans per wave); entries scoring >= T are
// appended to the row's candidate list with one atomic per workgroup and round.
template <int KPL>
__global__ __launch_bounds__(256) void select_gather_kernel(
    const float* __restrict__ scores, int L, int PB, int PE, PlanWs pw, int* __restrict__ pool,
    int* __restrict__ pool_len, int* __restrict__ cnt, float* __restrict__ cscore,
    int* __restrict__ cidx) {
  __shared__ int s_cnt[4];
  __shared__ int s_base;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = blockIdx.x * 4 + wave;
  const int n = pw.vlen[r];
  const int ns_cap = (L + kTmaxSpan - 1) / kTmaxSpan;
  const float* row = scores + (size_t)r * L;
  if (PB > 0 && slot < PB) {
    const int npb = pw.npb[r];
    int* prow = pool + (size_t)r * PB * PE;
    if (slot >= npb) {
      for (int i = lane; i < PE; i += 64) prow[(size_t)slot * PE + i] = -1;
      if (slot == 0 && lane == 0) pool_len[r] = 0;
    } else {
      const int blk = pw.selblk[(size_t)r * PB + slot];
      const int lo = blk * 128, len = min(128, n - lo);
      block_top_pe<KPL>(row, lo, len, PE, prow + (size_t)slot * PE);
      if (slot == npb - 1 && lane == 0) pool_len[r] = slot * PE + min(PE, len);
    }
  }
  const int nct = pw.nct[r];
  const uint32_t thr = pw.thr[r];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = blockIdx.x * 8; c0 < nct; c0 += gridDim.x * 8) {  // uniform per workgroup
    const int c = c0 + 2 * wave + (lane >> 5);
    const int sp = c < nct ? pw.candtile[(size_t)r * ns_cap + c] : -1;
    const int i = sp * kTmaxSpan + (lane & 31);
    const float v = (sp >= 0 && i < n) ? row[i] : -INFINITY;
    const bool take = sp >= 0 && i < n && mono_key(v) >= thr;
    const unsigned long long mk = __ballot(take);
    if (lane == 0) s_cnt[wave] = __popcll(mk);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int tot = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
      s_base = tot ? atomicAdd(&cnt[(size_t)r * kCntStride], tot) : 0;
    }
    __syncthreads();
    int p = s_base;
    for (int w2 = 0; w2 < wave; ++w2) p += s_cnt[w2];
    p += __popcll(mk & below);
    if (take && p < kTopkCap) {
      cscore[(size_t)r * kTopkCap + p] = v;
      cidx[(size_t)r * kTopkCap + p] = i;
    }
    __syncthreads();  // s_cnt / s_base are rewritten next round
  }
}

size_t full_select_ws_bytes(int R, int N, int PB, int K) {
  const size_t nt = (size_t)(N + kTmaxSpan - 1) / kTmaxSpan;
  size_t b = 0;
  b += align256((size_t)R * nt * sizeof(float));                 // span maxima
  b += 4 * align256((size_t)R * sizeof(int));                     // thr, npb, nct, vlen
  b += align256((size_t)R * (PB > 0 ? PB : 1) * sizeof(int));     // pool blocks
  b += align256((size_t)R * nt * sizeof(int));                    // candidate spans
  if (K > 0) {
    b += align256((size_t)R * kCntStride * sizeof(int));          // candidate counters
    b += 2 * align256((size_t)R * kTopkCap * sizeof(float));      // candidates
  }
  return b;
}

float* full_select_tmax(void* ws) { return static_cast<float*>(ws); }

bool full_select_supported(int N, int G) {
  return N <= kPlanThreads * kPlanMaxBlocks * 128 && G == 128;
}

hipError_t launch_full_select(const float* scores, int R, int N, const int* q_pos, int m, int PB,
                              int PE, int* pool, int* pool_len, int K, int* sel, void* ws,
                              hipStream_t st) {
  if (R == 0) return hipSuccess;
  char* p = static_cast<char*>(ws);
  const size_t nt = (size_t)(N + kTmaxSpan - 1) / kTmaxSpan;
  const float* tmax = reinterpret_cast<const float*>(p);
  p += align256((size_t)R * nt * sizeof(float));
  PlanWs pw;
  pw.thr = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * sizeof(int));
  pw.npb = reinterpret_cast<int*>(p);
  p += align256((size_t)R * sizeof(int));
  pw.nct = reinterpret_cast<int*>(p);
  p += align256((size_t)R * sizeof(int));
  pw.vlen = reinterpret_cast<int*>(p);
  p += align256((size_t)R * sizeof(int));
  pw.selblk = reinterpret_cast<int*>(p);
  p += align256((size_t)R * (PB > 0 ? PB : 1) * sizeof(int));
  pw.candtile = reinterpret_cast<int*>(p);
  p += align256((size_t)R * nt * sizeof(int));
  int* cnt = nullptr;
  float* cscore = nullptr;
  int* cidx = nullptr;
  if (K > 0) {
    cnt = reinterpret_cast<int*>(p);
    p += align256((size_t)R * kCntStride * sizeof(int));
    cscore = reinterpret_cast<float*>(p);
    p += align256((size_t)R * kTopkCap * sizeof(float));
    cidx = reinterpret_cast<int*>(p);
  }
  const int pb = pool ? PB : 0;
  const int nblk = (N + 127) / 128;
#define CSA2_PLAN(F_)                                                                             \
  hipLaunchKernelGGL(select_plan_kernel<F_>, dim3(R), dim3(kPlanThreads), 0, st, tmax, N, q_pos, m, \
                     sel ? K : 0, pb, pw, cnt)
  if (nblk <= kPlanThreads) CSA2_PLAN(1);
  else if (nblk <= 2 * kPlanThreads) CSA2_PLAN(2);
  else if (nblk <= 4 * kPlanThreads) CSA2_PLAN(4);
  else CSA2_PLAN(8);
#undef CSA2_PLAN
  // pool: one wave per pool block; candidates: 8 spans per workgroup and round
  const int wgs = max((pb + 3) / 4, 64);
  hipLaunchKernelGGL(select_gather_kernel<2>, dim3(wgs, R), dim3(256), 0, st, scores, N, pb, PE, pw,
                     pool, pool_len, cnt, cscore, cidx);
  if (sel)
    hipLaunchKernelGGL(topk_select_kernel, dim3(R), dim3(kSelThreads),
                       kTopkCap * sizeof(unsigned long long), st, scores, N, pw.vlen, nullptr, K, sel,
                       cnt, kCntStride, cscore, cidx);
  return hipGetLastError();
}

// Entries visible to each row (decode: all N; with positions: floor((t+1)/m)).
__global__ void visible_len_kernel(const int* __restrict__ q_pos, int m, int R, int N,
                                   int* __restrict__ vlen) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) vlen[r] = visible(q_pos, m, r, N);
}

hipError_t launch_visible_len(const int* q_pos, int m, int R, int N, int* vlen, hipStream_t st) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(visible_len_kernel, dim3((R + 255) / 256), dim3(256), 0, st, q_pos, m, R, N, vlen);
  return hipGetLastError();
}

}  // namespace csa2
