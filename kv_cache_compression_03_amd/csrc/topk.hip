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
    const float* __restrict__ cscore, const int* __restrict__ cidx) {
  extern __shared__ unsigned long long keys[];  // kTopkCap keys (64 KB)
  __shared__ __attribute__((aligned(16))) int chosen[2048];
  __shared__ uint32_t hist[512];
  __shared__ unsigned long long bcast[8];
  __shared__ int misc[32];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = row_len(valid_len, r, N);
  const bool direct = n <= kTopkCap;
  const int total = direct ? n : cnt[r];
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

// Rows of at most kRowCap entries (prefill: thousands of rows of 12K-16K visible
// entries) in one pass, one workgroup per row: the row is staged in LDS, the
// minimum T of C >= K chunk maxima bounds the K-th best score from below, the
// entries scoring >= T become 64-bit keys in LDS, and the K-th key is found by
// radix select as for short rows.  A row whose candidates overflow (heavy ties)
// falls back to the exact whole-row select.

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
  __shared__ float red[kSelThreads / 64];
  __shared__ uint32_t bitmap[kRowCap / 32];
  __shared__ int wsum[kSelThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = row_len(valid_len, r, N);
  const int k = min(K, n);
  const float* row = scores + (size_t)r * N;
  int total;
  // every load of a thread is issued before its first LDS write, so the row
  // arrives in one memory round trip rather than one per element
  constexpr int kPer = kRowCap / kSelThreads;
  float rv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * kSelThreads;
    rv[u] = i < n ? row[i] : 0.0f;
  }
  if (n <= kTopkCap) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < n) keys[i] = make_key(rv[u], i);
    }
    total = n;
  } else {
    // The row stays in registers (thread t holds entries t + 1024u).  Chunks are
    // sets of a thread's entries: any C >= K disjoint non-empty chunks have C
    // distinct maxima, so the K-th best score is at least the smallest of them.
    // C = 512 chunks (threads t and t + 512 together) when K <= 512, else one
    // chunk per thread (C = 1024) or per half of a thread's entries (C = 2048).
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      const float v = i < n ? rv[u] : -INFINITY;
      if (u < kPer / 2) m0 = fmaxf(m0, v);
      else m1 = fmaxf(m1, v);
    }
    float cm;  // this thread's share of min over chunk maxima
    if (K <= kSelThreads / 2) {
      float* pm = reinterpret_cast<float*>(keys);  // keys are written only later
      pm[tid] = fmaxf(m0, m1);
      __syncthreads();
      cm = tid < kSelThreads / 2 ? fmaxf(pm[tid], pm[tid + kSelThreads / 2]) : INFINITY;
    } else if (K <= kSelThreads) {
      cm = fmaxf(m0, m1);
    } else {
      cm = fminf(m0, m1);  // an empty half (max -inf) sends the row to the exact path below
    }
    if (tid == 0) misc[0] = 0;
    cm = wave_min(cm);
    if (lane == 0) red[wave] = cm;
    __syncthreads();
    float T = red[0];
#pragma unroll
    for (int w2 = 1; w2 < kSelThreads / 64; ++w2) T = fminf(T, red[w2]);
    const uint32_t tk = mono_key(T);
    // the wave's candidates of all kPer rounds take one slot range (one atomic);
    // the ballots are taken again for the placement rather than kept (sixteen
    // 64-bit masks in scalar registers would cost the second workgroup per CU)
    int wcnt = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      wcnt += __popcll(__ballot(tid + u * kSelThreads < n && mono_key(rv[u]) >= tk));
    int wpos = 0;
    if (lane == 0 && wcnt) wpos = atomicAdd(&misc[0], wcnt);
    wpos = __builtin_amdgcn_readfirstlane(wpos);
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      const bool take = i < n && mono_key(rv[u]) >= tk;
      const unsigned long long m = __ballot(take);
      const int pos = wpos + __popcll(m & below);
      if (take && pos < kTopkCap) keys[pos] = make_key(rv[u], i);
      wpos += __popcll(m);
    }
    __syncthreads();
    total = misc[0];
    __syncthreads();
  }
  if (total > kTopkCap || total < k) {
    int* sel = reinterpret_cast<int*>(keys + 1024);
    radix_select_row(row, n, k, sel, reinterpret_cast<uint32_t*>(keys), misc);
    for (int i = tid; i < k; i += kSelThreads) chosen[i] = sel[i];
    __syncthreads();
  } else {
    if (tid == 0) misc[0] = 0;
    __syncthreads();
    const unsigned long long T = k > 0 ? radix_kth_u64(keys, total, k, hist, bcast) : ~0ull;
    for (int i = tid; i < total; i += kSelThreads) {
      const unsigned long long key = keys[i];
      if (key >= T) chosen[atomicAdd(&misc[0], 1)] = key_index(key);
    }
    __syncthreads();
  }
  // output in ascending index order: mark the chosen indices (all < kRowCap) in a
  // bitmap; word w's set bits go to slots from the number of bits in words < w
  for (int w2 = tid; w2 < kRowCap / 32; w2 += kSelThreads) bitmap[w2] = 0u;
  __syncthreads();
  for (int i = tid; i < k; i += kSelThreads) atomicOr(&bitmap[chosen[i] >> 5], 1u << (chosen[i] & 31));
  __syncthreads();
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
  // the chosen indices in ascending order, in LDS (chosen[] was last read before
  // the bitmap barrier), then one parallel pass maps them through the candidate
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
                     out_idx, ws.cnt, ws.cscore, ws.cidx);
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
  const float* row = scores + (size_t)r * N;
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
  if (lane < cntb) prow[(size_t)slot * PE + rank] = mine;
  else if (lane < PE) prow[(size_t)slot * PE + lane] = -1;
  if (slot == nsel - 1 && lane == 0) pool_len[r] = slot * PE + cntb;
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

}  // namespace csa2
