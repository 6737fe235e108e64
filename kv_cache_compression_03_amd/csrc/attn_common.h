// Pieces shared by the sparse-attention kernels (attn.hip, attn_f16.hip, attn_rows.hip,
// attn_split.hip, attn_wide.hip).
#pragma once

#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kKC = 32;         // keys per chunk
constexpr int kMaxSplits = 64;  // key splits a row may be cut into
constexpr int kMaxSel = 2048;   // selection slots a row may hold (all staged in LDS)

// Softmax state is kept against a reference maximum that only moves when a new
// logit exceeds it by more than 2^kLazy (log2 units), so O is rarely rescaled;
// probabilities stay below 2^kLazy, far inside float range.
constexpr float kLazy = 8.0f;

// Workgroups are dispatched to the 8 XCDs round-robin by id, and each XCD has its
// own L2.  With >= 8 rows, all workgroups of a row (its key splits and head
// groups) are placed on one XCD, so the row's queries and partial results are
// shared through that L2.  Returns false for the padding ids of the last round.
CSA2_DEV bool xcd_map(int id, int rows, int per_row, int& row, int& unit) {
  if (rows < 8) {
    row = id / per_row;
    unit = id - row * per_row;
    return row < rows;
  }
  const int x = id & 7, k = id >> 3;
  const int lr = k / per_row;
  unit = k - lr * per_row;
  row = lr * 8 + x;
  return row < rows;
}
static inline int xcd_grid(int rows, int per_row) {
  return rows < 8 ? rows * per_row : 8 * ((rows + 7) / 8) * per_row;
}

// The window buffer of a sequence is a ring of S slots: the token at position
// p >= swa_pos0 sits in slot (p - swa_pos0) mod S (a buffer filled in order from
// swa_pos0 that has not wrapped is the plain linear case).  A query at position t
// sees positions max(t - n_win + 1, swa_pos0, t - S + 1) .. t: n consecutive
// positions starting in slot `lo`, wrapping at S.  Without positions (decode)
// every slot is visible.
struct WinRange {
  int lo, n;
};
CSA2_DEV WinRange window_of(const int* q_pos, int row, int S, long long swa_pos0, int n_win) {
  if (q_pos == nullptr) return {0, S};
  const long long t = q_pos[row];
  long long lo = t - n_win + 1;
  lo = lo < swa_pos0 ? swa_pos0 : lo;
  lo = lo < t - S + 1 ? t - S + 1 : lo;
  if (S <= 0 || t < lo) return {0, 0};
  return {(int)((lo - swa_pos0) % S), (int)(t - lo + 1)};
}
// slot of the i-th visible window token (0 <= i < n <= S)
CSA2_DEV int window_slot(const WinRange& w, int i, int S) {
  const int s = w.lo + i;
  return s >= S ? s - S : s;
}

// fp16 kernel (attn_f16.hip): 32-head groups, whole selection of a split staged;
// hg2 = 32-head groups per workgroup (1 or 2, H_q / 32 a multiple of hg2).
// Usable when H_q is a multiple of 32, d is 256 or 512 and 0 < swa_scale <= 128
// (probabilities times the window scale stay inside fp16 range and are formed as
// one power of two).
bool attn_f16_supported(int H_q, int d, float swa_scale);
hipError_t launch_sparse_attn_f16(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                  int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                  int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                  int H_q, int d, float sm_log2, const AttnPlan& p, int rows,
                                  int hg2, float* part_o, float* part_ml, float* out, float* lse,
                                  hipStream_t st);

// few-rows kernel (attn_rows.hip): a row's keys inside one workgroup per (row,
// 16 heads, output-dim part); dp = 1, 2 or 4 parts (4 only for d = 512).  Usable
// when H_q is a multiple of 16, d is 256 or 512, at most 512 selection slots and
// 128 visible window tokens, and 0 < swa_scale <= 128.
bool attn_rows_supported(int H_q, int d, int K, int S, int n_win, bool with_pos, float swa_scale);
hipError_t launch_sparse_attn_rows(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                   int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                   int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                   int H_q, int d, float sm_log2, int rows, int dp, float* out,
                                   float* lse, hipStream_t st);

// few-rows path in two launches (attn_split.hip): a workgroup per (row, 32-key
// chunk) scores the chunk for all 64 heads, then a workgroup per (row, 16 heads,
// 64 dims) forms P·V.  Usable when H_q is 64, d is 512, at most 512 selection
// slots and 128 visible window tokens, and 0 < swa_scale <= 128; needs
// attn_split_ws_bytes(rows, K, S) bytes of workspace.
bool attn_split_supported(int H_q, int d, int K, int S, int n_win, bool with_pos, float swa_scale);
size_t attn_split_ws_bytes(int rows, int K, int S);
hipError_t launch_sparse_attn_split(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                    int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                    int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                    float sm_log2, int rows, void* ws, float* out, float* lse,
                                    hipStream_t st);

// many-rows kernel (attn_wide.hip): a workgroup per (row, 64 heads), each wave 16
// heads over all dims, no split partials.  Usable when H_q is a multiple of 64, d
// is 256 or 512, at most 512 selection slots, 0 < swa_scale <= 128 and a sequence's
// codes (N x d/2 bytes) and window (S x d bytes) each below 2 GiB.
bool attn_wide_supported(int H_q, int d, int K, int N, int S, float swa_scale);
hipError_t launch_sparse_attn_wide(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                   int N, const int* sel, int K, const uint8_t* swa, float swa_scale,
                                   int S, long long swa_pos0, int n_win, const int* q_pos, int Tq,
                                   int H_q, int d, float sm_log2, int rows, float* out, float* lse,
                                   hipStream_t st);

}  // namespace csa2
