// Launchers of the CSA2 kernels, called by the C ABI layer (api.cpp) after it has
// validated every argument.  Each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

constexpr int kTopkCap = 8192;  // candidates a Top-K row sorts in LDS
constexpr int kTmaxSpan = 32;   // entries per score maximum the decode scan writes

// quant.hip
// Entry e of the input goes to cache row e * cap + row (defaults: contiguous).
hipError_t launch_quant_fp4(const float* kv, long long n, int d, uint8_t* codes, uint8_t* scales,
                            hipStream_t st, long long cap = 1, long long row = 0);
hipError_t launch_indexer_k(const uint8_t* codes, const uint8_t* scales, long long n, int d,
                            const uint16_t* W_ik, int d_i, uint16_t* k_idx, hipStream_t st,
                            long long cap = 1, long long row = 0);
// win [L, B, d] f32 -> E4M3 codes of win / swa_scale in swa[l][b][slot] ([L, B, S, d]).
// quantiser + indexer keys + window encode of a decode-step append in one launch
// (at most 256 entries, d <= 512, W_ik 16-byte aligned); win may be null (L = 0)
bool cache_append_fused_ok(int B, int d, int d_i, const void* W_ik);
hipError_t launch_cache_append(const float* kv, int B, int d, long long cap, long long row, uint8_t* codes,
                               uint8_t* scales, const uint16_t* W_ik, int d_i, uint16_t* k_idx,
                               const float* win, int L, int S, int slot, float swa_scale, uint8_t* swa,
                               hipStream_t st);
hipError_t launch_swa_append(const float* win, int L, int B, int S, int d, int slot, float swa_scale,
                             uint8_t* swa, hipStream_t st);

// compress.hip
hipError_t launch_compress(const void* H, bool bf16_in, int B, int T, int d_model, const void* W_kv,
                           const void* W_z, int d, int d_z, int m, long long pos0, int rope_dim,
                           double rope_theta, float* kv_out, hipStream_t st);

// index.hip: scores[b, t, i] for rows i < L of sequence b (rows gathered through
// `gather` when not null).
// Prefill indexer (index_prefill.hip): many queries, no gather.
bool index_prefill_supported(int Tq, int N, int h_i, int d_i, const int* gather);
hipError_t launch_index_prefill(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                const int* q_pos, int m, int B, int Tq, int N, int h_i, int d_i,
                                float* scores, hipStream_t st);
// tmax (optional): [B*Tq, ceil(L/kTmaxSpan)] maxima of each kTmaxSpan-entry span of
// every score row (-inf entries included), written with the scores; it takes the
// decode scan even for many queries.
hipError_t launch_index_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                               const int* gather, const int* gather_len, const int* q_pos, int m,
                               int B, int Tq, int N, int L, int h_i, int d_i, float* scores,
                               hipStream_t st, float* tmax = nullptr);

// topk.hip
struct TopkWs {
  float* cmax;      // [R, 2K]
  int* cnt;         // [R]
  float* cscore;    // [R, cap]
  int* cidx;        // [R, cap]
};
size_t topk_ws_bytes(int R, int N, int K);
TopkWs topk_ws_carve(void* ws, int R, int K);
hipError_t launch_topk(const float* scores, int R, int N, const int* valid_len, const int* cand_map,
                       int K, int* out_idx, const TopkWs& ws, hipStream_t st);

// pool (topk.hip)
size_t pool_ws_bytes(int R, int N, int G, int PB);
hipError_t launch_pool(const float* scores, int R, int N, const int* q_pos, int m, int G, int PB,
                       int PE, int* pool, int* pool_len, void* ws, hipStream_t st);

// Full-layer selection from the decode scan's tile maxima (topk.hip): the pool
// (PB best 128-entry blocks, PE best entries each; pool may be null) and the
// Top-K (sel [R, K]; may be null) of every row, visibility from q_pos / m.  The
// workspace starts with the tile maxima the scan writes (full_select_tmax).
bool full_select_supported(int N, int G);
size_t full_select_ws_bytes(int R, int N, int PB, int K);
float* full_select_tmax(void* ws);
hipError_t launch_full_select(const float* scores, int R, int N, const int* q_pos, int m, int PB,
                              int PE, int* pool, int* pool_len, int K, int* sel, void* ws,
                              hipStream_t st);
// vlen[r] = entries visible to row r (q_pos null: N)
hipError_t launch_visible_len(const int* q_pos, int m, int R, int N, int* vlen, hipStream_t st);

// attn.hip
struct AttnPlan {
  int waves, head_groups, n_splits, chunks_per_split;
};
AttnPlan attn_plan(int B, int Tq, int H_q, int K, int S);
size_t attn_ws_bytes(int B, int Tq, int H_q, int d, int K, int S);
hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, int N,
                              const int* sel, int K, const uint8_t* swa, float swa_scale, int S,
                              long long swa_pos0, int n_win, const int* q_pos, int B, int Tq,
                              int H_q, int d, float sm_scale, float* out, float* lse, void* ws,
                              hipStream_t st);

}  // namespace csa2
