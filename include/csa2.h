/*
 * csa2.h -- C ABI of the CSA2 compressed-sparse-attention layer for MI355X (gfx950).
 *
 * One CSA2 layer, as the pages on DeepSeek-V4.1-Flash describe it, cut into six
 * calls.  Sources, cited by page title and section:
 *   [deep-dive] "DeepSeek-V4.1-Flash deep dive", tanjunchen.github.io (2026-09-13):
 *               §2 projections C = H·W_KV, Z = H·W_Z; §3.1 data flow and the
 *               non-overlapping compressor; §3.2 Full / Reindex / Reuse modes and
 *               the layer schedule; §3.3 hierarchical indexer, 2,048 blocks x 8
 *               positions; §3.4 FP4 main KV after RoPE, FP8 window; §6.3 sizes.
 *   [daily]     "DeepSeek V4.1 Flash 将 KV 压缩推到模型架构层", blog.baizx.cool
 *               (2026-09-11), section 核心机制: E2M1 with one E4M3 scale per 16
 *               channels, shared candidate pool.
 *   [reading]   "DeepSeek-V4.1-Flash paper reading", inkeast.github.io, §4.2 mode
 *               table; every layer keeps its own query and window KV.
 *   [digest]    agihunt.info digest, section 已确认: selected entries are
 *               concatenated with the windowed KV before attention.
 *
 * Conventions shared by every call
 *   - All tensor arguments are DEVICE pointers to contiguous row-major buffers
 *     owned by the caller.  The library never allocates, frees or keeps a
 *     pointer after a call returns; scratch memory comes in through `ws`,
 *     sized by the matching *_workspace() query (a pure host function).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues kernels on it and returns; nothing synchronises the host.
 *   - bf16 tensors are passed as 16-bit patterns, FP8 as E4M3FN bytes (bias 7,
 *     max 448, never NaN on input), FP4 as packed E2M1 nibbles.
 *   - Indices are int32.  Top-K lists are ascending and padded with -1.
 *   - Return value: CSA2_OK or an error code.  All argument checks run before
 *     any launch, so outputs are untouched when a check fails; the reason is
 *     kept per thread in csa2_last_error().  CSA2_ERR_HIP reports a failed
 *     launch (hipGetLastError); a kernel's own faults surface at the caller's
 *     next synchronisation.
 *   - Calls are deterministic for a fixed device, shape and input.
 *   - Alignment: every pointer must be 16-byte aligned.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_API __attribute__((visibility("default")))

enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, out-of-range size */
  CSA2_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype, dim) */
  CSA2_ERR_WORKSPACE = 3,     /* ws smaller than the *_workspace() size */
  CSA2_ERR_HIP = 4            /* HIP launch error */
};

enum { CSA2_DTYPE_F32 = 0, CSA2_DTYPE_BF16 = 1 };

CSA2_API const char* csa2_version(void);
CSA2_API const char* csa2_status_string(int status);
/* Detail of the last failing call on this host thread ("" if none). */
CSA2_API const char* csa2_last_error(void);

/*
 * csa2_compress -- hidden states -> roped main-KV entries.
 * [deep-dive §2] C = H·W_KV, Z = H·W_Z; [deep-dive §3.1] each run of m tokens
 * folds into one entry, windows do not overlap, no absolute position enters the
 * fold; [deep-dive §3.4] the entries are rotated (RoPE) before quantisation.
 * Fold (reading): per channel, softmax over the m tokens of the block of Z,
 * entry = sum of weights * C.  Only complete blocks make entries.
 * Entry j of sequence b sits at position p_j = pos0 + (j+1)*m - 1; the last
 * rope_dim channels are rotated in pairs (d-r+2i, d-r+2i+1) by the angle
 * p_j * rope_theta^(-2i/r).
 *   H      [B, T, d_model]  f32 or bf16 (h_dtype)
 *   W_kv   [d_model, d]     f32 or bf16 (w_dtype, must equal h_dtype)
 *   W_z    [d_model, d_z]   d_z = d (per-channel weights) or 1 (one per token)
 *   kv_out [B, T/m, d]      f32 (T/m rounded down)
 * Float32 inputs (or d_z = 1): sums in float64, the result rounded once to
 * float32.  Bf16 inputs with d_z = d and d_model % 64 == 0: the projections run
 * on MFMA, exact bf16 products summed in float32.
 * Limits: m in {1,2,4}, d % 64 == 0, rope_dim even and <= d, pos0 % m == 0.
 */
CSA2_API int csa2_compress(const void* H, int h_dtype, int B, int T, int d_model,
                           const void* W_kv, const void* W_z, int w_dtype, int d, int d_z,
                           int m, long long pos0, int rope_dim, double rope_theta,
                           float* kv_out, void* stream);

/*
 * csa2_quant_fp4 -- FP4 main KV and the indexer key.
 * [daily 核心机制; deep-dive §3.4] E2M1 elements with one E4M3 scale per 16
 * channels; [deep-dive §3.1] the indexer K is a projection of the main KV.
 * Per group of 16 channels: s = E4M3(float32(amax / 6)) (nearest-even,
 * saturating), code = E2M1(float32(x / s)) (nearest-even, saturating, sign of x
 * kept; zero scale -> signed zero codes).
 *   kv     [n, d]    f32 entries (n = all entries of all sequences)
 *   codes  [n, d/2]  u8, byte i = code[2i] | code[2i+1] << 4
 *   scales [n, d/16] u8 E4M3
 *   W_ik   [d, d_i]  bf16 or NULL;  k_idx [n, d_i] bf16 or NULL (both or neither)
 *   k_idx = bf16(dequant(codes, scales) · W_ik): float64 sums, one rounding.
 * Limits: d % 32 == 0 and d <= 1024; d_i in {64, 128}.
 */
CSA2_API int csa2_quant_fp4(const float* kv, long long n, int d, uint8_t* codes, uint8_t* scales,
                            const void* W_ik, int d_i, void* k_idx, void* stream);

/*
 * csa2_indexer_keys -- the indexer keys of an existing FP4 cache.
 * [deep-dive §3.4] only the FP4 global KV is persisted; [deep-dive §3.1] the
 * indexer K is a projection of the main KV.  Reading: the key is formed from the
 * dequantised entry, so a cache reloaded from its codes and scales gets back
 * bit-identical keys: k_idx = bf16(dequant(codes, scales) · W_ik), float64 sums,
 * one rounding (the keys csa2_quant_fp4 writes).
 *   codes  [n, d/2] u8, scales [n, d/16] u8 E4M3 (as csa2_quant_fp4 writes them)
 *   W_ik   [d, d_i] bf16;  k_idx [n, d_i] bf16 (written)
 * Device pointers, owned by the caller; enqueued on `stream`.  Errors
 * (CSA2_ERR_INVALID_ARG / CSA2_ERR_UNSUPPORTED) are returned before any launch.
 * Limits: d % 32 == 0 and d <= 512; d_i in {64, 128}.
 */
CSA2_API int csa2_indexer_keys(const uint8_t* codes, const uint8_t* scales, long long n, int d,
                               const void* W_ik, int d_i, void* k_idx, void* stream);

/*
 * csa2_cache_append -- decode-step cache append: one new Main-KV entry per
 * sequence into row `row` of each sequence's FP4 cache (with its indexer key),
 * and the new token's window KV into slot `slot` of each layer's window.
 * [deep-dive §3.1] the compressor's entries become FP4 Main KV after RoPE
 * (§3.4) with the indexer K projected from them; [reading §4.2] every layer
 * keeps its own window of recent tokens, FP8 [deep-dive §3.4].  Quantisation
 * and key exactly as csa2_quant_fp4; window codes = E4M3(float32(win /
 * swa_scale)), nearest-even, saturating at 448, sign kept.
 *   kv     [B, d] f32: the new entries (from csa2_compress), or NULL when this
 *          token completes no entry (m > 1)
 *   codes  [B, cap, d/2], scales [B, cap, d/16]: the caches; entry b goes to
 *          row b * cap + row
 *   W_ik   [d, d_i] bf16 and k_idx [B, cap, d_i] bf16, or both NULL
 *   win    [L, B, d] f32: the token's window KV for L window buffers (L = 0: none)
 *   swa    [L, B, S, d] u8 E4M3: the windows; 0 <= slot < S (a ring: position mod S;
 *          attention without query positions reads every window token, in any order)
 * Other rows and slots are left untouched.  Limits as csa2_quant_fp4; the buffers
 * 16-byte aligned.  Calls that write the same rows concurrently race.
 */
CSA2_API int csa2_cache_append(const float* kv, int B, int d, long long cap, long long row,
                               uint8_t* codes, uint8_t* scales, const void* W_ik, int d_i,
                               void* k_idx, const float* win, int L, int S, int slot,
                               float swa_scale, uint8_t* swa, void* stream);

/*
 * csa2_index_full -- Full-mode indexer: score every visible entry, (first Full
 * layer of a decode step) build the shared candidate pool, and take the layer's
 * Top-K.
 * [deep-dive §3.1, §3.2] Indexer Q x Indexer K -> score -> Top-K;  reading: for
 * query t, s_j = sum_h w_h * max(0, q_h · k_j), accumulated in float32.
 * [deep-dive §3.3] the pool: blocks of G entries ranked by their best score,
 * the PB best blocks each give their PE best entries; union ascending.
 * Readings: Top-K ranks by (score desc, index asc) over the visible entries, min(K,
 * visible) of them, ascending, -1 padded; the Full layer's Top-K is global (not
 * restricted to the pool).
 *   q_idx  [B, Tq, h_i, d_i] bf16;  w [B, Tq, h_i] f32;  k_idx [B, N, d_i] bf16
 *   q_pos  [B, Tq] int32 query positions, or NULL (decode: every entry visible);
 *          with positions, entry j is visible to a query at t iff (j+1)*m - 1 <= t.
 *   scores [B, Tq, N] f32 out (-inf where not visible)
 *   pool   [B*Tq, PB*PE] int32 out or NULL; pool_len [B*Tq] int32 out.
 *          Rows of the pool are ascending entry indices, -1 beyond pool_len.
 *   sel    [B*Tq, K] int32 out or NULL: the Top-K of each query row.
 *   ws     >= csa2_index_full_workspace(B, Tq, N, h_i, d_i, G, PB, PE, K) bytes (pass
 *          G = 0 or PB = 0 without a pool, K = 0 without sel; 0 bytes when neither).
 * With a pool or sel, a decode-shaped call (up to 1,048,576 entries, G = 128 for
 * the pool) writes the maximum of every 32-entry span beside the scores; the pool
 * blocks and a provable lower bound of the K-th best score come from those
 * maxima, so only the pool blocks and the blocks that can hold a Top-K entry are
 * read again.
 * Limits: h_i in {4, 8, 16}, d_i in {64, 128}, G <= 256, PE <= 16, PB <= 2048,
 * K <= 2048.
 */
CSA2_API size_t csa2_index_full_workspace(int B, int Tq, int N, int h_i, int d_i, int G, int PB,
                                          int PE, int K);
CSA2_API int csa2_index_full(const void* q_idx, const float* w, const void* k_idx,
                             int B, int Tq, int N, int h_i, int d_i, const int* q_pos, int m,
                             float* scores, int* pool, int* pool_len, int G, int PB, int PE,
                             int K, int* sel, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_topk -- the K best entries of each row.
 * [deep-dive §3.3] Top-512 per query; reading: rank by (score descending, index
 * ascending), take min(K, visible), output ascending, pad with -1.
 *   scores    [R, N] f32
 *   valid_len [R] int32 or NULL: only the first valid_len[r] entries compete
 *   cand_map  [R, N] int32 or NULL: output cand_map[r][i] instead of i; each row
 *             must be ascending (so index order is kept), e.g. a candidate pool
 *   out_idx   [R, K] int32
 *   ws        >= csa2_topk_workspace(R, N, K) bytes (0 when N <= 16384)
 * Limits: 1 <= K <= 2048.  Scores must not be NaN.
 */
CSA2_API size_t csa2_topk_workspace(int R, int N, int K);
CSA2_API int csa2_topk(const float* scores, int R, int N, const int* valid_len, const int* cand_map,
                       int K, int* out_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_topk_noalloc -- csa2_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the scratch memory taken from
 * a static device array of CSA2_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends.  The caller passes only inputs and
 * outputs.  The array's address is looked up once per device, on the first call
 * with that device current.  Nothing is allocated by this call.
 *   Same arguments and limits as csa2_topk, without ws / ws_bytes.
 *   Returns CSA2_ERR_WORKSPACE (before any launch) when csa2_topk_workspace(R, N,
 *   K) exceeds CSA2_NOALLOC_SCRATCH_BYTES (about 480 rows of more than 16,384
 *   entries at K = 512).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (two streams, two host threads) race and must be ordered by the caller.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
CSA2_API int csa2_topk_noalloc(const float* scores, int R, int N, const int* valid_len,
                               const int* cand_map, int K, int* out_idx, void* stream);

/*
 * csa2_index_reindex -- Reindex mode: rescore only the shared pool with this
 * layer's own indexer query and take a fresh Top-K inside it.
 * [deep-dive §3.2, §3.3; reading §4.2] shared main KV and indexer K, fresh
 * indexer Q, search range fixed at the pool.  One query per sequence.
 *   q_idx [B, h_i, d_i] bf16;  w [B, h_i] f32;  k_idx [B, N, d_i] bf16
 *   pool  [B, P] int32 ascending entry indices;  pool_len [B] int32 (<= P)
 *   sel   [B, K] int32 out (entry indices ascending, -1 padded)
 *   ws    >= csa2_index_reindex_workspace(B, P, K) bytes
 */
CSA2_API size_t csa2_index_reindex_workspace(int B, int P, int K);
CSA2_API int csa2_index_reindex(const void* q_idx, const float* w, const void* k_idx,
                                const int* pool, const int* pool_len, int B, int P, int N,
                                int h_i, int d_i, int K, int* sel, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * csa2_sparse_attn -- main-Q attention over (selected FP4 entries ++ the layer's
 * own FP8 window).  [deep-dive §3.1] Main Q attends to the selected main KV and
 * the layer-local SWA KV; [digest 已确认] the two are concatenated;
 * [reading §4.2] each layer has its own query and window.
 * Reading: K = V = the whole dequantised entry (one KV shared by all heads);
 * one softmax over every key, logits (q·key)*sm_scale; window tokens are
 * E4M3 values times swa_scale; float32 accumulation.
 *   q      [B, Tq, H_q, d] bf16
 *   codes  [B, N, d/2], scales [B, N, d/16]: the FP4 main KV
 *   sel    [B, Tq, K] int32 ascending entry indices, -1 padded
 *   swa    [B, S, d] E4M3 window tokens, a ring of S slots: the token at
 *          position p >= swa_pos0 sits in slot (p - swa_pos0) mod S (a buffer
 *          filled in order from swa_pos0 that has not wrapped is the linear case,
 *          slot i = position swa_pos0 + i; csa2_cache_append's slot p mod S is the
 *          ring with swa_pos0 = 0).
 *   q_pos  [B, Tq] int32 or NULL.  With positions, a query at t sees the window
 *          tokens at positions max(t - n_win + 1, swa_pos0, t - S + 1) .. t; the
 *          caller keeps every position a query can see in its slot (S >= n_win +
 *          the number of later positions already written).  Without positions
 *          every one of the S slots is visible.
 *   out    [B, Tq, H_q, d] f32;  lse [B, Tq, H_q] f32 natural-log sum-exp or NULL
 *   sm_scale <= 0 selects 1/sqrt(d).
 *   ws     >= csa2_sparse_attn_workspace(B, Tq, H_q, d, K, S) bytes, device memory
 *          owned by the caller (NULL when that is 0); its contents need no set-up
 * Limits: d in {256, 512}, H_q % 16 == 0, K <= 2048.
 * Kernels, for 16-byte aligned q, out and caches, at most 512 selection slots
 * and 0 < swa_scale <= 128 (fp16 products, probabilities with 11 significant
 * bits, queries scaled into fp16 by a power of two per head):
 *   - up to 8 query rows at H_q = 64 and d = 512 with at most 128 visible window
 *     tokens: two launches; a workgroup per (row, 32-key chunk) scores the chunk
 *     once for all heads and leaves fp16 probabilities, the chunk's (max, sum)
 *     per head and its decoded values in ws, then a workgroup per (row, 16
 *     heads, 64 dims) merges the chunks and forms the output;
 *   - otherwise up to 64 query rows with at most 128 visible window tokens: all
 *     keys of a row inside one workgroup per (row, 16 heads, part of the dims),
 *     no partials, ws unused;
 *   - otherwise, with H_q % 64 == 0 and at least 65 (row, 64 heads) units: a
 *     workgroup per (row, 64 heads), no partials, ws unused.
 * Otherwise a split-K kernel and a merge launch, the partials in ws.
 * Precision: products are exact (entries, window values and probabilities are
 * carried in fp16 or bf16, both exact for the decoded values) and accumulate in
 * fp32.  When H_q % 32 == 0, 0 < swa_scale <= 128 and codes, scales and swa are
 * 16-byte aligned, the fp16 kernel runs (probabilities with 11 significant bits,
 * queries scaled into fp16 by a power of two per head); otherwise the bf16
 * kernel (probabilities as a bf16 pair, 16 bits).
 */
CSA2_API size_t csa2_sparse_attn_workspace(int B, int Tq, int H_q, int d, int K, int S);
CSA2_API int csa2_sparse_attn(const void* q, const uint8_t* codes, const uint8_t* scales, int N,
                              const int* sel, int K, const uint8_t* swa, float swa_scale, int S,
                              long long swa_pos0, int n_win, const int* q_pos, int B, int Tq,
                              int H_q, int d, float sm_scale, float* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
