// C ABI of the CSA2 library: argument checks, workspace sizes, kernel dispatch.
// Every check runs before any HIP call, so a rejected call touches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/csa2.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return CSA2_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED_PTR(p)                                                                   \
  do {                                                                                \
    if ((p) == nullptr) return fail(CSA2_ERR_INVALID_ARG, "%s: " #p " is null", fn); \
    if (!aligned16(p)) return fail(CSA2_ERR_INVALID_ARG, "%s: " #p " is not 16-byte aligned", fn); \
  } while (0)
#define OPT_PTR(p)                                                                    \
  do {                                                                                \
    if ((p) != nullptr && !aligned16(p))                                              \
      return fail(CSA2_ERR_INVALID_ARG, "%s: " #p " is not 16-byte aligned", fn);     \
  } while (0)
#define CHECK(cond, code, ...)                      \
  do {                                              \
    if (!(cond)) return fail((code), __VA_ARGS__);  \
  } while (0)

int hip_status(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" {

CSA2_API const char* csa2_version(void) { return "csa2-mi355x 0.1.0 (gfx950)"; }

CSA2_API const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported";
    case CSA2_ERR_WORKSPACE: return "workspace too small";
    case CSA2_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

CSA2_API const char* csa2_last_error(void) { return g_err; }

// ------------------------------------------------------------------ compress

CSA2_API int csa2_compress(const void* H, int h_dtype, int B, int T, int d_model, const void* W_kv,
                           const void* W_z, int w_dtype, int d, int d_z, int m, long long pos0,
                           int rope_dim, double rope_theta, float* kv_out, void* stream) {
  const char* fn = "csa2_compress";
  CHECK(B >= 0 && T >= 0 && d_model > 0, CSA2_ERR_INVALID_ARG, "%s: bad B/T/d_model", fn);
  CHECK(h_dtype == CSA2_DTYPE_F32 || h_dtype == CSA2_DTYPE_BF16, CSA2_ERR_UNSUPPORTED,
        "%s: h_dtype must be F32 or BF16", fn);
  CHECK(w_dtype == h_dtype, CSA2_ERR_UNSUPPORTED, "%s: w_dtype must equal h_dtype", fn);
  CHECK(m == 1 || m == 2 || m == 4, CSA2_ERR_UNSUPPORTED, "%s: m must be 1, 2 or 4", fn);
  CHECK(d > 0 && d % 64 == 0, CSA2_ERR_UNSUPPORTED, "%s: d must be a positive multiple of 64", fn);
  CHECK(d_z == d || d_z == 1, CSA2_ERR_INVALID_ARG, "%s: d_z must be d or 1", fn);
  CHECK(rope_dim >= 0 && rope_dim % 2 == 0 && rope_dim <= d, CSA2_ERR_INVALID_ARG,
        "%s: rope_dim must be even and <= d", fn);
  CHECK(rope_dim == 0 || rope_theta > 0.0, CSA2_ERR_INVALID_ARG, "%s: rope_theta must be > 0", fn);
  CHECK(pos0 >= 0 && pos0 % m == 0, CSA2_ERR_INVALID_ARG, "%s: pos0 must be >= 0 and a multiple of m", fn);
  if ((long long)B * (T / m) == 0) return ok();
  NEED_PTR(H);
  NEED_PTR(W_kv);
  NEED_PTR(W_z);
  NEED_PTR(kv_out);
  return hip_status(csa2::launch_compress(H, h_dtype == CSA2_DTYPE_BF16, B, T, d_model, W_kv, W_z, d,
                                          d_z, m, pos0, rope_dim, rope_theta, kv_out, S(stream)),
                    fn);
}

// ------------------------------------------------------------------ quantisation

CSA2_API int csa2_quant_fp4(const float* kv, long long n, int d, uint8_t* codes, uint8_t* scales,
                            const void* W_ik, int d_i, void* k_idx, void* stream) {
  const char* fn = "csa2_quant_fp4";
  CHECK(n >= 0, CSA2_ERR_INVALID_ARG, "%s: n < 0", fn);
  CHECK(d > 0 && d % 32 == 0 && d <= 1024, CSA2_ERR_UNSUPPORTED, "%s: d must be a multiple of 32 in [32, 1024]", fn);
  CHECK((W_ik == nullptr) == (k_idx == nullptr), CSA2_ERR_INVALID_ARG,
        "%s: W_ik and k_idx must both be given or both be null", fn);
  if (W_ik) {
    CHECK(d_i == 64 || d_i == 128, CSA2_ERR_UNSUPPORTED, "%s: d_i must be 64 or 128", fn);
    CHECK(d <= 512, CSA2_ERR_UNSUPPORTED, "%s: the indexer-key projection needs d <= 512", fn);
  }
  if (n == 0) return ok();
  NEED_PTR(kv);
  NEED_PTR(codes);
  NEED_PTR(scales);
  OPT_PTR(W_ik);
  OPT_PTR(k_idx);
  hipError_t e = csa2::launch_quant_fp4(kv, n, d, codes, scales, S(stream));
  if (e == hipSuccess && W_ik)
    e = csa2::launch_indexer_k(codes, scales, n, d, static_cast<const uint16_t*>(W_ik), d_i,
                               static_cast<uint16_t*>(k_idx), S(stream));
  return hip_status(e, fn);
}

CSA2_API int csa2_indexer_keys(const uint8_t* codes, const uint8_t* scales, long long n, int d,
                               const void* W_ik, int d_i, void* k_idx, void* stream) {
  const char* fn = "csa2_indexer_keys";
  CHECK(n >= 0, CSA2_ERR_INVALID_ARG, "%s: n < 0", fn);
  CHECK(d > 0 && d % 32 == 0 && d <= 512, CSA2_ERR_UNSUPPORTED, "%s: d must be a multiple of 32 in [32, 512]", fn);
  CHECK(d_i == 64 || d_i == 128, CSA2_ERR_UNSUPPORTED, "%s: d_i must be 64 or 128", fn);
  if (n == 0) return ok();
  NEED_PTR(codes);
  NEED_PTR(scales);
  NEED_PTR(W_ik);
  NEED_PTR(k_idx);
  return hip_status(csa2::launch_indexer_k(codes, scales, n, d, static_cast<const uint16_t*>(W_ik), d_i,
                                           static_cast<uint16_t*>(k_idx), S(stream)),
                    fn);
}

// ------------------------------------------------------------------ decode cache append

CSA2_API int csa2_cache_append(const float* kv, int B, int d, long long cap, long long row,
                               uint8_t* codes, uint8_t* scales, const void* W_ik, int d_i,
                               void* k_idx, const float* win, int L, int S_, int slot,
                               float swa_scale, uint8_t* swa, void* stream) {
  const char* fn = "csa2_cache_append";
  CHECK(B >= 0 && L >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(d > 0 && d % 32 == 0 && d <= 1024, CSA2_ERR_UNSUPPORTED, "%s: d must be a multiple of 32 in [32, 1024]", fn);
  CHECK((W_ik == nullptr) == (k_idx == nullptr), CSA2_ERR_INVALID_ARG,
        "%s: W_ik and k_idx must both be given or both be null", fn);
  if (W_ik) {
    CHECK(d_i == 64 || d_i == 128, CSA2_ERR_UNSUPPORTED, "%s: d_i must be 64 or 128", fn);
    CHECK(d <= 512, CSA2_ERR_UNSUPPORTED, "%s: the indexer-key projection needs d <= 512", fn);
  }
  if (kv) CHECK(cap >= 1 && row >= 0 && row < cap, CSA2_ERR_INVALID_ARG, "%s: row must be in [0, cap)", fn);
  if (L > 0) {
    CHECK(S_ >= 1 && slot >= 0 && slot < S_, CSA2_ERR_INVALID_ARG, "%s: slot must be in [0, S)", fn);
    CHECK(std::isfinite(swa_scale) && swa_scale > 0.0f, CSA2_ERR_INVALID_ARG,
          "%s: swa_scale must be finite and > 0", fn);
  }
  if (B == 0) return ok();
  OPT_PTR(kv);
  OPT_PTR(W_ik);
  OPT_PTR(k_idx);
  if (kv) {
    NEED_PTR(codes);
    NEED_PTR(scales);
  }
  if (L > 0) {
    NEED_PTR(win);
    NEED_PTR(swa);
  }
  hipError_t e = hipSuccess;
  if (kv && W_ik && csa2::cache_append_fused_ok(B, d, d_i, W_ik))   // one launch for all of it
    return hip_status(csa2::launch_cache_append(kv, B, d, cap, row, codes, scales,
                                                static_cast<const uint16_t*>(W_ik), d_i,
                                                static_cast<uint16_t*>(k_idx), L > 0 ? win : nullptr, L,
                                                S_, slot, swa_scale, swa, S(stream)),
                      fn);
  if (kv) {
    e = csa2::launch_quant_fp4(kv, B, d, codes, scales, S(stream), cap, row);
    if (e == hipSuccess && W_ik)
      e = csa2::launch_indexer_k(codes, scales, B, d, static_cast<const uint16_t*>(W_ik), d_i,
                                 static_cast<uint16_t*>(k_idx), S(stream), cap, row);
  }
  if (e == hipSuccess && L > 0) e = csa2::launch_swa_append(win, L, B, S_, d, slot, swa_scale, swa, S(stream));
  return hip_status(e, fn);
}

// ------------------------------------------------------------------ Full-mode indexer

static bool index_dims_ok(int h_i, int d_i) {
  return (h_i == 4 || h_i == 8 || h_i == 16) && (d_i == 64 || d_i == 128);
}

// Workspace of csa2_index_full for the way the call runs: the decode scan with
// the Full-layer selection from its tile maxima, or the scores first and then the
// separate pool and Top-K passes (prefill-shaped calls, other block sizes).
static bool index_full_fused(int Tq, int N, int h_i, int d_i, int G, bool pool, bool sel) {
  return (pool || sel) && !csa2::index_prefill_supported(Tq, N, h_i, d_i, nullptr) &&
         csa2::full_select_supported(N, pool ? G : 128);
}

static size_t index_full_ws(int B, int Tq, int N, int h_i, int d_i, int G, int PB, int K, bool pool,
                            bool sel) {
  const int R = B * Tq;
  if (!pool && !sel) return 0;
  if (index_full_fused(Tq, N, h_i, d_i, G, pool, sel))
    return csa2::full_select_ws_bytes(R, N, pool ? PB : 0, sel ? K : 0);
  size_t a = pool ? csa2::pool_ws_bytes(R, N, G, PB) : 0;
  size_t b = sel ? csa2::topk_ws_bytes(R, N, K) : 0;
  return align256((size_t)R * sizeof(int)) + (a > b ? a : b);  // visible entries per row first
}

CSA2_API size_t csa2_index_full_workspace(int B, int Tq, int N, int h_i, int d_i, int G, int PB,
                                          int PE, int K) {
  (void)PE;
  if (B <= 0 || Tq <= 0 || N <= 0) return 0;
  const bool pool = G > 0 && PB > 0, sel = K > 0;
  return index_full_ws(B, Tq, N, h_i, d_i, G, PB, K, pool, sel);
}

CSA2_API int csa2_index_full(const void* q_idx, const float* w, const void* k_idx, int B, int Tq,
                             int N, int h_i, int d_i, const int* q_pos, int m, float* scores,
                             int* pool, int* pool_len, int G, int PB, int PE, int K, int* sel,
                             void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa2_index_full";
  CHECK(B >= 0 && Tq >= 0 && N >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(B <= 65535 && (long long)B * Tq <= 65535 && (long long)N < (1LL << 31) - 1,
        CSA2_ERR_INVALID_ARG, "%s: B*Tq must be <= 65535", fn);
  CHECK(index_dims_ok(h_i, d_i), CSA2_ERR_UNSUPPORTED, "%s: h_i must be 4/8/16 and d_i 64/128", fn);
  CHECK(q_pos == nullptr || m >= 1, CSA2_ERR_INVALID_ARG, "%s: m must be >= 1 with positions", fn);
  if (pool) {
    CHECK(pool_len != nullptr, CSA2_ERR_INVALID_ARG, "%s: pool_len is null", fn);
    CHECK(G >= 1 && G <= 256, CSA2_ERR_UNSUPPORTED, "%s: G must be in [1, 256]", fn);
    CHECK(PE >= 1 && PE <= 16, CSA2_ERR_UNSUPPORTED, "%s: PE must be in [1, 16]", fn);
    CHECK(PB >= 1 && PB <= 2048, CSA2_ERR_UNSUPPORTED, "%s: PB must be in [1, 2048]", fn);
  }
  if (sel) CHECK(K >= 1 && K <= 2048, CSA2_ERR_UNSUPPORTED, "%s: K must be in [1, 2048]", fn);
  const size_t need = (long long)B * Tq * N == 0
                          ? 0
                          : index_full_ws(B, Tq, N, h_i, d_i, G, PB, K, pool != nullptr, sel != nullptr);
  CHECK(ws_bytes >= need, CSA2_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  CHECK(need == 0 || ws != nullptr, CSA2_ERR_WORKSPACE, "%s: workspace is null", fn);
  OPT_PTR(ws);
  if ((long long)B * Tq * N == 0) return ok();
  NEED_PTR(q_idx);
  NEED_PTR(w);
  NEED_PTR(k_idx);
  NEED_PTR(scores);
  OPT_PTR(q_pos);
  OPT_PTR(pool);
  OPT_PTR(pool_len);
  OPT_PTR(sel);
  const int R = B * Tq;
  const auto* q16 = static_cast<const uint16_t*>(q_idx);
  const auto* k16 = static_cast<const uint16_t*>(k_idx);
  if (index_full_fused(Tq, N, h_i, d_i, G, pool != nullptr, sel != nullptr)) {
    // decode scan writing tile maxima, then pool and Top-K from them
    hipError_t e = csa2::launch_index_scores(q16, w, k16, nullptr, nullptr, q_pos, m, B, Tq, N, N, h_i,
                                             d_i, scores, S(stream), csa2::full_select_tmax(ws));
    if (e == hipSuccess)
      e = csa2::launch_full_select(scores, R, N, q_pos, m, pool ? PB : 0, PE, pool, pool_len,
                                   sel ? K : 0, sel, ws, S(stream));
    return hip_status(e, fn);
  }
  hipError_t e = csa2::launch_index_scores(q16, w, k16, nullptr, nullptr, q_pos, m, B, Tq, N, N, h_i,
                                           d_i, scores, S(stream));
  if (e == hipSuccess && pool) {
    char* base = static_cast<char*>(ws) + align256((size_t)R * sizeof(int));
    e = csa2::launch_pool(scores, R, N, q_pos, m, G, PB, PE, pool, pool_len, base, S(stream));
  }
  if (e == hipSuccess && sel) {
    int* vlen = static_cast<int*>(ws);
    e = csa2::launch_visible_len(q_pos, m, R, N, vlen, S(stream));
    csa2::TopkWs tw{};
    if (e == hipSuccess && csa2::topk_ws_bytes(R, N, K))
      tw = csa2::topk_ws_carve(static_cast<char*>(ws) + align256((size_t)R * sizeof(int)), R, K);
    if (e == hipSuccess) e = csa2::launch_topk(scores, R, N, vlen, nullptr, K, sel, tw, S(stream));
  }
  return hip_status(e, fn);
}

// ------------------------------------------------------------------ Top-K

CSA2_API size_t csa2_topk_workspace(int R, int N, int K) {
  if (R <= 0 || N <= 0 || K <= 0) return 0;
  return csa2::topk_ws_bytes(R, N, K);
}

CSA2_API int csa2_topk(const float* scores, int R, int N, const int* valid_len, const int* cand_map,
                       int K, int* out_idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa2_topk";
  CHECK(R >= 0 && N >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(K >= 1 && K <= 2048, CSA2_ERR_UNSUPPORTED, "%s: K must be in [1, 2048]", fn);
  CHECK((long long)N < (1LL << 31) - 1 && R <= 65535, CSA2_ERR_INVALID_ARG, "%s: N or R too large", fn);
  if (R == 0) return ok();
  const size_t need = csa2_topk_workspace(R, N, K);
  CHECK(ws_bytes >= need, CSA2_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  CHECK(need == 0 || ws != nullptr, CSA2_ERR_WORKSPACE, "%s: workspace is null", fn);
  NEED_PTR(out_idx);
  if (N > 0) NEED_PTR(scores);
  OPT_PTR(valid_len);
  OPT_PTR(cand_map);
  OPT_PTR(ws);
  csa2::TopkWs tw{};
  if (need) tw = csa2::topk_ws_carve(ws, R, K);
  return hip_status(csa2::launch_topk(scores, R, N, valid_len, cand_map, K, out_idx, tw, S(stream)), fn);
}

}  // extern "C"

// ------------------------------------------------------------------ Top-K without allocation

// Scratch of csa2_topk_noalloc: one copy per GPU, held until the process ends.
// On the host `scratch` names a host-side stand-in, never the device memory:
// every use on the host goes through the address hipGetSymbolAddress returns for
// the current device.
static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  CHECK(dev >= 0 && dev < kMaxDevices, CSA2_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev,
        kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CSA2_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" {

CSA2_API int csa2_topk_noalloc(const float* scores, int R, int N, const int* valid_len,
                               const int* cand_map, int K, int* out_idx, void* stream) {
  const char* fn = "csa2_topk_noalloc";
  CHECK(R >= 0 && N >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(K >= 1 && K <= 2048, CSA2_ERR_UNSUPPORTED, "%s: K must be in [1, 2048]", fn);
  CHECK((long long)N < (1LL << 31) - 1 && R <= 65535, CSA2_ERR_INVALID_ARG, "%s: N or R too large", fn);
  if (R == 0) return ok();
  const size_t need = csa2_topk_workspace(R, N, K);
  CHECK(need <= CSA2_NOALLOC_SCRATCH_BYTES, CSA2_ERR_WORKSPACE,
        "%s: %d rows of %d entries need %zu bytes of scratch, the static array holds %zu", fn, R, N,
        need, (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
  NEED_PTR(out_idx);
  if (N > 0) NEED_PTR(scores);
  OPT_PTR(valid_len);
  OPT_PTR(cand_map);
  csa2::TopkWs tw{};
  if (need) {
    void* base = nullptr;
    const int st = scratch_address(&base, fn);
    if (st != CSA2_OK) return st;
    tw = csa2::topk_ws_carve(base, R, K);
  }
  return hip_status(csa2::launch_topk(scores, R, N, valid_len, cand_map, K, out_idx, tw, S(stream)), fn);
}

// ------------------------------------------------------------------ Reindex

CSA2_API size_t csa2_index_reindex_workspace(int B, int P, int K) {
  if (B <= 0 || P <= 0 || K <= 0) return 0;
  return align256((size_t)B * P * sizeof(float)) + csa2::topk_ws_bytes(B, P, K);
}

CSA2_API int csa2_index_reindex(const void* q_idx, const float* w, const void* k_idx, const int* pool,
                                const int* pool_len, int B, int P, int N, int h_i, int d_i, int K,
                                int* sel, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa2_index_reindex";
  CHECK(B >= 0 && P >= 0 && N >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(index_dims_ok(h_i, d_i), CSA2_ERR_UNSUPPORTED, "%s: h_i must be 4/8/16 and d_i 64/128", fn);
  CHECK(K >= 1 && K <= 2048, CSA2_ERR_UNSUPPORTED, "%s: K must be in [1, 2048]", fn);
  CHECK(B <= 65535, CSA2_ERR_INVALID_ARG, "%s: B must be <= 65535", fn);
  if (B == 0) return ok();
  CHECK(P >= 1, CSA2_ERR_INVALID_ARG, "%s: P must be >= 1", fn);
  const size_t need = csa2_index_reindex_workspace(B, P, K);
  CHECK(ws_bytes >= need, CSA2_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  NEED_PTR(ws);
  NEED_PTR(q_idx);
  NEED_PTR(w);
  NEED_PTR(k_idx);
  NEED_PTR(pool);
  NEED_PTR(pool_len);
  NEED_PTR(sel);
  float* sc = static_cast<float*>(ws);
  void* tws_base = static_cast<char*>(ws) + align256((size_t)B * P * sizeof(float));
  csa2::TopkWs tw{};
  if (csa2::topk_ws_bytes(B, P, K)) tw = csa2::topk_ws_carve(tws_base, B, K);
  // pool entries must index the key cache: pool values are checked on the device
  // (rows outside [0, N) would not be gathered) -- see launch_index_scores.
  hipError_t e = csa2::launch_index_scores(static_cast<const uint16_t*>(q_idx), w,
                                           static_cast<const uint16_t*>(k_idx), pool, pool_len,
                                           nullptr, 1, B, 1, N, P, h_i, d_i, sc, S(stream));
  if (e == hipSuccess) e = csa2::launch_topk(sc, B, P, pool_len, pool, K, sel, tw, S(stream));
  return hip_status(e, fn);
}

// ------------------------------------------------------------------ sparse attention

CSA2_API size_t csa2_sparse_attn_workspace(int B, int Tq, int H_q, int d, int K, int S_) {
  if (B <= 0 || Tq <= 0 || H_q <= 0 || d <= 0 || K < 0 || S_ < 0) return 0;
  if (H_q % 16) return 0;
  return csa2::attn_ws_bytes(B, Tq, H_q, d, K, K + S_);
}

CSA2_API int csa2_sparse_attn(const void* q, const uint8_t* codes, const uint8_t* scales, int N,
                              const int* sel, int K, const uint8_t* swa, float swa_scale, int S_,
                              long long swa_pos0, int n_win, const int* q_pos, int B, int Tq,
                              int H_q, int d, float sm_scale, float* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  const char* fn = "csa2_sparse_attn";
  CHECK(B >= 0 && Tq >= 0 && N >= 0 && S_ >= 0 && K >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(d == 256 || d == 512, CSA2_ERR_UNSUPPORTED, "%s: d must be 256 or 512", fn);
  CHECK(H_q > 0 && H_q % 16 == 0, CSA2_ERR_UNSUPPORTED, "%s: H_q must be a positive multiple of 16", fn);
  CHECK(K <= 2048, CSA2_ERR_UNSUPPORTED, "%s: K must be <= 2048", fn);
  CHECK(q_pos == nullptr || n_win >= 1, CSA2_ERR_INVALID_ARG, "%s: n_win must be >= 1", fn);
  CHECK((long long)B * Tq <= 65535, CSA2_ERR_INVALID_ARG, "%s: B*Tq must be <= 65535", fn);
  CHECK(std::isfinite(swa_scale), CSA2_ERR_INVALID_ARG, "%s: swa_scale must be finite", fn);
  if ((long long)B * Tq == 0) return ok();
  const size_t need = csa2_sparse_attn_workspace(B, Tq, H_q, d, K, S_);
  CHECK(ws_bytes >= need, CSA2_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  CHECK(need == 0 || ws != nullptr, CSA2_ERR_WORKSPACE, "%s: workspace is null", fn);
  NEED_PTR(q);
  NEED_PTR(out);
  if (K > 0) NEED_PTR(sel);
  if (K > 0 && N > 0) {
    NEED_PTR(codes);
    NEED_PTR(scales);
  }
  if (S_ > 0) NEED_PTR(swa);
  OPT_PTR(q_pos);
  OPT_PTR(lse);
  OPT_PTR(ws);
  const float sc = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt((float)d);
  return hip_status(csa2::launch_sparse_attn(static_cast<const uint16_t*>(q), codes, scales, N, sel, K,
                                             swa, swa_scale, S_, swa_pos0, n_win, q_pos, B, Tq, H_q,
                                             d, sc, out, lse, ws, S(stream)),
                    fn);
}

}  // extern "C"
