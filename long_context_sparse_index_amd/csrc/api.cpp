// C ABI of libdsa (declared in include/dsa.h): argument validation, dispatch to the gfx950
// kernels, and the query-chunked forward driver.  Nothing here allocates or synchronises;
// every launch goes on the caller's stream.  A shape without a kernel is an error, never a
// fallback (page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens",
// section "Four optimizations", item 1, shows what a silent dense fallback costs).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

dsa_status ok() {
  g_last_error[0] = '\0';
  return DSA_OK;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxI32 = (int64_t{1} << 31) - 1;

size_t align256(size_t n) { return (n + 255) & ~size_t{255}; }

int64_t score_ld(int64_t n_pools) { return ((n_pools > 0 ? n_pools : 1) + 3) & ~int64_t{3}; }

#define DSA_REQUIRE(cond, ...) \
  do {                         \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

dsa_status check_index_args(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            int64_t n_pools, int32_t h_i, int32_t d_i, int32_t dtype) {
  DSA_REQUIRE(q_idx && k_idx && w, "index: null q_idx, k_idx or w");
  DSA_REQUIRE(dtype == DSA_DTYPE_BF16 || dtype == DSA_DTYPE_FP8_E4M3, "index: bad dtype %d",
              dtype);
  DSA_REQUIRE(h_i >= 1 && d_i >= 1, "index: h_i and d_i must be positive");
  DSA_REQUIRE(n_pools >= 0 && n_pools <= kMaxI32, "index: n_pools out of range");
  if (h_i > dsa::indexer_max_heads())
    return fail(DSA_ERR_UNSUPPORTED, "index: h_i = %d > %d", h_i, dsa::indexer_max_heads());
  if (!dsa::indexer_supported(d_i, dtype))
    return fail(DSA_ERR_UNSUPPORTED, "index: no kernel for d_i = %d with dtype %d", d_i, dtype);
  const int64_t elt = dtype == DSA_DTYPE_BF16 ? 2 : 1;
  DSA_REQUIRE(q_row_stride >= int64_t{h_i} * d_i, "index: q_row_stride < h_i * d_i");
  DSA_REQUIRE(k_row_stride >= d_i, "index: k_row_stride < d_i");
  DSA_REQUIRE(w_row_stride == 0 || w_row_stride >= h_i, "index: w_row_stride must be 0 or >= h_i");
  DSA_REQUIRE(aligned(q_idx, 16) && aligned(k_idx, 16) && aligned(w, 4),
              "index: q_idx/k_idx must be 16-byte aligned, w 4-byte aligned");
  DSA_REQUIRE((q_row_stride * elt) % 16 == 0 && (k_row_stride * elt) % 16 == 0,
              "index: row strides must be multiples of 16 bytes");
  return DSA_OK;
}

dsa_status check_scores(const float* scores, int64_t ld, int64_t n_pools) {
  DSA_REQUIRE(scores, "null scores");
  DSA_REQUIRE(ld >= n_pools && ld % 4 == 0, "ld_scores must be >= n_pools and a multiple of 4");
  DSA_REQUIRE(aligned(scores, 16), "scores must be 16-byte aligned");
  return DSA_OK;
}

dsa_status check_topk_args(int64_t n_pools, int32_t k, const int32_t* idx) {
  DSA_REQUIRE(idx && aligned(idx, 4), "topk: null or misaligned idx");
  DSA_REQUIRE(n_pools >= 0 && n_pools <= kMaxI32, "topk: n_pools out of range");
  DSA_REQUIRE(k >= 1, "topk: k must be >= 1");
  if (k > dsa::topk_max_k())
    return fail(DSA_ERR_UNSUPPORTED, "topk: k = %d > %d", k, dsa::topk_max_k());
  return DSA_OK;
}

dsa_status check_attn_args(const void* q, const void* kv, int64_t ld_kv, const void* v,
                           int64_t ld_v, const int32_t* idx, int32_t k, int64_t n_pools,
                           int32_t h, int32_t d_qk, int32_t d_v, float scale) {
  DSA_REQUIRE(q && kv && idx, "attn: null q, kv or idx");
  DSA_REQUIRE(h >= 1 && d_qk >= 1 && d_v >= 1 && k >= 1, "attn: h, d_qk, d_v, k must be >= 1");
  DSA_REQUIRE(n_pools >= 0 && n_pools <= kMaxI32, "attn: n_pools out of range");
  DSA_REQUIRE(std::isfinite(scale), "attn: scale must be finite");
  if (h > 64) return fail(DSA_ERR_UNSUPPORTED, "attn: h = %d > 64", h);
  if (!dsa::attn_shape_supported(d_qk, d_v))
    return fail(DSA_ERR_UNSUPPORTED, "attn: no kernel for d_qk = %d, d_v = %d", d_qk, d_v);
  if (k > dsa::attn_max_k())
    return fail(DSA_ERR_UNSUPPORTED, "attn: k = %d > %d", k, dsa::attn_max_k());
  DSA_REQUIRE(ld_kv >= d_qk && ld_kv % 8 == 0, "attn: ld_kv must be >= d_qk, multiple of 8");
  DSA_REQUIRE(aligned(q, 16) && aligned(kv, 16) && aligned(idx, 4),
              "attn: q, kv must be 16-byte aligned, idx 4-byte aligned");
  if (v) {
    DSA_REQUIRE(ld_v >= d_v && ld_v % 8 == 0, "attn: ld_v must be >= d_v, multiple of 8");
    DSA_REQUIRE(aligned(v, 16), "attn: v must be 16-byte aligned");
  } else {
    DSA_REQUIRE(d_v <= d_qk, "attn: aliased V needs d_v <= d_qk");
  }
  return DSA_OK;
}

// Fused select (indexer -> top-k without a score matrix in the common case).  Workspace of
// one chunk of `rows` queries, each part 256-byte aligned:
//   sample  [rows, ld_s] fp32   scores of every 16th pool (threshold estimate)
//   cand    [rows, cap]  u64    candidate lists (order key << 32 | pool)
//   t_est, cnt, fail [rows] u32/u32/i32; any_fail (one i32)
//   scores  [rows, ld]   fp32   full scores, written only for the exact fallback
constexpr int kSampleShift = 4;
// The chunked driver takes the fused select for chunks whose first row sees at least this
// many pools; on shorter rows the score-row select is as fast (measured on MI355X: the
// candidate top-k's fixed per-row work then outweighs the score traffic it saves).
constexpr int64_t kFusedMinVisible = 49152;
// ... and only with more indexer heads than this: with at most 16 heads the score pass keeps
// its key rows across tile groups (which the candidate pass does not), and the score-row
// select is the faster one (1M tokens at 8 heads: 706 against 747 ms per forward step).
constexpr int kFusedMinHeads = 17;

struct FusedLayout {
  size_t sample, cand, t_est, cnt, fail, any, scores, total;
  int64_t ld_s, ld;
};

FusedLayout fused_layout(int64_t rows, int64_t n_pools) {
  FusedLayout L{};
  const int64_t cols = (n_pools + (int64_t{1} << kSampleShift) - 1) >> kSampleShift;
  L.ld_s = score_ld(cols);
  L.ld = score_ld(n_pools);
  const size_t r = static_cast<size_t>(rows);
  size_t off = 0;
  L.sample = off;
  off += align256(r * L.ld_s * sizeof(float));
  L.cand = off;
  off += align256(r * dsa::topk_cand_cap() * sizeof(uint64_t));
  L.t_est = off;
  off += align256(r * sizeof(uint32_t));
  L.cnt = off;
  off += align256(r * sizeof(uint32_t));
  L.fail = off;
  off += align256(r * sizeof(int32_t));
  L.any = off;
  off += 256;
  L.scores = off;
  off += align256(r * L.ld * sizeof(float));
  L.total = off;
  return L;
}

// Indexer scores and top-k of rows [q_start, q_start + nq) through the fused select: sampled
// scores -> per-row threshold -> indexer emitting candidates -> top-k over the candidates;
// rows whose candidate list cannot give the exact answer are redone by the plain indexer and
// score-row top-k, both gated on device flags (no host synchronisation).  ws holds
// fused_layout(nq, n_pools).total bytes, 256-byte aligned.
hipError_t run_fused_select(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            int32_t h_i, int32_t d_i, int32_t dtype, int64_t q_start,
                            int64_t nq, int64_t n_pools, int32_t k, int32_t* idx, char* ws,
                            hipStream_t s) {
  const FusedLayout L = fused_layout(nq, n_pools);
  float* sample = reinterpret_cast<float*>(ws + L.sample);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + L.cand);
  uint32_t* t_est = reinterpret_cast<uint32_t*>(ws + L.t_est);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
  int32_t* redo = reinterpret_cast<int32_t*>(ws + L.fail);
  int32_t* any = reinterpret_cast<int32_t*>(ws + L.any);
  float* scores = reinterpret_cast<float*>(ws + L.scores);

  dsa::IndexerOpts sopt;
  sopt.pool_shift = kSampleShift;
  hipError_t e = dsa::launch_index_scores(q_idx, q_row_stride, k_idx, k_row_stride, w,
                                          w_row_stride, sample, L.ld_s, q_start, nq, n_pools,
                                          h_i, d_i, dtype, 0, s, sopt);
  if (e != hipSuccess) return e;
  e = dsa::launch_topk_threshold(sample, L.ld_s, q_start, nq, n_pools, kSampleShift, k, t_est,
                                 cnt, any, s);
  if (e != hipSuccess) return e;
  dsa::IndexerOpts copt;
  copt.t_est = t_est;
  copt.cand_cnt = cnt;
  copt.cand = cand;
  copt.cand_cap = dsa::topk_cand_cap();
  e = dsa::launch_index_scores(q_idx, q_row_stride, k_idx, k_row_stride, w, w_row_stride,
                               nullptr, 0, q_start, nq, n_pools, h_i, d_i, dtype, 0, s, copt);
  if (e != hipSuccess) return e;
  dsa::TopkCand cs;
  cs.cand = cand;
  cs.cap = dsa::topk_cand_cap();
  cs.cnt = cnt;
  cs.t_est = t_est;
  cs.fail = redo;
  cs.any_fail = any;
  e = dsa::launch_topk_from_cand(cs, q_start, nq, n_pools, k, idx, s);
  if (e != hipSuccess) return e;
  dsa::IndexerOpts gopt;
  gopt.gate = any;
  gopt.gate_rows = redo;
  e = dsa::launch_index_scores(q_idx, q_row_stride, k_idx, k_row_stride, w, w_row_stride,
                               scores, L.ld, q_start, nq, n_pools, h_i, d_i, dtype, 0, s, gopt);
  if (e != hipSuccess) return e;
  return dsa::launch_topk(scores, L.ld, q_start, nq, n_pools, k, idx, nullptr, 0, s, redo);
}

dsa_status check_out_dtype(int32_t o_dtype) {
  DSA_REQUIRE(o_dtype == DSA_DTYPE_F32 || o_dtype == DSA_DTYPE_BF16,
              "attn: o_dtype must be DSA_DTYPE_F32 or DSA_DTYPE_BF16");
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_last_error; }

int dsa_abi_version(void) { return 2; }

dsa_status dsa_index_scores(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            float* scores, int64_t ld_scores, int64_t q_start, int64_t nq,
                            int64_t n_pools, int32_t h_i, int32_t d_i, int32_t dtype,
                            int32_t accumulate, void* stream) {
  if (dsa_status st = check_index_args(q_idx, q_row_stride, k_idx, k_row_stride, w,
                                       w_row_stride, n_pools, h_i, d_i, dtype))
    return st;
  if (dsa_status st = check_scores(scores, ld_scores, n_pools)) return st;
  DSA_REQUIRE(q_start >= 0 && nq >= 0, "index: q_start and nq must be >= 0");
  DSA_REQUIRE(accumulate == 0 || accumulate == 1, "index: accumulate must be 0 or 1");
  return hip_status(
      dsa::launch_index_scores(q_idx, q_row_stride, k_idx, k_row_stride, w, w_row_stride,
                               scores, ld_scores, q_start, nq, n_pools, h_i, d_i, dtype,
                               accumulate, static_cast<hipStream_t>(stream)),
      "dsa_index_scores launch");
}

size_t dsa_topk_workspace_bytes(int64_t nq, int64_t n_pools, int32_t k) {
  return dsa::topk_workspace_bytes(nq, n_pools, k);
}

dsa_status dsa_topk(const float* scores, int64_t ld_scores, int64_t q_start, int64_t nq,
                    int64_t n_pools, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                    void* stream) {
  if (dsa_status st = check_scores(scores, ld_scores, n_pools)) return st;
  if (dsa_status st = check_topk_args(n_pools, k, idx)) return st;
  DSA_REQUIRE(q_start >= 0 && nq >= 0, "topk: q_start and nq must be >= 0");
  const size_t need = dsa::topk_workspace_bytes(nq, n_pools, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "topk: workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : size_t{0});
  return hip_status(dsa::launch_topk(scores, ld_scores, q_start, nq, n_pools, k, idx, ws,
                                     ws_bytes, static_cast<hipStream_t>(stream)),
                    "dsa_topk launch");
}

dsa_status dsa_sparse_attn_fwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                               int64_t ld_v, const int32_t* idx, int32_t k, void* o,
                               int32_t o_dtype, float* lse, int64_t nq, int64_t n_pools,
                               int32_t h, int32_t d_qk, int32_t d_v, float scale,
                               void* stream) {
  if (dsa_status st = check_attn_args(q, kv, ld_kv, v, ld_v, idx, k, n_pools, h, d_qk, d_v,
                                      scale))
    return st;
  if (dsa_status st = check_out_dtype(o_dtype)) return st;
  DSA_REQUIRE(o && lse && aligned(o, 16) && aligned(lse, 4), "attn: null or misaligned o/lse");
  DSA_REQUIRE(nq >= 0, "attn: nq must be >= 0");
  return hip_status(dsa::launch_sparse_attn_fwd(q, kv, ld_kv, v, ld_v, idx, k, o,
                                                o_dtype == DSA_DTYPE_F32, lse, nq, n_pools, h,
                                                d_qk, d_v, scale,
                                                static_cast<hipStream_t>(stream)),
                    "dsa_sparse_attn_fwd launch");
}

size_t dsa_sparse_attn_bwd_workspace_bytes(int64_t nq, int32_t h) {
  return dsa::attn_bwd_workspace_bytes(nq, h);
}

dsa_status dsa_sparse_attn_bwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                               int64_t ld_v, const int32_t* idx, int32_t k, const void* o,
                               int32_t o_dtype, const float* lse, const void* d_o, float* dq,
                               float* dkv, float* dv, int64_t nq, int64_t n_pools, int32_t h,
                               int32_t d_qk, int32_t d_v, float scale, void* ws,
                               size_t ws_bytes, void* stream) {
  if (dsa_status st = check_attn_args(q, kv, ld_kv, v, ld_v, idx, k, n_pools, h, d_qk, d_v,
                                      scale))
    return st;
  if (dsa_status st = check_out_dtype(o_dtype)) return st;
  DSA_REQUIRE(o && lse && d_o && dq && dkv, "attn_bwd: null o, lse, d_o, dq or dkv");
  DSA_REQUIRE(aligned(o, 16) && aligned(d_o, 16) && aligned(dq, 16) && aligned(dkv, 16) &&
                  aligned(lse, 4),
              "attn_bwd: o, d_o, dq, dkv must be 16-byte aligned");
  DSA_REQUIRE(!v || dv, "attn_bwd: dv is required when a separate v is given");
  DSA_REQUIRE(!dv || aligned(dv, 16), "attn_bwd: dv must be 16-byte aligned");
  DSA_REQUIRE(nq >= 0, "attn_bwd: nq must be >= 0");
  const size_t need = dsa::attn_bwd_workspace_bytes(nq, h);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "attn_bwd: workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : size_t{0});
  return hip_status(dsa::launch_sparse_attn_bwd(q, kv, ld_kv, v, ld_v, idx, k, o,
                                                o_dtype == DSA_DTYPE_F32, lse, d_o, dq,
                                                dkv, dv, nq, n_pools, h, d_qk, d_v, scale, ws,
                                                static_cast<hipStream_t>(stream)),
                    "dsa_sparse_attn_bwd launch");
}

dsa_status dsa_sparse_attn_bwd_noalloc(const void* q, const void* kv, int64_t ld_kv,
                                       const void* v, int64_t ld_v, const int32_t* idx,
                                       int32_t k, const void* o, int32_t o_dtype,
                                       const float* lse, const void* d_o, float* dq, float* dkv,
                                       float* dv, int64_t nq, int64_t n_pools, int32_t h,
                                       int32_t d_qk, int32_t d_v, float scale, void* stream) {
  if (dsa_status st = check_attn_args(q, kv, ld_kv, v, ld_v, idx, k, n_pools, h, d_qk, d_v,
                                      scale))
    return st;
  if (dsa_status st = check_out_dtype(o_dtype)) return st;
  DSA_REQUIRE(o && lse && d_o && dq && dkv, "attn_bwd_noalloc: null o, lse, d_o, dq or dkv");
  DSA_REQUIRE(aligned(o, 16) && aligned(d_o, 16) && aligned(dq, 16) && aligned(dkv, 16) &&
                  aligned(lse, 4),
              "attn_bwd_noalloc: o, d_o, dq, dkv must be 16-byte aligned");
  DSA_REQUIRE(!v || dv, "attn_bwd_noalloc: dv is required when a separate v is given");
  DSA_REQUIRE(!dv || aligned(dv, 16), "attn_bwd_noalloc: dv must be 16-byte aligned");
  DSA_REQUIRE(nq >= 0, "attn_bwd_noalloc: nq must be >= 0");
  const int64_t cap = dsa::attn_bwd_scratch_floats();
  if (nq > cap / h)
    return fail(DSA_ERR_UNSUPPORTED,
                "attn_bwd_noalloc: nq * h = %lld * %d exceeds the static scratch of %lld "
                "per-row deltas (use dsa_sparse_attn_bwd with a workspace)",
                static_cast<long long>(nq), h, static_cast<long long>(cap));
  if (nq == 0) return ok();
  float* scratch = nullptr;
  if (dsa_status st = hip_status(dsa::attn_bwd_scratch(&scratch),
                                 "attn_bwd_noalloc: static scratch lookup"))
    return st;
  return hip_status(dsa::launch_sparse_attn_bwd(q, kv, ld_kv, v, ld_v, idx, k, o,
                                                o_dtype == DSA_DTYPE_F32, lse, d_o, dq, dkv, dv,
                                                nq, n_pools, h, d_qk, d_v, scale, scratch,
                                                static_cast<hipStream_t>(stream)),
                    "dsa_sparse_attn_bwd_noalloc launch");
}

size_t dsa_sparse_attn_bwd_deterministic_workspace_bytes(int64_t nq, int32_t h,
                                                         int64_t n_pools, int32_t k,
                                                         int32_t d_qk, int32_t d_v,
                                                         int32_t separate_dv) {
  if (nq <= 0 || h <= 0 || k <= 0 || d_qk <= 0 || d_v <= 0) return 0;
  return align256(dsa::attn_bwd_workspace_bytes(nq, h)) +
         dsa::attn_bwd_det_bytes(nq, n_pools, k, d_qk, d_v, separate_dv != 0);
}

dsa_status dsa_sparse_attn_bwd_deterministic(
    const void* q, const void* kv, int64_t ld_kv, const void* v, int64_t ld_v,
    const int32_t* idx, int32_t k, const void* o, int32_t o_dtype, const float* lse,
    const void* d_o, float* dq, float* dkv, float* dv, int64_t nq, int64_t n_pools, int32_t h,
    int32_t d_qk, int32_t d_v, float scale, void* ws, size_t ws_bytes, void* stream) {
  if (dsa_status st = check_attn_args(q, kv, ld_kv, v, ld_v, idx, k, n_pools, h, d_qk, d_v,
                                      scale))
    return st;
  if (dsa_status st = check_out_dtype(o_dtype)) return st;
  DSA_REQUIRE(o && lse && d_o && dq && dkv, "attn_bwd_det: null o, lse, d_o, dq or dkv");
  DSA_REQUIRE(aligned(o, 16) && aligned(d_o, 16) && aligned(dq, 16) && aligned(dkv, 16) &&
                  aligned(lse, 4),
              "attn_bwd_det: o, d_o, dq, dkv must be 16-byte aligned");
  DSA_REQUIRE(!v || dv, "attn_bwd_det: dv is required when a separate v is given");
  DSA_REQUIRE(!dv || aligned(dv, 16), "attn_bwd_det: dv must be 16-byte aligned");
  DSA_REQUIRE(nq >= 0, "attn_bwd_det: nq must be >= 0");
  if (nq == 0) return ok();
  const size_t need = dsa_sparse_attn_bwd_deterministic_workspace_bytes(nq, h, n_pools, k, d_qk,
                                                                        d_v, dv != nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE,
                "attn_bwd_det: 256-byte aligned workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : size_t{0});
  char* base = static_cast<char*>(ws);
  void* det = base + align256(dsa::attn_bwd_workspace_bytes(nq, h));
  return hip_status(dsa::launch_sparse_attn_bwd(q, kv, ld_kv, v, ld_v, idx, k, o,
                                                o_dtype == DSA_DTYPE_F32, lse, d_o, dq, dkv,
                                                dv, nq, n_pools, h, d_qk, d_v, scale, ws,
                                                static_cast<hipStream_t>(stream), det),
                    "dsa_sparse_attn_bwd_deterministic launch");
}

dsa_status dsa_pool_keys(const void* x, int64_t ld_x, const float* gate, int64_t n_tokens,
                         int32_t d, void* out, int64_t ld_out, void* stream) {
  DSA_REQUIRE(n_tokens >= 0, "pool_keys: n_tokens must be >= 0");
  DSA_REQUIRE((x && gate && out) || n_tokens < 4, "pool_keys: null x, gate or out");
  DSA_REQUIRE(d >= 1, "pool_keys: d must be >= 1");
  if (d % 8 != 0) return fail(DSA_ERR_UNSUPPORTED, "pool_keys: d = %d is not a multiple of 8", d);
  DSA_REQUIRE(ld_x >= d && ld_out >= d && ld_x % 8 == 0 && ld_out % 8 == 0,
              "pool_keys: ld_x and ld_out must be >= d and multiples of 8");
  DSA_REQUIRE(aligned(x, 16) && aligned(out, 16) && aligned(gate, 4),
              "pool_keys: x and out must be 16-byte aligned, gate 4-byte aligned");
  return hip_status(dsa::launch_pool_keys(x, ld_x, gate, n_tokens, d, out, ld_out,
                                          static_cast<hipStream_t>(stream)),
                    "dsa_pool_keys launch");
}

size_t dsa_index_topk_workspace_bytes(int64_t nq, int64_t n_pools, int32_t k) {
  if (nq <= 0 || k <= 0 || n_pools < 0) return 0;
  return fused_layout(nq, n_pools).total;
}

dsa_status dsa_index_topk(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                          int64_t k_row_stride, const float* w, int64_t w_row_stride,
                          int64_t q_start, int64_t nq, int64_t n_pools, int32_t h_i,
                          int32_t d_i, int32_t dtype, int32_t k, int32_t* idx, void* ws,
                          size_t ws_bytes, void* stream) {
  if (dsa_status st = check_index_args(q_idx, q_row_stride, k_idx, k_row_stride, w,
                                       w_row_stride, n_pools, h_i, d_i, dtype))
    return st;
  if (dsa_status st = check_topk_args(n_pools, k, idx)) return st;
  DSA_REQUIRE(q_start >= 0 && nq >= 0, "index_topk: q_start and nq must be >= 0");
  if (!dsa::topk_fused_supported(k))
    return fail(DSA_ERR_UNSUPPORTED, "index_topk: k = %d > %d for the fused select", k,
                2 * dsa::topk_cand_cap() / 3);
  if (nq == 0) return ok();
  const size_t need = dsa_index_topk_workspace_bytes(nq, n_pools, k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE,
                "index_topk: 256-byte aligned workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : size_t{0});
  return hip_status(run_fused_select(q_idx, q_row_stride, k_idx, k_row_stride, w,
                                     w_row_stride, h_i, d_i, dtype, q_start, nq, n_pools, k,
                                     idx, static_cast<char*>(ws),
                                     static_cast<hipStream_t>(stream)),
                    "dsa_index_topk launch");
}

size_t dsa_forward_chunked_workspace_bytes(int64_t n_pools, int64_t chunk, int32_t k) {
  if (chunk <= 0 || k <= 0 || n_pools < 0) return 0;
  const int64_t ld = score_ld(n_pools);
  const size_t idx_bytes = align256(static_cast<size_t>(chunk) * k * sizeof(int32_t));
  if (dsa::topk_fused_supported(k))
    return idx_bytes + fused_layout(chunk, n_pools).total +
           align256(dsa::topk_workspace_bytes(chunk, n_pools, k));
  return align256(static_cast<size_t>(chunk) * ld * sizeof(float)) + idx_bytes +
         align256(dsa::topk_workspace_bytes(chunk, n_pools, k));
}

dsa_status dsa_forward_chunked(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                               int64_t k_row_stride, const float* w, int64_t w_row_stride,
                               int32_t h_i, int32_t d_i, int32_t idx_dtype, const void* q,
                               const void* kv, int64_t ld_kv, const void* v, int64_t ld_v,
                               int32_t h, int32_t d_qk, int32_t d_v, float scale, int32_t k,
                               int64_t n_tokens, int64_t n_pools, int64_t chunk, void* o,
                               int32_t o_dtype, float* lse, int32_t* idx_out, void* ws,
                               size_t ws_bytes, void* stream) {
  if (dsa_status st = check_index_args(q_idx, q_row_stride, k_idx, k_row_stride, w,
                                       w_row_stride, n_pools, h_i, d_i, idx_dtype))
    return st;
  // When idx_out is NULL the indices live in the (aligned) workspace; check the rest with an
  // aligned stand-in pointer.
  static const int32_t kAlignedStandIn[4] = {0, 0, 0, 0};
  const int32_t* idx_probe = idx_out ? idx_out : kAlignedStandIn;
  if (dsa_status st = check_attn_args(q, kv, ld_kv, v, ld_v, idx_probe, k, n_pools, h, d_qk,
                                      d_v, scale))
    return st;
  if (dsa_status st = check_topk_args(n_pools, k, idx_probe)) return st;
  if (dsa_status st = check_out_dtype(o_dtype)) return st;
  DSA_REQUIRE(o && lse && aligned(o, 16) && aligned(lse, 4), "chunked: null or misaligned o/lse");
  DSA_REQUIRE(n_tokens >= 0 && chunk >= 1, "chunked: n_tokens must be >= 0 and chunk >= 1");
  const size_t need = dsa_forward_chunked_workspace_bytes(n_pools, chunk, k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE, "chunked: 256-byte aligned workspace of %zu bytes needed, %zu given",
                need, ws ? ws_bytes : size_t{0});

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ld = score_ld(n_pools);
  const bool fused = dsa::topk_fused_supported(k);
  char* base = static_cast<char*>(ws);
  // Layout: idx chunk, then either the fused select's workspace (one chunk) or the score
  // chunk and the top-k workspace.
  int32_t* idx_ws = reinterpret_cast<int32_t*>(base);
  char* rest = base + align256(static_cast<size_t>(chunk) * k * sizeof(int32_t));
  // The score-row path uses the fused layout's score buffer when the fused select exists.
  float* scores = reinterpret_cast<float*>(rest + (fused ? fused_layout(chunk, n_pools).scores : 0));
  char* topk_ws = reinterpret_cast<char*>(scores) +
                  align256(static_cast<size_t>(chunk) * ld * sizeof(float));
  const size_t topk_bytes = dsa::topk_workspace_bytes(chunk, n_pools, k);
  const int64_t ielt = idx_dtype == DSA_DTYPE_BF16 ? 2 : 1;

  for (int64_t t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int64_t nq = (n_tokens - t0) < chunk ? (n_tokens - t0) : chunk;
    const void* q_idx_c = static_cast<const char*>(q_idx) + t0 * q_row_stride * ielt;
    int32_t* idx_chunk = idx_out ? idx_out + t0 * k : idx_ws;
    hipError_t e;
    if (fused && h_i >= kFusedMinHeads &&
        std::min<int64_t>(n_pools, (t0 + 1) / 4) >= kFusedMinVisible) {
      e = run_fused_select(q_idx_c, q_row_stride, k_idx, k_row_stride, w + t0 * w_row_stride,
                           w_row_stride, h_i, d_i, idx_dtype, t0, nq, n_pools, k, idx_chunk,
                           rest, s);
      if (e != hipSuccess) return hip_status(e, "dsa_forward_chunked: select launch");
    } else {
      e = dsa::launch_index_scores(q_idx_c, q_row_stride, k_idx, k_row_stride,
                                   w + t0 * w_row_stride, w_row_stride, scores, ld, t0, nq,
                                   n_pools, h_i, d_i, idx_dtype, 0, s);
      if (e != hipSuccess) return hip_status(e, "dsa_forward_chunked: indexer launch");
      e = dsa::launch_topk(scores, ld, t0, nq, n_pools, k, idx_chunk, topk_ws, topk_bytes, s);
      if (e != hipSuccess) return hip_status(e, "dsa_forward_chunked: top-k launch");
    }
    const size_t o_elt = o_dtype == DSA_DTYPE_F32 ? 4 : 2;
    e = dsa::launch_sparse_attn_fwd(static_cast<const uint16_t*>(q) + t0 * h * d_qk, kv, ld_kv,
                                    v, ld_v, idx_chunk, k,
                                    static_cast<char*>(o) + t0 * h * d_v * o_elt,
                                    o_dtype == DSA_DTYPE_F32, lse + t0 * h, nq, n_pools, h,
                                    d_qk, d_v, scale, s);
    if (e != hipSuccess) return hip_status(e, "dsa_forward_chunked: attention launch");
  }
  return ok();
}

}  // extern "C"
