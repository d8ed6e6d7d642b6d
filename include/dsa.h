/*
 * dsa.h - C ABI of libdsa, an MI355X (gfx950) implementation of the DeepSeek Sparse
 * Attention (DSA) layer's hot path: indexer scores, per-query top-k selection, sparse MQA
 * attention forward and backward, and a query-chunked forward driver.
 *
 * What the layer is (page "SkyRL extends GLM-5.3-Flash training context to 1 million
 * tokens"):
 *   - section "Model and bottleneck": an indexer scores every pooled key entry, one pool per
 *     4 tokens, for every query; attention then reads only about 2048 selected entries per
 *     query, so the quadratic cost sits in the indexer;
 *   - section "Four optimizations", item 1 (DSA truly sparse): the indexer is computed in
 *     query chunks so the score matrix never exists beyond one chunk; the selected pool
 *     indices are int32; the sparse kernel runs on DeepSeek-V3.2-shaped tensors; a kernel
 *     that does not support a shape must not silently fall back to dense attention.
 * The pages print no formula; the definitions used here are stated on each call.
 *
 * Conventions for every call:
 *   - All tensor pointers are device memory owned by the caller.  The library allocates
 *     nothing, keeps no global state besides a thread-local error string, never
 *     synchronises, and enqueues its kernels on `stream` (a hipStream_t passed as void*;
 *     NULL is the null stream).  Calls are asynchronous.
 *   - Arguments are validated before anything is launched.  On an error nothing is
 *     launched, a status is returned and dsa_last_error() describes it.
 *   - Visibility: pool s is visible to query position t iff 4s + 3 <= t, i.e. query t sees
 *     the prefix [0, V(t)) with V(t) = min(n_pools, floor((t + 1) / 4)).
 *   - bf16 tensors are passed as pointers to 16-bit bfloat16 values, fp8 tensors as
 *     pointers to bytes in the OCP FP8 E4M3 ("e4m3fn") encoding.
 *   - Vector alignment: bf16/fp8 tensor base pointers must be 16-byte aligned and their row
 *     strides (in elements) a multiple of 16 bytes' worth of elements; fp32 score matrices
 *     must be 16-byte aligned with ld_scores a multiple of 4.  Violations return
 *     DSA_ERR_INVALID_ARGUMENT.
 *   - Sizes a kernel is not built for return DSA_ERR_UNSUPPORTED (never a fallback).
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad stride or alignment */
  DSA_ERR_UNSUPPORTED = 2,      /* a size or dtype no kernel is built for */
  DSA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  DSA_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} dsa_status;

typedef enum dsa_dtype {
  DSA_DTYPE_BF16 = 0,
  DSA_DTYPE_FP8_E4M3 = 1,
  DSA_DTYPE_F32 = 2
} dsa_dtype;

/* Human-readable name of a status code (static string). */
const char* dsa_status_string(dsa_status status);

/* Description of the last error returned on the calling thread ("" if none). */
const char* dsa_last_error(void);

/* ABI version of this header (bumped on incompatible changes). */
int dsa_abi_version(void);

/*
 * dsa_index_scores - lightning-indexer scores of a chunk of queries against all pools.
 * Source: page "SkyRL ... 1 million tokens", section "Model and bottleneck" (every query
 * scores every visible pooled key) and section "Four optimizations", item 1 (computed per
 * query chunk; the indexer is sharded over tensor-parallel ranks, whose partial sums the
 * `accumulate` mode adds up).  Formula (the lightning indexer as published with
 * DeepSeek-V3.2; the pages give none):
 *     I[t, s] = sum_{j < h_i} w[t, j] * max(0, sum_{d < d_i} q[t, j, d] * k[s, d])
 * with one pooled key row k[s, :] shared by all indexer heads.
 *
 *   q_idx         [nq, h_i, d_i] (bf16 or fp8 per `dtype`); token r's row starts at
 *                 q_idx + r * q_row_stride elements (q_row_stride >= h_i * d_i); heads are
 *                 contiguous rows of d_i.  Row r is query position t = q_start + r.
 *   k_idx         [n_pools, d_i], row stride k_row_stride elements (>= d_i).
 *   w             fp32 head weights; token r's weights start at w + r * w_row_stride
 *                 (w_row_stride 0: one vector of h_i weights for all tokens).
 *   scores        [nq, ld_scores] fp32 output (ld_scores >= n_pools).  For each row only
 *                 the visible prefix [0, V(t)) is written; entries beyond it are untouched.
 *   accumulate    0: scores = I;  1: scores += I (sums partial scores of head shares).
 *   Supported: bf16 with d_i in {32, 64, 128, 256}; fp8 with d_i in {128, 256};
 *   1 <= h_i <= 64.
 * Arithmetic: bf16 or fp8 MFMA products with fp32 accumulation; ReLU and the weighted head
 * sum in fp32 registers.  On integer-valued inputs whose sums stay below 2^24 the result
 * is exact and therefore independent of summation order.
 */
dsa_status dsa_index_scores(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            float* scores, int64_t ld_scores, int64_t q_start, int64_t nq,
                            int64_t n_pools, int32_t h_i, int32_t d_i, int32_t dtype,
                            int32_t accumulate, void* stream);

/*
 * dsa_topk - per-query top-k pool selection.
 * Source: page "SkyRL ... 1 million tokens", section "Model and bottleneck" (about 2048
 * keys kept per query) and section "Four optimizations", item 1 (selected pool indices are
 * int32).  Row r (query position t = q_start + r) ranks its visible scores
 * scores[r, 0 .. V(t)-1] by score descending, lower pool index first among equal scores
 * (+0 and -0 are equal), and writes the first min(k, V(t)) pool indices to idx[r, :], in
 * that order; the remaining k - min(k, V(t)) slots are set to -1.  Bit-exact.
 *   scores  [nq, ld_scores] fp32 (only the visible prefix of each row is read).
 *   idx     [nq, k] int32 output.
 *   ws      workspace of at least dsa_topk_workspace_bytes(nq, n_pools, k) bytes (may be
 *           NULL when that is 0).
 *   Supported: 1 <= k <= 4096.  NaN scores are outside the contract.
 */
dsa_status dsa_topk(const float* scores, int64_t ld_scores, int64_t q_start, int64_t nq,
                    int64_t n_pools, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                    void* stream);
size_t dsa_topk_workspace_bytes(int64_t nq, int64_t n_pools, int32_t k);

/*
 * dsa_index_topk - dsa_index_scores followed by dsa_topk for rows [q_start, q_start + nq),
 * with the same result (idx bit-identical to the two calls), usually without writing the
 * score matrix.  Source: page "SkyRL ... 1 million tokens", section "Four optimizations",
 * item 1 (indexer computed per query chunk, only int32 indices leave it); carrying the
 * chunking down into the indexer's own tiles is this library's extension.
 * Steps: scores of every 16th visible pool give each row a threshold about 1.5 k keys deep
 * (rows with at most 4096 visible pools take every visible pool); the indexer then keeps,
 * per row, only the (score, pool) pairs at or above the threshold; the top-k is resolved
 * over those.  A row whose list does not hold between k and 4096 pairs (heavy ties at the
 * threshold, adversarial score layouts) is redone exactly: the plain indexer writes the
 * chunk's scores into the workspace and dsa_topk's select runs on that row.  Both redo
 * launches are always enqueued and do nothing on the device when no row needs them.
 *   Operands as dsa_index_scores (accumulate = 0) and dsa_topk.
 *   ws: at least dsa_index_topk_workspace_bytes(nq, n_pools, k) bytes, 256-byte aligned
 *   (candidate lists of 32 KB per row plus a full score buffer for the redo).
 *   Supported: as dsa_index_scores; 1 <= k <= 2730 (DSA_ERR_UNSUPPORTED above: use the two
 *   calls).
 */
dsa_status dsa_index_topk(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                          int64_t k_row_stride, const float* w, int64_t w_row_stride,
                          int64_t q_start, int64_t nq, int64_t n_pools, int32_t h_i,
                          int32_t d_i, int32_t dtype, int32_t k, int32_t* idx, void* ws,
                          size_t ws_bytes, void* stream);
size_t dsa_index_topk_workspace_bytes(int64_t nq, int64_t n_pools, int32_t k);

/*
 * dsa_sparse_attn_fwd - sparse MQA attention over the selected pooled KV rows.
 * Source: page "SkyRL ... 1 million tokens", section "Model and bottleneck" (attention
 * reads only the selected entries) and section "Four optimizations", item 1 (DeepSeek-V3.2
 * shaped tensors: a 576-wide latent KV row shared by all query heads, whose first 512
 * columns are the value).  For query row r, head h and the valid slots j of idx[r, :]
 * (idx != -1):
 *     logit_j = scale * q[r, h, :] . K[idx[r, j], :]
 *     O[r, h, :] = sum_j softmax(logit)_j * V[idx[r, j], :],  LSE[r, h] = ln sum_j exp(logit_j)
 * K is kv[:, 0:d_qk].  V is v[:, 0:d_v] when v is given, else kv[:, 0:d_v] (aliased latent
 * row).  A row without valid slots gives O = 0 and LSE = -inf.
 *   q    [nq, h, d_qk] bf16, dense.
 *   kv   [n_pools, ld_kv] bf16 (ld_kv >= d_qk);  v [n_pools, ld_v] bf16 or NULL.
 *   idx  [nq, k] int32 in [-1, n_pools); -1 slots may sit anywhere.
 *   o    [nq, h, d_v] output, fp32 (o_dtype DSA_DTYPE_F32) or bf16 (DSA_DTYPE_BF16, the
 *        fp32 result rounded to nearest even once);  lse [nq, h] fp32 (natural log).
 *   Supported: (d_qk, d_v) in {(128, 128), (576, 512), (512, 512), (256, 256)} (the last two
 *   are the latent row without its rotary columns, NoPE, full and half width),
 *   1 <= h <= 64, 1 <= k <= 4096 (any k, e.g. 2051).
 *   Slots holding a value outside [-1, n_pools) are skipped like -1 (never dereferenced).
 * Arithmetic: bf16 MFMA for q.K with fp32 accumulation, fp32 softmax; on rows with fewer
 * than 512 valid slots each probability enters the P.V MFMA as a pair of bf16 values (its
 * rounding and the rounding of the remainder, about 16 significant bits), on longer rows as
 * one bf16 value (8 bits; a relative error of at most 2^-8 per probability, about 1e-3 of
 * the RMS of O on average); fp32 accumulation of O and of the row sums.
 */
dsa_status dsa_sparse_attn_fwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                               int64_t ld_v, const int32_t* idx, int32_t k, void* o,
                               int32_t o_dtype, float* lse, int64_t nq, int64_t n_pools,
                               int32_t h, int32_t d_qk, int32_t d_v, float scale,
                               void* stream);

/*
 * dsa_sparse_attn_bwd - gradients of dsa_sparse_attn_fwd.
 * The pages describe training but print no backward; this is the exact gradient of the
 * forward above.  With P_j = exp(logit_j - LSE), dP_j = dO . V_j, D = sum_j P_j dP_j
 * (computed as dO . O), dS_j = P_j (dP_j - D):
 *     dq[r, h, :]       = scale * sum_j dS_j K_j           (overwritten)
 *     dkv[idx_j, 0:d_qk] += scale * sum_{r,h} dS_j q[r, h, :]
 *     dv[idx_j, :]      += sum_{r,h} P_j dO[r, h, :]       (dv given), or, when dv is NULL,
 *     dkv[idx_j, 0:d_v] += the same                         (V aliased to kv[:, 0:d_v]).
 *   Inputs are those of the forward plus o (its output, fp32 or bf16 per o_dtype), lse
 *   (fp32, its output) and d_o [nq, h, d_v] bf16.  dq [nq, h, d_qk] fp32.  dkv [n_pools, d_qk] fp32 and
 *   dv [n_pools, d_v] fp32 are accumulated with fp32 atomics: the caller zeroes them (or
 *   keeps a running sum); the summation order, and so the last bits, vary run to run.
 *   dv must be non-NULL when v is non-NULL.
 *   ws: workspace of at least dsa_sparse_attn_bwd_workspace_bytes(nq, h) bytes.
 *   Supported: as the forward.
 */
dsa_status dsa_sparse_attn_bwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                               int64_t ld_v, const int32_t* idx, int32_t k, const void* o,
                               int32_t o_dtype, const float* lse, const void* d_o, float* dq,
                               float* dkv,
                               float* dv, int64_t nq, int64_t n_pools, int32_t h,
                               int32_t d_qk, int32_t d_v, float scale, void* ws,
                               size_t ws_bytes, void* stream);
size_t dsa_sparse_attn_bwd_workspace_bytes(int64_t nq, int32_t h);

/*
 * dsa_sparse_attn_bwd_noalloc - dsa_sparse_attn_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight training or
 * serving loops, harnesses that forbid allocation).  Same operands, results and arithmetic as
 * dsa_sparse_attn_bwd (same kernels); the per-row deltas D = dO . O that dsa_sparse_attn_bwd
 * keeps in its workspace go to a static device array of 2^22 floats (16 MiB) inside the
 * library instead.  Each GPU the library runs on holds one such array until the process
 * ends; the first call on a device looks up its address (hipGetSymbolAddress, no
 * allocation).  The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Every delta is written before it is read, so nothing needs clearing between
 * calls.
 *   Limit: nq * h <= 4194304 (e.g. 65536 query rows of 64 heads); a larger call returns
 *   DSA_ERR_UNSUPPORTED before anything is launched (split the rows over several calls, or
 *   use dsa_sparse_attn_bwd).
 *   All calls on one GPU share its array: calls that overlap in time on one GPU (on
 *   different streams, or from several threads) race on it and give wrong results.  Calls
 *   ordered on one stream are safe.
 *   Supported: as the forward.
 */
dsa_status dsa_sparse_attn_bwd_noalloc(const void* q, const void* kv, int64_t ld_kv,
                                       const void* v, int64_t ld_v, const int32_t* idx,
                                       int32_t k, const void* o, int32_t o_dtype,
                                       const float* lse, const void* d_o, float* dq, float* dkv,
                                       float* dv, int64_t nq, int64_t n_pools, int32_t h,
                                       int32_t d_qk, int32_t d_v, float scale, void* stream);

/*
 * dsa_sparse_attn_bwd_deterministic - dsa_sparse_attn_bwd with results that do not vary from
 * run to run (bit-identical dq, dkv, dv for the same inputs), without atomics.  The pages
 * train the layer but print no backward; reproducible gradients are this library's option.
 * dq is computed as in dsa_sparse_attn_bwd (it never used atomics).  For dK and dV the query
 * rows go in chunks of up to 4096: each (row, slot) pair's head-summed dK row (with dV added
 * into its first d_v columns when dv is NULL, or a separate dV row) is written to a staging
 * buffer; the chunk's selection is sorted by pool with a stable radix sort, so that the pairs
 * of every pool keep their row-major (row, slot) order; then each pool's staged rows are
 * added in that order, in fp32, and the sum is added to the pool's row of dkv (and dv).
 * Chunks are processed in row order.  Every sum therefore has a fixed order.
 *   Arguments as dsa_sparse_attn_bwd (dkv and dv are still accumulated: the caller zeroes
 *   them or keeps a running sum).  Any idx is accepted as for the forward (-1 or out-of-range
 *   slots are skipped, a pool repeated in a row contributes once per slot).
 *   ws: at least dsa_sparse_attn_bwd_deterministic_workspace_bytes(nq, h, n_pools, k, d_qk,
 *   d_v, separate_dv = (dv != NULL)) bytes, 256-byte aligned: the per-row deltas, the
 *   staging rows of one chunk (min(nq, 4096) * k * (d_qk [+ d_v]) fp32, 19.3 GB for 4096 rows
 *   of k = 2048 with 576-wide rows) and the sort buffers (about 20 bytes per pair plus 4 per
 *   pool).
 *   Supported: as the forward.
 */
dsa_status dsa_sparse_attn_bwd_deterministic(
    const void* q, const void* kv, int64_t ld_kv, const void* v, int64_t ld_v,
    const int32_t* idx, int32_t k, const void* o, int32_t o_dtype, const float* lse,
    const void* d_o, float* dq, float* dkv, float* dv, int64_t nq, int64_t n_pools, int32_t h,
    int32_t d_qk, int32_t d_v, float scale, void* ws, size_t ws_bytes, void* stream);
size_t dsa_sparse_attn_bwd_deterministic_workspace_bytes(int64_t nq, int32_t h,
                                                         int64_t n_pools, int32_t k,
                                                         int32_t d_qk, int32_t d_v,
                                                         int32_t separate_dv);

/*
 * dsa_pool_keys - pooled key rows, one per 4 tokens, from per-token rows and gate scores.
 * Source: page "SkyRL ... 1 million tokens", section "Model and bottleneck" (the indexer
 * scores "one pool per 4 tokens") and section "Four optimizations", item 3 (pools are formed
 * with "k-pool gate scores").  The pages print no formula; the reading implemented: pool s is
 * the average of the rows of tokens 4s .. 4s+3 weighted by the softmax of their gate scores,
 *     out[s, c] = sum_{i<4} softmax(gate[4s .. 4s+3])_i * x[4s+i, c],
 * for s < floor(n_tokens / 4) (a partial last pool is never visible to any query, since pool
 * s becomes visible at token 4s+3, so it is not formed).  The same call pools any bf16 key
 * table: the indexer keys (d = d_i) and the latent KV rows (d = 576).
 *   x     [n_tokens, ld_x] bf16 (columns [0, d) are pooled);  gate [n_tokens] fp32.
 *   out   [n_tokens / 4, ld_out] bf16 output (columns [0, d) written).
 *   Supported: d a multiple of 8; ld_x, ld_out multiples of 8 (>= d); x, out 16-byte aligned.
 *   With n_tokens < 4 no pool is formed, nothing is accessed and the pointers may be NULL.
 * Arithmetic: fp32 softmax and weighted sum, one rounding to bf16 (nearest, ties to even).
 */
dsa_status dsa_pool_keys(const void* x, int64_t ld_x, const float* gate, int64_t n_tokens,
                         int32_t d, void* out, int64_t ld_out, void* stream);

/*
 * dsa_forward_chunked - the whole DSA forward over n_tokens queries, one query chunk at a
 * time: for each chunk [t0, t0 + chunk) it runs the select (dsa_index_topk on chunks whose
 * first row sees at least 49152 pools when k <= 2730 and h_i > 16, else dsa_index_scores
 * into one reused fp32 score buffer in the workspace and dsa_topk; the indices are the same
 * either way), then dsa_sparse_attn_fwd.  Source: page
 * "SkyRL ... 1 million tokens", section "Four optimizations", item 1 (indexer scores
 * computed in chunks per query, so the quadratic score matrix never exists beyond one
 * chunk).  Results do not depend on `chunk`.
 *   Indexer operands as dsa_index_scores with q_start = 0 and nq = n_tokens
 *   (w_row_stride counts from token 0).  Attention operands as dsa_sparse_attn_fwd with
 *   nq = n_tokens.  topk: k.  idx_out [n_tokens, k] int32 or NULL (then the indices live
 *   only in the workspace, one chunk at a time).
 *   ws: at least dsa_forward_chunked_workspace_bytes(n_pools, chunk, k) bytes.
 */
dsa_status dsa_forward_chunked(const void* q_idx, int64_t q_row_stride, const void* k_idx,
                               int64_t k_row_stride, const float* w, int64_t w_row_stride,
                               int32_t h_i, int32_t d_i, int32_t idx_dtype, const void* q,
                               const void* kv, int64_t ld_kv, const void* v, int64_t ld_v,
                               int32_t h, int32_t d_qk, int32_t d_v, float scale, int32_t k,
                               int64_t n_tokens, int64_t n_pools, int64_t chunk, void* o,
                               int32_t o_dtype, float* lse, int32_t* idx_out, void* ws,
                               size_t ws_bytes, void* stream);
size_t dsa_forward_chunked_workspace_bytes(int64_t n_pools, int64_t chunk, int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
