// Internal launchers of the libdsa kernels (called by the C ABI layer after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Optional behaviour of the indexer launch.  pool_shift s: score only every 2^s-th pool
// (column c of the output is pool c * 2^s).  gate: when non-null, the launch does nothing
// unless *gate != 0 (read on the device); gate_rows (non-null): only query tiles that hold
// a row r with gate_rows[r] != 0 are computed.  cand (non-null): instead of writing scores,
// append (order key << 32 | pool) of every visible entry whose order key is >= t_est[row] to
// cand[row * cand_cap + slot], slots taken from cand_cnt[row] (the caller zeroes it; a count
// past cand_cap means entries were dropped).
struct IndexerOpts {
  int pool_shift = 0;
  const int32_t* gate = nullptr;
  const int32_t* gate_rows = nullptr;
  const uint32_t* t_est = nullptr;
  uint32_t* cand_cnt = nullptr;
  uint64_t* cand = nullptr;
  int cand_cap = 0;
};

bool indexer_supported(int d_i, int dtype);
int indexer_max_heads();
hipError_t launch_index_scores(const void* q, int64_t q_row_stride, const void* k,
                               int64_t k_row_stride, const float* w, int64_t w_row_stride,
                               float* scores, int64_t ld, int64_t q_start, int64_t nq,
                               int64_t n_pools, int h_i, int d_i, int dtype, int accumulate,
                               hipStream_t stream, const IndexerOpts& opt = IndexerOpts());

int topk_max_k();
size_t topk_workspace_bytes(int64_t nq, int64_t n_pools, int k);
// gate (non-null): rows r with gate[r] == 0 are skipped (their idx rows are left as they are).
hipError_t launch_topk(const float* scores, int64_t ld, int64_t q_start, int64_t nq,
                       int64_t n_pools, int k, int32_t* idx, void* ws, size_t ws_bytes,
                       hipStream_t stream, const int32_t* gate = nullptr);

// Fused select (indexer candidates -> top-k).  Candidate lists: cand[row * cap + slot] =
// (order key << 32) | pool, cnt[row] entries written by the indexer (more than cap means
// some were dropped).  fail[row] is set to 1 (and *any_fail to 1) for rows whose list cannot
// give the exact result; 0 otherwise.
struct TopkCand {
  const uint64_t* cand = nullptr;
  int cap = 0;
  const uint32_t* cnt = nullptr;
  const uint32_t* t_est = nullptr;
  int32_t* fail = nullptr;
  int32_t* any_fail = nullptr;
};
int topk_cand_cap();
bool topk_fused_supported(int k);
hipError_t launch_topk_threshold(const float* sample, int64_t ld_sample, int64_t q_start,
                                 int64_t nq, int64_t n_pools, int shift, int k, uint32_t* t_est,
                                 uint32_t* cnt, int32_t* any_fail, hipStream_t stream);
hipError_t launch_topk_from_cand(const TopkCand& cs, int64_t q_start, int64_t nq,
                                 int64_t n_pools, int k, int32_t* idx, hipStream_t stream);

bool attn_shape_supported(int d_qk, int d_v);
int attn_max_k();
hipError_t launch_sparse_attn_fwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                                  int64_t ld_v, const int32_t* idx, int k, void* o, int o_f32,
                                  float* lse, int64_t nq, int64_t n_pools, int h, int d_qk,
                                  int d_v, float scale, hipStream_t stream);

size_t attn_bwd_workspace_bytes(int64_t nq, int h);
// The allocation-free backward keeps its per-row deltas in a static device array of this
// many floats; attn_bwd_scratch gives that array's address on the current device (looked
// up once per device, thread-safe).
int64_t attn_bwd_scratch_floats();
hipError_t attn_bwd_scratch(float** out);
// Bytes of the deterministic backward's own workspace (staging rows of one query chunk and
// the per-pool reduction's sort buffers), beside the per-row deltas.
size_t attn_bwd_det_bytes(int64_t nq, int64_t n_pools, int k, int d_qk, int d_v,
                          bool separate_dv);
// det_ws (non-null, 256-byte aligned, attn_bwd_det_bytes(...) bytes): deterministic dK/dV
// (staged rows reduced per pool in a fixed order); null: fp32 atomics.
hipError_t launch_sparse_attn_bwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                                  int64_t ld_v, const int32_t* idx, int k, const void* o,
                                  int o_f32, const float* lse, const void* d_o, float* dq, float* dkv,
                                  float* dv, int64_t nq, int64_t n_pools, int h, int d_qk,
                                  int d_v, float scale, void* ws, hipStream_t stream,
                                  void* det_ws = nullptr);

// Deterministic per-pool sums of staged rows (bwd_reduce.hip).  idx [rows, k] is the
// selection of the staged chunk; stage_k [rows * k, w_k] (and stage_v [rows * k, w_v], or
// null) hold one row per (row, slot).  out_k[s] (and out_v[s]) += the rows of the pairs that
// selected pool s, added in row-major (row, slot) order.  ws: pool_reduce_workspace_bytes.
size_t pool_reduce_workspace_bytes(int64_t n_entries, int64_t n_pools);
hipError_t launch_pool_reduce(const int32_t* idx, int64_t rows, int k, int64_t n_pools,
                              const float* stage_k, int w_k, float* out_k,
                              const float* stage_v, int w_v, float* out_v, void* ws,
                              hipStream_t s);

// Pooled keys (pool.hip): out[s, :d] = the gate-softmax-weighted average of rows 4s .. 4s+3
// of x, for s < n_tokens / 4, in bf16.  d a multiple of 8; x, out 16-byte aligned with row
// strides (elements) multiples of 8.
hipError_t launch_pool_keys(const void* x, int64_t ld_x, const float* gate, int64_t n_tokens,
                            int d, void* out, int64_t ld_out, hipStream_t stream);

}  // namespace dsa
