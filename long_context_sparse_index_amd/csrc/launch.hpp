// Internal launchers of the libdsa kernels (called by the C ABI layer after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

bool indexer_supported(int d_i, int dtype);
int indexer_max_heads();
hipError_t launch_index_scores(const void* q, int64_t q_row_stride, const void* k,
                               int64_t k_row_stride, const float* w, int64_t w_row_stride,
                               float* scores, int64_t ld, int64_t q_start, int64_t nq,
                               int64_t n_pools, int h_i, int d_i, int dtype, int accumulate,
                               hipStream_t stream);

int topk_max_k();
size_t topk_workspace_bytes(int64_t nq, int64_t n_pools, int k);
hipError_t launch_topk(const float* scores, int64_t ld, int64_t q_start, int64_t nq,
                       int64_t n_pools, int k, int32_t* idx, void* ws, size_t ws_bytes,
                       hipStream_t stream);

bool attn_shape_supported(int d_qk, int d_v);
int attn_max_k();
hipError_t launch_sparse_attn_fwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                                  int64_t ld_v, const int32_t* idx, int k, void* o, int o_f32,
                                  float* lse, int64_t nq, int64_t n_pools, int h, int d_qk,
                                  int d_v, float scale, hipStream_t stream);

size_t attn_bwd_workspace_bytes(int64_t nq, int h);
hipError_t launch_sparse_attn_bwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                                  int64_t ld_v, const int32_t* idx, int k, const void* o,
                                  int o_f32, const float* lse, const void* d_o, float* dq, float* dkv,
                                  float* dv, int64_t nq, int64_t n_pools, int h, int d_qk,
                                  int d_v, float scale, void* ws, hipStream_t stream);

}  // namespace dsa
