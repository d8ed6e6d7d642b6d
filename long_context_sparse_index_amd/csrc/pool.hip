// Pooled keys: one key row per 4 tokens, on gfx950.
//
// Page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens": the indexer scores
// "one pool per 4 tokens" (section "Model and bottleneck"), pooled with "k-pool gate scores"
// (section "Four optimizations", item 3).  The pages print no formula; the reading taken:
//     w_i = softmax(g[4s], .., g[4s+3])_i,   pooled[s, :] = sum_{i<4} w_i x[4s+i, :]
// for s < floor(n_tokens / 4), rounded once to bf16.  The same call pools any key table
// (the indexer keys, the latent KV rows).
//
// One thread per 8 columns of a pool: four 16-byte row loads, the gate softmax and the
// weighted sum in fp32, one packed round-to-nearest-even conversion, one 16-byte store.
// Consecutive threads take consecutive column chunks of a pool, so loads and stores are
// coalesced; the kernel is bound by HBM (8 bytes read per 2 written for each column).

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kPoolThreads = 256;

__global__ __launch_bounds__(kPoolThreads) void pool_keys_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const float* __restrict__ gate,
    int64_t n_pools, int chunks, uint16_t* __restrict__ out, int64_t ld_out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPoolThreads + threadIdx.x;
  if (t >= n_pools * chunks) return;
  const int64_t s = t / chunks;
  const int c = static_cast<int>(t - s * chunks) * 8;
  float g[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) g[i] = gate[4 * s + i];
  const float m = __builtin_fmaxf(__builtin_fmaxf(g[0], g[1]), __builtin_fmaxf(g[2], g[3]));
  float e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = expf(g[i] - m);
  const float inv = 1.0f / ((e[0] + e[1]) + (e[2] + e[3]));
  u32x4 rows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    rows[i] = *reinterpret_cast<const u32x4*>(x + (4 * s + i) * ld_x + c);
  f32x8 acc;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = e[i] * inv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = __builtin_fmaf(w, __uint_as_float(rows[i][j] << 16), acc[2 * j]);
      acc[2 * j + 1] = __builtin_fmaf(w, __uint_as_float(rows[i][j] & 0xFFFF0000u), acc[2 * j + 1]);
    }
  }
  const bf16x8 r = __builtin_convertvector(acc, bf16x8);
  *reinterpret_cast<u32x4*>(out + s * ld_out + c) = __builtin_bit_cast(u32x4, r);
}

}  // namespace

hipError_t launch_pool_keys(const void* x, int64_t ld_x, const float* gate, int64_t n_tokens,
                            int d, void* out, int64_t ld_out, hipStream_t stream) {
  const int64_t n_pools = n_tokens / 4;
  const int chunks = d / 8;
  const int64_t threads = n_pools * chunks;
  if (threads <= 0) return hipSuccess;
  const int64_t blocks = (threads + kPoolThreads - 1) / kPoolThreads;
  if (blocks >= (int64_t{1} << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pool_keys_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPoolThreads),
                     0, stream, static_cast<const uint16_t*>(x), ld_x, gate, n_pools, chunks,
                     static_cast<uint16_t*>(out), ld_out);
  return hipGetLastError();
}

}  // namespace dsa
