// Per-query top-k selection of pooled keys by indexer score on gfx950.
//
// Page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens", section "Model and
// bottleneck": each query keeps about 2048 pooled keys; section "Four optimizations", item 1:
// the selected pool indices are int32.  Output order: score descending, lower pool index
// first among equal scores, -1 in the slots beyond the visible count.
//
// One 1024-thread block per query row.  Scores are mapped to order-preserving 32-bit keys.
// A most-significant-digit radix select (11, 11, 10 bits) finds the k-th largest key:
// each pass histograms the next digit of the keys that match the digits fixed so far in an
// LDS histogram, and a block-wide suffix scan picks the digit bin that holds the k-th
// element.  The search stops early once the chosen bin is taken whole.  A last pass walks
// the row in index order with a block-wide prefix scan (wave shuffles, then one LDS step),
// which gives every key above the threshold a slot and hands the remaining slots to the
// threshold-equal keys of lowest index, so ties resolve exactly as a stable full sort.  The
// k winners are sorted in LDS by a bitonic network on (~key, index) and written out.
// Rows with no more visible pools than k skip the select and sort the whole prefix.

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kMaxK = 4096;
constexpr int kBins = 2048;

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t index) {
  return (static_cast<uint64_t>(~key) << 32) | index;  // ascending = key desc, index asc
}

// Block-wide exclusive scan of one uint32 per thread; returns the exclusive prefix and
// writes the block total to *total.  All threads must call it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tmp,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tmp[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < kTopkWaves ? wave_tmp[lane] : 0u;
    uint32_t wi = w;
#pragma unroll
    for (int off = 1; off < kTopkWaves; off <<= 1) {
      const uint32_t o = __shfl_up(wi, off, 64);
      if (lane >= off) wi += o;
    }
    if (lane < kTopkWaves) wave_tmp[kTopkWaves + lane] = wi - w;  // exclusive wave offsets
    if (lane == kTopkWaves - 1) wave_tmp[2 * kTopkWaves] = wi;
  }
  __syncthreads();
  const uint32_t res = wave_tmp[kTopkWaves + wid] + incl - v;
  *total = wave_tmp[2 * kTopkWaves];
  __syncthreads();  // wave_tmp may be reused right after
  return res;
}

__device__ void bitonic_sort(uint64_t* buf, int n2) {
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n2 >> 1); i += kTopkThreads) {
        const int pos = 2 * i - (i & (stride - 1));
        const int partner = pos + stride;
        const bool up = (pos & size) == 0;
        const uint64_t a = buf[pos];
        const uint64_t b = buf[partner];
        if ((a > b) == up) {
          buf[pos] = b;
          buf[partner] = a;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int64_t ld, int64_t q_start,
                                                            int64_t n_pools, int k,
                                                            int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t buf[kMaxK];
  __shared__ uint32_t wave_tmp[2 * kTopkWaves + 1];
  __shared__ uint32_t pick[2];

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t vis64 = visible_pools(q_start + r, n_pools);
  const int vis = static_cast<int>(vis64);
  const float* srow = scores + r * ld;
  int32_t* orow = idx + r * k;

  if (vis <= k) {
    const int n2 = next_pow2(vis > 0 ? vis : 1);
    for (int i = tid; i < n2; i += kTopkThreads)
      buf[i] = i < vis ? composite(float_order_key(srow[i]), static_cast<uint32_t>(i)) : ~0ull;
    __syncthreads();
    bitonic_sort(buf, n2);
    for (int i = tid; i < k; i += kTopkThreads)
      orow[i] = i < vis ? static_cast<int32_t>(buf[i] & 0xFFFFFFFFu) : -1;
    return;
  }

  const int n4 = (vis + 3) >> 2;  // float4 groups; the row is padded to ld (a multiple of 4)
  uint32_t prefix = 0u, mask = 0u;
  int krem = k;
  const int shifts[3] = {21, 10, 0};
  const uint32_t digit_masks[3] = {0x7FFu, 0x7FFu, 0x3FFu};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t dmask = digit_masks[pass];
    for (int b = tid; b < kBins; b += kTopkThreads) hist[b] = 0u;
    __syncthreads();
    for (int i4 = tid; i4 < n4; i4 += kTopkThreads) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(srow + 4 * i4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e;
        if (i < vis) {
          const uint32_t key = float_order_key(v[e]);
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
        }
      }
    }
    __syncthreads();
    // Suffix scan from the top bin: thread t holds bins hi = 2047 - 2t and lo = hi - 1.
    const int hi = kBins - 1 - 2 * tid;
    const int lo = hi - 1;
    const uint32_t h_hi = hist[hi];
    const uint32_t h_lo = hist[lo];
    uint32_t total;
    const uint32_t above = block_exclusive_scan(h_hi + h_lo, wave_tmp, &total);
    const uint32_t need = static_cast<uint32_t>(krem);
    if (above < need && above + h_hi >= need) {
      pick[0] = static_cast<uint32_t>(hi);
      pick[1] = above;
    } else if (above + h_hi < need && above + h_hi + h_lo >= need) {
      pick[0] = static_cast<uint32_t>(lo);
      pick[1] = above + h_hi;
    }
    __syncthreads();
    const uint32_t bin = pick[0];
    const uint32_t above_bin = pick[1];
    const uint32_t in_bin = hist[bin];
    prefix |= bin << shift;
    mask |= dmask << shift;
    krem -= static_cast<int>(above_bin);
    __syncthreads();  // hist / pick are rewritten by the next pass
    if (in_bin == static_cast<uint32_t>(krem)) break;  // the whole bin is selected
  }

  // Ordered selection: keys above the threshold prefix take slots [0, k - krem); keys equal
  // to it take [k - krem, k) in ascending index order.
  const uint32_t n_gt = static_cast<uint32_t>(k - krem);
  uint32_t run_gt = 0u, run_eq = 0u;
  for (int base4 = 0; base4 < n4; base4 += kTopkThreads) {
    const int i4 = base4 + tid;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (i4 < n4) v = *reinterpret_cast<const f32x4*>(srow + 4 * i4);
    uint32_t keys[4];
    uint32_t cgt = 0u, ceq = 0u;
    uint32_t flags = 0u;  // bit e: above, bit 4+e: equal
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * i4 + e;
      keys[e] = float_order_key(v[e]);
      if (i4 < n4 && i < vis) {
        const uint32_t mk = keys[e] & mask;
        if (mk > prefix) {
          flags |= 1u << e;
          ++cgt;
        } else if (mk == prefix) {
          flags |= 1u << (4 + e);
          ++ceq;
        }
      }
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan(cgt | (ceq << 16), wave_tmp, &tot);
    uint32_t pos_gt = run_gt + (pre & 0xFFFFu);
    uint32_t rank_eq = run_eq + (pre >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = static_cast<uint32_t>(4 * i4 + e);
      if (flags & (1u << e)) {
        buf[pos_gt++] = composite(keys[e], i);
      } else if (flags & (1u << (4 + e))) {
        if (rank_eq < static_cast<uint32_t>(krem)) buf[n_gt + rank_eq] = composite(keys[e], i);
        ++rank_eq;
      }
    }
    run_gt += tot & 0xFFFFu;
    run_eq += tot >> 16;
    if (run_gt >= n_gt && run_eq >= static_cast<uint32_t>(krem)) break;  // uniform
  }
  const int n2 = next_pow2(k);
  for (int i = k + tid; i < n2; i += kTopkThreads) buf[i] = ~0ull;
  __syncthreads();
  bitonic_sort(buf, n2);
  for (int i = tid; i < k; i += kTopkThreads)
    orow[i] = static_cast<int32_t>(buf[i] & 0xFFFFFFFFu);
}

}  // namespace

int topk_max_k() { return kMaxK; }

size_t topk_workspace_bytes(int64_t, int64_t, int) { return 0; }

hipError_t launch_topk(const float* scores, int64_t ld, int64_t q_start, int64_t nq,
                       int64_t n_pools, int k, int32_t* idx, void*, size_t,
                       hipStream_t stream) {
  if (nq <= 0) return hipSuccess;
  if (nq >= (int64_t{1} << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<unsigned>(nq)), dim3(kTopkThreads), 0,
                     stream, scores, ld, q_start, n_pools, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
