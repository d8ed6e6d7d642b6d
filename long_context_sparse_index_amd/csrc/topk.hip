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
constexpr int kBins0 = 4096;  // first digit: the top 12 bits of the key
constexpr int kCand = 4096;   // candidate list: keys of the first digit's threshold bin

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

// Picks, from a histogram of nbins bins (nbins / 1024 consecutive bins per thread, counted
// from the top), the bin holding the need-th largest key: returns it and writes the count
// of keys in higher bins and in the bin.  All threads call it.
__device__ __forceinline__ uint32_t pick_bin(const uint32_t* hist, int nbins, uint32_t need,
                                             uint32_t* wave_tmp, uint32_t* pick,
                                             uint32_t* above_bin, uint32_t* in_bin) {
  const int per = nbins / kTopkThreads;  // 1, 2 or 4
  const int top = nbins - 1 - per * static_cast<int>(threadIdx.x);
  uint32_t h[4] = {0u, 0u, 0u, 0u};
  uint32_t mine = 0u;
  for (int j = 0; j < per; ++j) {
    h[j] = hist[top - j];
    mine += h[j];
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan(mine, wave_tmp, &total);
  for (int j = 0; j < per; ++j) {
    if (above < need && above + h[j] >= need) {
      pick[0] = static_cast<uint32_t>(top - j);
      pick[1] = above;
      pick[2] = h[j];
    }
    above += h[j];
  }
  __syncthreads();
  const uint32_t bin = pick[0];
  *above_bin = pick[1];
  *in_bin = pick[2];
  __syncthreads();  // pick is rewritten by the next call
  return bin;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int64_t ld, int64_t q_start,
                                                            int64_t n_pools, int k,
                                                            int32_t* __restrict__ idx) {
  // The first-digit histogram is dead before the candidate list is written: they share LDS.
  __shared__ uint64_t cand[kCand];  // (key << 32) | pool, in pool order
  __shared__ uint32_t hist[1024];   // 10-bit digit histograms
  __shared__ uint64_t buf[kMaxK];
  uint32_t* const hist0 = reinterpret_cast<uint32_t*>(cand);  // kBins0 counters
  static_assert(kBins0 * 4 <= kCand * 8, "first histogram fits the candidate list");
  __shared__ uint32_t wave_tmp[2 * kTopkWaves + 1];
  __shared__ uint32_t pick[3];

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
  // Histogram of the keys of the row that match (prefix, mask), on bits [shift, shift + 10).
  auto row_hist10 = [&](uint32_t prefix, uint32_t mask, int shift) {
    for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
    __syncthreads();
    for (int i4 = tid; i4 < n4; i4 += kTopkThreads) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(srow + 4 * i4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = float_order_key(v[e]);
        if (4 * i4 + e < vis && (key & mask) == prefix)
          atomicAdd(&hist[(key >> shift) & 0x3FFu], 1u);
      }
    }
    __syncthreads();
  };

  // Pass A: the top 12 bits of every visible key.
  for (int b = tid; b < kBins0; b += kTopkThreads) hist0[b] = 0u;
  __syncthreads();
  for (int i4 = tid; i4 < n4; i4 += kTopkThreads) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(srow + 4 * i4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * i4 + e < vis) atomicAdd(&hist0[float_order_key(v[e]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t above0, in0;
  const uint32_t b0 = pick_bin(hist0, kBins0, static_cast<uint32_t>(k), wave_tmp, pick,
                               &above0, &in0);
  uint32_t prefix = b0 << 20, mask = 0xFFF00000u;
  int krem = k - static_cast<int>(above0);
  // The bin is taken whole, or its keys fit the candidate list: one more pass over the row
  // places every key above the bin and moves the bin's keys to the candidates.  Otherwise
  // the remaining bits are resolved over the row itself.
  const bool whole = in0 == static_cast<uint32_t>(krem);
  const bool use_cand = !whole && in0 <= static_cast<uint32_t>(kCand);
  if (!whole && !use_cand) {
    for (int shift = 10; shift >= 0; shift -= 10) {
      row_hist10(prefix, mask, shift);
      uint32_t above_bin, in_bin;
      const uint32_t bin = pick_bin(hist, 1024, static_cast<uint32_t>(krem), wave_tmp, pick,
                                    &above_bin, &in_bin);
      prefix |= bin << shift;
      mask |= 0x3FFu << shift;
      krem -= static_cast<int>(above_bin);
      if (in_bin == static_cast<uint32_t>(krem)) break;
    }
  }

  // Ordered pass over the row: keys above the threshold prefix take slots [0, k - krem) in
  // pool order; keys equal to it take [k - krem, k) in pool order (lowest pools first), or
  // with candidates, go to the candidate list in pool order.
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
        if (use_cand)
          cand[rank_eq] = (static_cast<uint64_t>(keys[e]) << 32) | i;  // rank_eq < in0
        else if (rank_eq < static_cast<uint32_t>(krem))
          buf[n_gt + rank_eq] = composite(keys[e], i);
        ++rank_eq;
      }
    }
    run_gt += tot & 0xFFFFu;
    run_eq += tot >> 16;
    if (run_gt >= n_gt && run_eq >= (use_cand ? in0 : static_cast<uint32_t>(krem)))
      break;  // uniform
  }

  if (use_cand) {
    __syncthreads();
    // The remaining 20 bits over the candidates only.
    const int nc = static_cast<int>(in0);
    for (int shift = 10; shift >= 0; shift -= 10) {
      for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
      __syncthreads();
      for (int i = tid; i < nc; i += kTopkThreads) {
        const uint32_t key = static_cast<uint32_t>(cand[i] >> 32);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0x3FFu], 1u);
      }
      __syncthreads();
      uint32_t above_bin, in_bin;
      const uint32_t bin = pick_bin(hist, 1024, static_cast<uint32_t>(krem), wave_tmp, pick,
                                    &above_bin, &in_bin);
      prefix |= bin << shift;
      mask |= 0x3FFu << shift;
      krem -= static_cast<int>(above_bin);
      if (in_bin == static_cast<uint32_t>(krem)) break;
    }
    // Ordered selection among the candidates (in pool order; thread t takes the entries
    // [4 t, 4 t + 4)): above the prefix -> the slots after the row's winners, equal -> the
    // last krem slots, lowest pools first.
    const uint32_t base_gt = n_gt;
    const uint32_t n_gt_all = static_cast<uint32_t>(k - krem);
    uint32_t cgt = 0u, ceq = 0u, flags = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * tid + e;
      if (i < nc) {
        const uint32_t mk = static_cast<uint32_t>(cand[i] >> 32) & mask;
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
    uint32_t pos_gt = base_gt + (pre & 0xFFFFu);
    uint32_t rank_eq = pre >> 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * tid + e;
      if (i >= nc) continue;
      const uint64_t c = cand[i];
      const uint32_t key = static_cast<uint32_t>(c >> 32);
      const uint32_t pool = static_cast<uint32_t>(c);
      if (flags & (1u << e)) {
        buf[pos_gt++] = composite(key, pool);
      } else if (flags & (1u << (4 + e))) {
        if (rank_eq < static_cast<uint32_t>(krem)) buf[n_gt_all + rank_eq] = composite(key, pool);
        ++rank_eq;
      }
    }
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
