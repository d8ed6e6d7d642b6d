// Deterministic reduction of the sparse-attention backward's dK/dV contributions, without
// atomics.
//
// The pages train the layer (page "SkyRL extends GLM-5.3-Flash training context to 1 million
// tokens", from the title on) but print no backward; reproducible gradients are this
// library's option.  The dK/dV kernel of the deterministic backward writes the head-summed
// contribution of every (query row, selection slot) pair to a staging row instead of adding
// it atomically into the selected pool's gradient row.  This file turns those rows into the
// per-pool sums in a fixed order:
//   1. an inverted index (pool -> the pairs that selected it): a stable least-significant-
//      digit radix sort of the chunk's selection entries by pool, 4 bits per pass, whose
//      input order is the pairs' own order (row-major, slot-minor), so each pool's pairs come
//      out in that order whatever the thread timing;
//   2. segment bounds: the first sorted position of every pool (binary search);
//   3. one workgroup per pool adds its staging rows in the sorted order (one fp32 sum per
//      column, sequential) and adds the result to the pool's gradient row (read-modify-write:
//      no other workgroup touches that row).
// Every step is order-fixed, so the result is bit-identical from run to run.

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortPer = 8;                         // elements per lane
constexpr int kSortTile = kSortThreads * kSortPer;  // 2048 elements per workgroup
constexpr int kDigitBits = 4;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Element e of the tile: wave w owns the contiguous range [w * 512, w * 512 + 512) and takes
// it in 8 rounds of 64 consecutive elements, so (wave, round, lane) order is index order.
__device__ __forceinline__ int64_t tile_elem(int64_t base, int wave, int round, int lane) {
  return base + wave * (kSortPer * 64) + round * 64 + lane;
}

// Sort key of a selection entry (first pass): the pool, or n_pools for an empty or
// out-of-range slot (those sort last and are never reduced).
__device__ __forceinline__ int32_t entry_key(int32_t v, int32_t n_pools) {
  return (v >= 0 && v < n_pools) ? v : n_pools;
}

// Digit histogram of each tile: hist[d * n_tiles + tile].
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(
    const int32_t* __restrict__ keys, int64_t n, int shift, int32_t n_pools,
    uint32_t* __restrict__ hist, int64_t n_tiles) {
  __shared__ uint32_t wcount[kSortWaves][kBins];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
  uint32_t cnt = 0;  // lane d < kBins counts digit d over the wave's rounds
  for (int r = 0; r < kSortPer; ++r) {
    const int64_t i = tile_elem(base, wid, r, lane);
    const bool ok = i < n;
    int32_t key = ok ? keys[i] : 0;
    if (FIRST) key = entry_key(key, n_pools);
    const int d = (key >> shift) & (kBins - 1);
    for (int b = 0; b < kBins; ++b) {
      const unsigned long long m = __ballot(ok && d == b);
      if (lane == b) cnt += static_cast<uint32_t>(__popcll(m));
    }
  }
  if (lane < kBins) wcount[wid][lane] = cnt;
  __syncthreads();
  if (threadIdx.x < kBins) {
    uint32_t s = 0;
    for (int w = 0; w < kSortWaves; ++w) s += wcount[w][threadIdx.x];
    hist[threadIdx.x * n_tiles + blockIdx.x] = s;
  }
}

// Exclusive prefix sum of a[0 .. n) in place, by one workgroup of 1024 threads, in rounds
// of 16384 entries: a coalesced load into LDS, a sequential sum of 16 consecutive entries per
// thread, a block scan of those sums, the sequential rewrite, a coalesced store.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;
constexpr int kScanRound = kScanThreads * kScanPer;
__device__ __forceinline__ int scan_slot(int e) { return (e / kScanPer) * (kScanPer + 1) + e % kScanPer; }

__global__ __launch_bounds__(kScanThreads) void exclusive_scan_kernel(uint32_t* __restrict__ a,
                                                                      int64_t n) {
  __shared__ uint32_t buf[kScanThreads * (kScanPer + 1)];  // padded: no bank conflicts
  __shared__ uint32_t part[kScanThreads];
  const int tid = threadIdx.x;
  uint32_t carry = 0;
  for (int64_t base = 0; base < n; base += kScanRound) {
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int e = j * kScanThreads + tid;
      buf[scan_slot(e)] = base + e < n ? a[base + e] : 0u;
    }
    __syncthreads();
    uint32_t* mine = buf + tid * (kScanPer + 1);
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) s += mine[j];
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
      const uint32_t v = tid >= d ? part[tid - d] : 0u;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    uint32_t run = carry + part[tid] - s;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const uint32_t v = mine[j];
      mine[j] = run;
      run += v;
    }
    carry += part[kScanThreads - 1];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int e = j * kScanThreads + tid;
      if (base + e < n) a[base + e] = buf[scan_slot(e)];
    }
    __syncthreads();
  }
}

// Stable scatter of one pass: element i of the tile goes to
//   offset[digit][tile] + (elements of the tile before i with the same digit).
// FIRST: keys come from the selection (mapped by entry_key) and values are the positions.
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const int32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in, int64_t n,
    int shift, int32_t n_pools, const uint32_t* __restrict__ offs, int64_t n_tiles,
    int32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out) {
  __shared__ uint32_t run[kSortWaves][kBins];  // per wave: elements of each digit so far
  __shared__ uint32_t goff[kBins];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
  if (lane < kBins) run[wid][lane] = 0;
  if (threadIdx.x < kBins) goff[threadIdx.x] = offs[threadIdx.x * n_tiles + blockIdx.x];
  __syncthreads();
  int32_t key[kSortPer], val[kSortPer];
  uint32_t rank[kSortPer];
#pragma unroll
  for (int r = 0; r < kSortPer; ++r) {
    const int64_t i = tile_elem(base, wid, r, lane);
    const bool ok = i < n;
    key[r] = ok ? keys_in[i] : 0;
    if (FIRST) {
      key[r] = entry_key(key[r], n_pools);
      val[r] = static_cast<int32_t>(i);
    } else {
      val[r] = ok ? vals_in[i] : 0;
    }
    const int d = (key[r] >> shift) & (kBins - 1);
    // lanes of this round holding the same digit
    unsigned long long same = __ballot(ok);
#pragma unroll
    for (int b = 0; b < kDigitBits; ++b) {
      const unsigned long long m = __ballot(ok && ((d >> b) & 1));
      same &= ((d >> b) & 1) ? m : ~m;
    }
    // (a wave's LDS accesses complete in program order: every lane reads its digit's count
    // before the last lane of that digit writes the new one)
    asm volatile("" ::: "memory");
    const uint32_t before = run[wid][d];
    rank[r] = before + static_cast<uint32_t>(lanes_below(same));
    // the last lane of each digit in this round advances that digit's count
    const bool last = ok && (same >> lane) == 1ull;
    asm volatile("" ::: "memory");
    if (last) run[wid][d] = rank[r] + 1;
    asm volatile("" ::: "memory");
    if (!ok) rank[r] = 0xFFFFFFFFu;
  }
  __syncthreads();
  // offsets of the earlier waves' elements of each digit within the tile
  uint32_t wbase[kSortPer];
#pragma unroll
  for (int r = 0; r < kSortPer; ++r) {
    const int d = (key[r] >> shift) & (kBins - 1);
    uint32_t o = goff[d];
    for (int w = 0; w < wid; ++w) o += run[w][d];
    wbase[r] = o;
  }
#pragma unroll
  for (int r = 0; r < kSortPer; ++r) {
    if (rank[r] == 0xFFFFFFFFu) continue;
    const uint32_t pos = wbase[r] + rank[r];
    if (pos >= static_cast<uint64_t>(n)) continue;  // never taken when counts agree
    keys_out[pos] = key[r];
    vals_out[pos] = val[r];
  }
}

// seg[s] = first sorted position of pool s (s in [0, n_pools]); pool s's entries are
// [seg[s], seg[s + 1]).  Keys are sorted, with n_pools marking empty slots at the end: one
// thread per pool finds the first key >= s by binary search.
__global__ __launch_bounds__(256) void segment_bounds_kernel(const int32_t* __restrict__ keys,
                                                             int64_t n, int32_t n_pools,
                                                             int32_t* __restrict__ seg) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (s > n_pools) return;
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < s)
      lo = mid + 1;
    else
      hi = mid;
  }
  seg[s] = static_cast<int32_t>(lo);
}

// out[s, :] += sum over the pool's sorted entries e of stage[e, :], in sorted order.  One
// workgroup per pool, one lane per 4 columns.
// (Bounds: seg values and staged positions lie in [0, n] and [0, n) by construction; they
// are clamped anyway so that no read can leave the buffers.)
template <int W>
__global__ __launch_bounds__(((W / 4 + 63) / 64) * 64) void pool_reduce_kernel(
    const int32_t* __restrict__ seg, const int32_t* __restrict__ vals, int64_t n,
    const float* __restrict__ stage, float* __restrict__ out) {
  constexpr int kUnroll = 8;
  const int64_t s = blockIdx.x;
  const int c = threadIdx.x;
  const int64_t beg = seg[s] < 0 ? 0 : seg[s];
  const int64_t end = seg[s + 1] < n ? seg[s + 1] : n;
  if (beg >= end || c >= W / 4) return;
  auto row = [&](int64_t e) {
    const uint32_t v = static_cast<uint32_t>(vals[e]);
    return stage + static_cast<int64_t>(v < n ? v : 0) * W + 4 * c;
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int64_t e = beg;
  for (; e + kUnroll <= end; e += kUnroll) {
    f32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = *reinterpret_cast<const f32x4*>(row(e + u));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += x[u];
  }
  for (; e < end; ++e) acc += *reinterpret_cast<const f32x4*>(row(e));
  f32x4* o = reinterpret_cast<f32x4*>(out + s * W + 4 * c);
  *o = *o + acc;
}

int64_t tiles_of(int64_t n) { return (n + kSortTile - 1) / kSortTile; }

int pass_count(int64_t n_pools) {
  int bits = 1;
  while ((int64_t{1} << bits) <= n_pools) ++bits;  // keys lie in [0, n_pools]
  return (bits + kDigitBits - 1) / kDigitBits;
}

size_t align256(size_t b) { return (b + 255) & ~size_t{255}; }

struct ReduceLayout {
  size_t keys[2], vals[2], hist, seg, total;
};

ReduceLayout reduce_layout(int64_t n_entries, int64_t n_pools) {
  ReduceLayout L{};
  const size_t n = static_cast<size_t>(n_entries > 0 ? n_entries : 0);
  size_t off = 0;
  for (int i = 0; i < 2; ++i) {
    L.keys[i] = off;
    off += align256(n * sizeof(int32_t));
    L.vals[i] = off;
    off += align256(n * sizeof(int32_t));
  }
  L.hist = off;
  off += align256(static_cast<size_t>(kBins * tiles_of(n_entries)) * sizeof(uint32_t));
  L.seg = off;
  off += align256(static_cast<size_t>(n_pools + 2) * sizeof(int32_t));
  L.total = off;
  return L;
}

template <int W>
hipError_t launch_reduce_w(const int32_t* seg, const int32_t* vals, int64_t n,
                           const float* stage, float* out, int64_t n_pools, hipStream_t s) {
  hipLaunchKernelGGL((pool_reduce_kernel<W>), dim3(static_cast<unsigned>(n_pools)),
                     dim3(((W / 4 + 63) / 64) * 64), 0, s, seg, vals, n, stage, out);
  return hipGetLastError();
}

hipError_t launch_reduce(int w, const int32_t* seg, const int32_t* vals, int64_t n,
                         const float* stage, float* out, int64_t n_pools, hipStream_t s) {
  switch (w) {
    case 128: return launch_reduce_w<128>(seg, vals, n, stage, out, n_pools, s);
    case 256: return launch_reduce_w<256>(seg, vals, n, stage, out, n_pools, s);
    case 512: return launch_reduce_w<512>(seg, vals, n, stage, out, n_pools, s);
    case 576: return launch_reduce_w<576>(seg, vals, n, stage, out, n_pools, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t pool_reduce_workspace_bytes(int64_t n_entries, int64_t n_pools) {
  return reduce_layout(n_entries, n_pools).total;
}

hipError_t launch_pool_reduce(const int32_t* idx, int64_t rows, int k, int64_t n_pools,
                              const float* stage_k, int w_k, float* out_k,
                              const float* stage_v, int w_v, float* out_v, void* ws,
                              hipStream_t s) {
  const int64_t n = rows * k;
  if (n <= 0 || n_pools <= 0) return hipSuccess;
  if (n >= (int64_t{1} << 31) || n_pools >= (int64_t{1} << 31) - 1)
    return hipErrorInvalidConfiguration;
  const ReduceLayout L = reduce_layout(n, n_pools);
  char* base = static_cast<char*>(ws);
  int32_t* keys[2] = {reinterpret_cast<int32_t*>(base + L.keys[0]),
                      reinterpret_cast<int32_t*>(base + L.keys[1])};
  int32_t* vals[2] = {reinterpret_cast<int32_t*>(base + L.vals[0]),
                      reinterpret_cast<int32_t*>(base + L.vals[1])};
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist);
  int32_t* seg = reinterpret_cast<int32_t*>(base + L.seg);
  const int64_t n_tiles = tiles_of(n);
  const int32_t np = static_cast<int32_t>(n_pools);
  const int passes = pass_count(n_pools);
  int cur = 0;
  for (int p = 0; p < passes; ++p) {
    const int shift = p * kDigitBits;
    if (p == 0)
      hipLaunchKernelGGL((radix_hist_kernel<true>), dim3(static_cast<unsigned>(n_tiles)),
                         dim3(kSortThreads), 0, s, idx, n, shift, np, hist, n_tiles);
    else
      hipLaunchKernelGGL((radix_hist_kernel<false>), dim3(static_cast<unsigned>(n_tiles)),
                         dim3(kSortThreads), 0, s, keys[cur], n, shift, np, hist, n_tiles);
    hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, hist,
                       kBins * n_tiles);
    const int nxt = p == 0 ? 0 : cur ^ 1;
    if (p == 0)
      hipLaunchKernelGGL((radix_scatter_kernel<true>), dim3(static_cast<unsigned>(n_tiles)),
                         dim3(kSortThreads), 0, s, idx, nullptr, n, shift, np, hist, n_tiles,
                         keys[nxt], vals[nxt]);
    else
      hipLaunchKernelGGL((radix_scatter_kernel<false>), dim3(static_cast<unsigned>(n_tiles)),
                         dim3(kSortThreads), 0, s, keys[cur], vals[cur], n, shift, np, hist,
                         n_tiles, keys[nxt], vals[nxt]);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    cur = nxt;
  }
  hipLaunchKernelGGL(segment_bounds_kernel, dim3(static_cast<unsigned>((n_pools + 1 + 255) / 256)),
                     dim3(256), 0, s, keys[cur], n, np, seg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_reduce(w_k, seg, vals[cur], n, stage_k, out_k, n_pools, s);
  if (e != hipSuccess || !stage_v) return e;
  return launch_reduce(w_v, seg, vals[cur], n, stage_v, out_v, n_pools, s);
}

}  // namespace dsa
