// Per-query top-k selection of pooled keys by indexer score on gfx950.
//
// Page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens", section "Model and
// bottleneck": each query keeps about 2048 pooled keys; section "Four optimizations", item 1:
// the selected pool indices are int32.  Output order: score descending, lower pool index
// first among equal scores, -1 in the slots beyond the visible count.
//
// One 1024-thread block per query row.  Scores are mapped to order-preserving 32-bit keys.
// Pass A streams the row into an LDS histogram of the top 12 key bits, and a block-wide
// suffix scan picks the bin holding the k-th largest key.  When that bin is taken whole or
// holds at most 4096 keys (the usual case), pass B streams the row once more and moves the
// keys above the bin to the winner list and the bin's keys to an LDS candidate list, both
// through LDS slot counters, so pass B needs no block-wide synchronisation.  The remaining
// 20 key bits are then resolved over the candidates alone (two 10-bit digit histograms);
// if more candidates share the exact threshold key than slots remain, a select on the
// pool index among them keeps the lowest pools, so ties resolve exactly as a stable full
// sort.  A bin too large for the list is resolved over the row itself, followed by a
// pool-ordered pass (block-wide prefix scans) that gives the remaining slots to the
// threshold-equal keys of lowest pool.  The k winners are sorted on (~key, pool) by a
// bitonic network held in registers (lane shuffles within a wave, LDS across waves) and
// written out.  Rows with no more visible pools than k sort the whole prefix.

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kMaxK = 4096;
constexpr int kBins0 = 4096;  // first digit: the top 12 bits of the key
constexpr int kCand = 4096;   // candidate list: keys of the first digit's threshold bin
constexpr int kLoads = 2;     // float4 loads in flight per thread while streaming a row
constexpr int kSampleMinVis = 32768;  // rows at least this long take the sampled select
constexpr int kPeelMax = 8;           // winners peeled off before a halved final sort

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

// Value of lane (lane ^ LS) of the wave, by VALU cross-lane moves: DPP quad permutes for 1
// and 2, a half-row mirror (lane ^ 7) then a quad reversal (lane ^ 3) for 4, a row rotation
// by 8 for 8, and the gfx950 row and half-wave swaps for 16 and 32.
template <int LS>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  if constexpr (LS == 1) {
    return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (LS == 2) {
    return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (LS == 4) {
    const uint32_t m = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
    return __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true);               // quad_perm [3,2,1,0]
  } else if constexpr (LS == 8) {
    return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else if constexpr (LS == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(LS == 32, "lane strides 1..32");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

template <int LS>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v) {
  const uint32_t lo = lane_xor<LS>(static_cast<uint32_t>(v));
  const uint32_t hi = lane_xor<LS>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v, int ls) {
  switch (ls) {
    case 1: return lane_xor_u64<1>(v);
    case 2: return lane_xor_u64<2>(v);
    case 4: return lane_xor_u64<4>(v);
    case 8: return lane_xor_u64<8>(v);
    case 16: return lane_xor_u64<16>(v);
    default: return lane_xor_u64<32>(v);
  }
}

// Ascending bitonic sort of buf[0, 1024 R).  Index bits [0, log2 R) select one of the R
// registers of a thread, the next 6 bits the lane and the top 4 bits the wave, so the most
// frequent (smallest) strides are register pairs, the next ones VALU lane exchanges, and
// only strides across waves go through LDS, alternating between buf and alt so that one
// barrier per such stage suffices.
template <int R>
__device__ __forceinline__ void bitonic_sort_regs(uint64_t* buf, uint64_t* alt) {
  constexpr int kLogR = R == 1 ? 0 : (R == 2 ? 1 : 2);
  constexpr int kN = kTopkThreads * R;
  static_assert(R == 1 || R == 2 || R == 4, "1, 2 or 4 keys per thread");
  const int lane = threadIdx.x & 63;
  const int base = ((threadIdx.x >> 6) << (6 + kLogR)) | (lane << kLogR);
  uint64_t v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = buf[base | j];
  bool to_alt = false;
#pragma unroll
  for (int size = 2; size <= kN; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < R) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          if (j & stride) continue;
          const uint64_t a = v[j], b = v[j | stride];
          const bool up = ((base | j) & size) == 0;
          const bool sw = (b < a) == up;
          v[j] = sw ? b : a;
          v[j | stride] = sw ? a : b;
        }
      } else if (stride < 64 * R) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int i = base | j;
          const uint64_t p = lane_xor_u64(v[j], stride >> kLogR);
          const bool take_min = ((i & size) == 0) == ((i & stride) == 0);
          v[j] = ((p < v[j]) == take_min) ? p : v[j];
        }
      } else {
        uint64_t* x = to_alt ? alt : buf;
        to_alt = !to_alt;
#pragma unroll
        for (int j = 0; j < R; ++j) x[base | j] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int i = base | j;
          const uint64_t p = x[i ^ stride];
          const bool take_min = ((i & size) == 0) == ((i & stride) == 0);
          v[j] = ((p < v[j]) == take_min) ? p : v[j];
        }
      }
    }
  }
  __syncthreads();  // the last LDS stage may still read buf
#pragma unroll
  for (int j = 0; j < R; ++j) buf[base | j] = v[j];
  __syncthreads();
}

// Sorts buf[0, n2) ascending, n2 a power of two <= kMaxK; buf[n2, max(n2, 1024)) must hold
// ~0 (padding sorts last).  alt is scratch of the same size.
__device__ __forceinline__ void sort_keys(uint64_t* buf, uint64_t* alt, int n2) {
  if (n2 <= kTopkThreads)
    bitonic_sort_regs<1>(buf, alt);
  else if (n2 <= 2 * kTopkThreads)
    bitonic_sort_regs<2>(buf, alt);
  else
    bitonic_sort_regs<4>(buf, alt);
}

// First digit window of a select over keys known to lie in [lo, hi]: they share the bits
// above the highest bit where lo and hi differ (mask, prefix), and the 10-bit window ends at
// that bit, so the keys spread over the histogram instead of piling into the few bins of a
// shared exponent (fewer digit rounds and fewer colliding LDS atomics).
__device__ __forceinline__ void digit_window(uint32_t lo, uint32_t hi, uint32_t* mask,
                                             uint32_t* prefix, int* shift) {
  const uint32_t diff = lo ^ hi;
  if (diff == 0u) {  // one key value: a single window over the low bits, ties by pool
    *mask = 0xFFFFFC00u;
    *shift = 0;
  } else {
    const int hb = 31 - __builtin_clz(diff);
    *mask = ~((2u << hb) - 1u);  // 2u << 31 == 0: no shared bits
    *shift = hb >= 9 ? hb - 9 : 0;
  }
  *prefix = lo & *mask;
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

// FROM_CAND: the row's candidates come from a list written by the indexer (TopkCand)
// instead of a score row; the row is flagged for the exact fallback when the list does not
// hold between k and kCand entries.  Otherwise a non-null gate skips rows whose gate is 0.
template <bool FROM_CAND>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void topk_kernel(const float* __restrict__ scores,
                                                            int64_t ld, int64_t q_start,
                                                            int64_t n_pools, int k,
                                                            int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ gate,
                                                            TopkCand cs) {
  // The first-digit histogram is dead before the candidate list is written: they share LDS.
  __shared__ uint64_t cand[kCand];  // (key << 32) | pool
  __shared__ uint32_t hist[1024];   // 10-bit digit histograms
  __shared__ uint64_t buf[kMaxK];
  uint32_t* const hist0 = reinterpret_cast<uint32_t*>(cand);  // kBins0 counters
  static_assert(kBins0 * 4 <= kCand * 8, "first histogram fits the candidate list");
  __shared__ uint32_t wave_tmp[2 * kTopkWaves + 1];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t fill[3];  // slots taken in buf and in cand; sample size
  __shared__ uint32_t cand_max;  // largest key collected by the sampled path
  __shared__ uint64_t peel_max[kTopkWaves];  // per-wave maxima while peeling the tail
  __shared__ uint32_t peel_pos;

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  if (!FROM_CAND && gate && gate[r] == 0) return;
  const int64_t vis64 = visible_pools(q_start + r, n_pools);
  const int vis = static_cast<int>(vis64);
  const float* srow = scores + r * ld;
  int32_t* orow = idx + r * k;

  // Exact resolution among the candidates cand[0, nc): the keys are known to hold every
  // key of the row that can still be selected above the current prefix (mask, prefix),
  // krem slots remain.  10-bit digit windows at `shift` and then shift - 10 ... 0 (a last
  // window may overlap bits already fixed); a prefix held by more candidates than slots
  // after all 32 bits is an exact tie, resolved by pool.  Winners (keys above the prefix,
  // or on it and among the lowest pools) go to buf through fill[0].
  auto resolve_candidates = [&](int nc, uint32_t prefix, uint32_t mask, int krem, int shift) {
    bool tied = false;
    uint32_t n_tied = 0u;  // candidates on the final prefix (when tied: the exact key)
    for (;; shift = shift > 10 ? shift - 10 : (shift > 0 ? 0 : -1)) {
      if (shift < 0) break;
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
      n_tied = in_bin;
      tied = in_bin != static_cast<uint32_t>(krem);
      if (!tied) break;
    }
    // More candidates carry the threshold key than slots remain: the lowest pools among
    // them win.  Up to one per thread, each tied candidate counts the tied pools below
    // its own (pools are distinct, so these ranks are exact) and the one ranked krem - 1
    // gives the largest winning pool.  More of them: a select on ~pool (larger = lower
    // pool) over 10-bit windows at bits 22, 12, 2 and 0 ends with exactly krem of them.
    uint32_t pprefix = 0u, pmask = 0u;
    if (tied && n_tied <= static_cast<uint32_t>(kTopkThreads)) {
      if (tid == 0) fill[1] = 0u;  // the candidate count is no longer needed
      __syncthreads();
      for (int i = tid; i < nc; i += kTopkThreads) {
        const uint64_t c = cand[i];
        if (static_cast<uint32_t>(c >> 32) == prefix)
          hist[atomicAdd(&fill[1], 1u)] = static_cast<uint32_t>(c);  // < n_tied
      }
      __syncthreads();
      if (tid < static_cast<int>(n_tied)) {
        const uint32_t mine = hist[tid];
        uint32_t rank = 0u;
        for (int i = 0; i < static_cast<int>(n_tied); ++i) rank += hist[i] < mine ? 1u : 0u;
        if (rank == static_cast<uint32_t>(krem - 1)) pick[0] = mine;
      }
      __syncthreads();
      pmask = ~0u;
      pprefix = ~pick[0];  // winners: pool <= that pool
    } else if (tied) {
      for (int pshift = 22;; pshift = pshift > 2 ? pshift - 10 : 0) {
        for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
        __syncthreads();
        for (int i = tid; i < nc; i += kTopkThreads) {
          const uint64_t c = cand[i];
          const uint32_t npool = ~static_cast<uint32_t>(c);
          if (static_cast<uint32_t>(c >> 32) == prefix && (npool & pmask) == pprefix)
            atomicAdd(&hist[(npool >> pshift) & 0x3FFu], 1u);
        }
        __syncthreads();
        uint32_t above_bin, in_bin;
        const uint32_t bin = pick_bin(hist, 1024, static_cast<uint32_t>(krem), wave_tmp, pick,
                                      &above_bin, &in_bin);
        pprefix |= bin << pshift;
        pmask |= 0x3FFu << pshift;
        krem -= static_cast<int>(above_bin);
        if (in_bin == static_cast<uint32_t>(krem) || pshift == 0) break;
      }
    }
    // Winners among the candidates: above the prefix, or on it and (when tied) at or
    // above the pool threshold.
    for (int i = tid; i < nc; i += kTopkThreads) {
      const uint64_t c = cand[i];
      const uint32_t key = static_cast<uint32_t>(c >> 32);
      const uint32_t pool = static_cast<uint32_t>(c);
      const uint32_t mk = key & mask;
      if (mk > prefix || (mk == prefix && (~pool & pmask) >= pprefix))
        buf[atomicAdd(&fill[0], 1u)] = composite(key, pool);  // k winners in all
    }
  };

  // Sorts the k winners in buf[0, k) ascending on (~key, pool).  When k is a little above a
  // power of two (k = 2051 of the Flash shape), the k - 2^m worst winners are peeled off to
  // the tail first, largest first, by block-wide maxima (three barriers each), so the
  // bitonic network sorts 2^m keys instead of 2^(m+1).
  auto sort_winners = [&]() {
    int n2 = max(next_pow2(k), kTopkThreads);
    int kk = k;
    const int half = n2 >> 1;
    if (n2 > kTopkThreads && k - half <= kPeelMax) {
      const int lane = tid & 63;
      __syncthreads();  // every winner is in buf
      for (int m = k; m > half; --m) {  // the largest of buf[0, m) goes to buf[m - 1]
        uint64_t v = 0ull;
        for (int j = tid; j < m; j += kTopkThreads) v = buf[j] > v ? buf[j] : v;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          const uint64_t o = lane_xor_u64(v, off);
          v = o > v ? o : v;
        }
        if (lane == 0) peel_max[tid >> 6] = v;
        __syncthreads();
        uint64_t gm = peel_max[0];
#pragma unroll
        for (int w = 1; w < kTopkWaves; ++w) gm = peel_max[w] > gm ? peel_max[w] : gm;
        for (int j = tid; j < m; j += kTopkThreads)
          if (buf[j] == gm) peel_pos = static_cast<uint32_t>(j);  // winners are distinct
        __syncthreads();
        if (tid == 0) {
          const uint32_t pos = peel_pos;
          buf[pos] = buf[m - 1];
          buf[m - 1] = gm;
        }
        __syncthreads();
      }
      n2 = half;
      kk = half;
    }
    for (int i = kk + tid; i < n2; i += kTopkThreads) buf[i] = ~0ull;
    __syncthreads();
    sort_keys(buf, cand, n2);
  };

  if constexpr (FROM_CAND) {
    // The list holds every visible entry whose key is >= the row's threshold (all visible
    // entries when the threshold is 0).  With at least k (or all vis <= k) and at most kCand
    // of them it holds the k winners, resolved here as in the sampled path; any other count
    // leaves the row to the fallback (indexer scores + the score-row select).
    // Every list has room for kCand entries: all of it is requested before the count
    // arrives (entries past the count are ignored), so the loads take one round trip.
    static_assert(kCand == 4 * kTopkThreads, "four list entries per thread");
    const uint64_t* crow = cs.cand + r * cs.cap;
    uint64_t pre[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pre[u] = crow[u * kTopkThreads + tid];
    const uint32_t n = cs.cnt[r];
    const bool usable = vis <= k ? n == static_cast<uint32_t>(vis)
                                 : (n >= static_cast<uint32_t>(k) &&
                                    n <= static_cast<uint32_t>(kCand));
    if (tid == 0) {
      cs.fail[r] = usable ? 0 : 1;
      if (!usable) atomicOr(cs.any_fail, 1);
    }
    if (!usable) return;
    if (vis <= k) {
      const int n2 = max(next_pow2(vis > 0 ? vis : 1), kTopkThreads);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = u * kTopkThreads + tid;
        if (i < n2)
          buf[i] = i < vis ? composite(static_cast<uint32_t>(pre[u] >> 32),
                                       static_cast<uint32_t>(pre[u]))
                           : ~0ull;
      }
      __syncthreads();
      sort_keys(buf, cand, n2);
      for (int i = tid; i < k; i += kTopkThreads)
        orow[i] = i < vis ? static_cast<int32_t>(buf[i] & 0xFFFFFFFFu) : -1;
      return;
    }
    if (tid < 3) fill[tid] = 0u;
    if (tid == 0) cand_max = 0u;
    __syncthreads();
    uint32_t my_max = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = u * kTopkThreads + tid;
      if (i < static_cast<int>(n)) {
        cand[i] = pre[u];
        const uint32_t key = static_cast<uint32_t>(pre[u] >> 32);
        my_max = key > my_max ? key : my_max;
      }
    }
    if (my_max) atomicMax(&cand_max, my_max);
    __syncthreads();
    const uint32_t t_est = cs.t_est[r];
    uint32_t mask, prefix;
    int shift;
    digit_window(t_est, cand_max, &mask, &prefix, &shift);
    resolve_candidates(static_cast<int>(n), prefix, mask, k, shift);
    sort_winners();
    for (int i = tid; i < k; i += kTopkThreads)
      orow[i] = static_cast<int32_t>(buf[i] & 0xFFFFFFFFu);
    return;
  }

  if (vis <= k) {
    const int n2 = max(next_pow2(vis > 0 ? vis : 1), kTopkThreads);
    for (int i = tid; i < n2; i += kTopkThreads)
      buf[i] = i < vis ? composite(float_order_key(srow[i]), static_cast<uint32_t>(i)) : ~0ull;
    __syncthreads();
    sort_keys(buf, cand, n2);
    for (int i = tid; i < k; i += kTopkThreads)
      orow[i] = i < vis ? static_cast<int32_t>(buf[i] & 0xFFFFFFFFu) : -1;
    return;
  }

  const int n4 = (vis + 3) >> 2;  // float4 groups; the row is padded to ld (a multiple of 4)
  // Calls f(i4, v) for every float4 group of the row, kLoads loads in flight per thread.
  // Groups past the row end carry keys with index >= vis, which f must skip.
  auto stream_row = [&](auto&& f) {
    for (int base = 0; base < n4; base += kLoads * kTopkThreads) {
      f32x4 v[kLoads];
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int i4 = base + u * kTopkThreads + tid;
        v[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kLoads; ++u) f(base + u * kTopkThreads + tid, v[u]);
    }
  };

  // Long rows: estimate the key ranked about 1.5 k from a 1/16 sample of the row, then
  // one pass collects every key at or above the estimate into the candidate list.  When
  // the list holds at least k and at most kCand keys it contains the k winners, which are
  // then resolved from LDS alone: the row is read 1 1/16 times instead of twice.  Any
  // other count (rare; heavy ties) falls back to the two-pass select below.
  bool sampled = false;
  if (vis >= kSampleMinVis && 3 * k <= 2 * kCand) {
    if (tid < 3) fill[tid] = 0u;
    if (tid == 0) cand_max = 0u;
    for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
    __syncthreads();
    // The sample: 256-byte pieces (16 float4), one every 4 KB (256 float4) of the row, or
    // sparser on rows past 2^18 keys so that there are at most 256 pieces: four per group
    // of 16 threads, all loaded before any is used (one memory latency per sample pass).
    const int piece_stride = 256 * ((n4 + 65535) / 65536);
    auto stream_sample = [&](auto&& f) {
      f32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i4 = piece_stride * ((tid >> 4) + 64 * j) + (tid & 15);
        v[j] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) f(piece_stride * ((tid >> 4) + 64 * j) + (tid & 15), v[j]);
    };
    uint32_t n_local = 0u;
    stream_sample([&](int i4, const f32x4& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * i4 + e < vis) {
          atomicAdd(&hist[float_order_key(v[e]) >> 22], 1u);
          ++n_local;
        }
    });
    if (n_local) atomicAdd(&fill[2], n_local);
    __syncthreads();
    const uint32_t n_sample = fill[2];
    // Rank of the estimate in the sample: 1.5 k scaled to the sample (at least 1).
    const int64_t target = k + k / 2;
    uint32_t rank = static_cast<uint32_t>((target * n_sample + vis / 2) / vis);
    rank = rank < 1u ? 1u : (rank > n_sample ? n_sample : rank);
    uint32_t above1, in1;
    const uint32_t bin1 = pick_bin(hist, 1024, rank, wave_tmp, pick, &above1, &in1);
    const uint32_t prefix1 = bin1 << 22;
    for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
    __syncthreads();
    stream_sample([&](int i4, const f32x4& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = float_order_key(v[e]);
        if (4 * i4 + e < vis && (key & 0xFFC00000u) == prefix1)
          atomicAdd(&hist[(key >> 12) & 0x3FFu], 1u);
      }
    });
    __syncthreads();
    uint32_t above2, in2;
    const uint32_t bin2 = pick_bin(hist, 1024, rank - above1, wave_tmp, pick, &above2, &in2);
    const uint32_t t_est = prefix1 | (bin2 << 12);  // lower edge of the estimate's 20-bit bin
    uint32_t my_max = 0u;
    stream_row([&](int i4, const f32x4& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t i = static_cast<uint32_t>(4 * i4 + e);
        const uint32_t key = float_order_key(v[e]);
        if (static_cast<int>(i) < vis && key >= t_est) {
          const uint32_t slot = atomicAdd(&fill[1], 1u);
          if (slot < static_cast<uint32_t>(kCand))
            cand[slot] = (static_cast<uint64_t>(key) << 32) | i;
          my_max = key > my_max ? key : my_max;
        }
      }
    });
    if (my_max) atomicMax(&cand_max, my_max);
    __syncthreads();
    const uint32_t n_cand = fill[1];
    sampled = n_cand >= static_cast<uint32_t>(k) && n_cand <= static_cast<uint32_t>(kCand);
    __syncthreads();  // fill[] is reset below
    if (sampled) {
      // The candidates lie in [t_est, cand_max]: the top bits those two share are fixed, and
      // the select starts right below them.
      uint32_t mask, prefix;
      int shift;
      digit_window(t_est, cand_max, &mask, &prefix, &shift);
      resolve_candidates(static_cast<int>(n_cand), prefix, mask, k, shift);
    }
  }

  if (!sampled) {
    // Pass A: the top 12 bits of every visible key.
    for (int b = tid; b < kBins0; b += kTopkThreads) hist0[b] = 0u;
    if (tid < 2) fill[tid] = 0u;
    __syncthreads();
    stream_row([&](int i4, const f32x4& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * i4 + e < vis) atomicAdd(&hist0[float_order_key(v[e]) >> 20], 1u);
    });
    __syncthreads();
    uint32_t above0, in0;
    const uint32_t b0 = pick_bin(hist0, kBins0, static_cast<uint32_t>(k), wave_tmp, pick,
                                 &above0, &in0);
    uint32_t prefix = b0 << 20, mask = 0xFFF00000u;
    int krem = k - static_cast<int>(above0);
    const bool whole = in0 == static_cast<uint32_t>(krem);

    if (whole || in0 <= static_cast<uint32_t>(kCand)) {
      // Pass B, in any order: keys above the bin (and the bin's own when it is taken whole)
      // are winners; the bin's keys otherwise go to the candidate list.  The final sort
      // orders the winners, so slots come from LDS counters.
      stream_row([&](int i4, const f32x4& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t i = static_cast<uint32_t>(4 * i4 + e);
          const uint32_t key = float_order_key(v[e]);
          const uint32_t d = key >> 20;
          if (static_cast<int>(i) < vis && d >= b0) {
            if (d > b0 || whole)
              buf[atomicAdd(&fill[0], 1u)] = composite(key, i);  // < above0 + in0 (whole) <= k
            else
              cand[atomicAdd(&fill[1], 1u)] = (static_cast<uint64_t>(key) << 32) | i;  // < in0
          }
        }
      });
      __syncthreads();
      // The remaining 20 key bits over the bin's keys only (their winners join buf).
      if (!whole) resolve_candidates(static_cast<int>(in0), prefix, mask, krem, 10);
    } else {
      // The bin holds more keys than the candidate list: resolve the remaining bits over the
      // row, then one ordered pass places the keys above the threshold and hands the krem
      // slots left to the threshold-equal keys of lowest pool.
      for (int shift = 10; shift >= 0; shift -= 10) {
        for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
        __syncthreads();
        stream_row([&](int i4, const f32x4& v) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = float_order_key(v[e]);
            if (4 * i4 + e < vis && (key & mask) == prefix)
              atomicAdd(&hist[(key >> shift) & 0x3FFu], 1u);
          }
        });
        __syncthreads();
        uint32_t above_bin, in_bin;
        const uint32_t bin = pick_bin(hist, 1024, static_cast<uint32_t>(krem), wave_tmp, pick,
                                      &above_bin, &in_bin);
        prefix |= bin << shift;
        mask |= 0x3FFu << shift;
        krem -= static_cast<int>(above_bin);
        if (in_bin == static_cast<uint32_t>(krem)) break;
      }
      // Thread t takes the 16 consecutive keys [16 t, 16 t + 16) of each 16384-key group, so a
      // block scan of the per-thread counts gives pool-ordered ranks.
      constexpr int kU = 4;  // float4 per thread per group
      const uint32_t n_gt = static_cast<uint32_t>(k - krem);
      uint32_t run_gt = 0u, run_eq = 0u;
      for (int base4 = 0; base4 < n4; base4 += kU * kTopkThreads) {
        f32x4 cur[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i4 = base4 + kU * tid + u;
          cur[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        uint32_t cgt = 0u, ceq = 0u;
        uint32_t flags = 0u;  // bit e: above, bit 16 + e: equal
#pragma unroll
        for (int e = 0; e < 4 * kU; ++e) {
          const int i = 4 * (base4 + kU * tid) + e;
          const uint32_t mk = float_order_key(cur[e >> 2][e & 3]) & mask;
          if (i < vis) {
            if (mk > prefix) {
              flags |= 1u << e;
              ++cgt;
            } else if (mk == prefix) {
              flags |= 1u << (16 + e);
              ++ceq;
            }
          }
        }
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan(cgt | (ceq << 16), wave_tmp, &tot);
        if (flags != 0u) {
          uint32_t pos_gt = run_gt + (pre & 0xFFFFu);
          uint32_t rank_eq = run_eq + (pre >> 16);
#pragma unroll
          for (int e = 0; e < 4 * kU; ++e) {
            const uint32_t i = static_cast<uint32_t>(4 * (base4 + kU * tid) + e);
            const uint32_t key = float_order_key(cur[e >> 2][e & 3]);
            if (flags & (1u << e)) {
              buf[pos_gt++] = composite(key, i);
            } else if (flags & (1u << (16 + e))) {
              if (rank_eq < static_cast<uint32_t>(krem)) buf[n_gt + rank_eq] = composite(key, i);
              ++rank_eq;
            }
          }
        }
        run_gt += tot & 0xFFFFu;
        run_eq += tot >> 16;
        if (run_gt >= n_gt && run_eq >= static_cast<uint32_t>(krem)) break;  // uniform
      }
    }
  }

  sort_winners();
  for (int i = tid; i < k; i += kTopkThreads)
    orow[i] = static_cast<int32_t>(buf[i] & 0xFFFFFFFFu);
}

// Per-row threshold for the fused select, from the scores of every 2^shift-th visible pool
// (sample row of vs = ceil(V / 2^shift) entries): the lower edge of a key bin (20 bits
// below the sample's common key prefix, or the top 22 key bits on very long rows) that
// holds the sample key ranked 1.5 k * vs / V, so that about 1.5 k keys of the full row
// reach it.  Rows with at most kCand visible pools get threshold 0 (every visible key).  Also
// zeroes the row's candidate count, and block 0 the any-fallback flag.
__global__ __launch_bounds__(kTopkThreads) void threshold_kernel(
    const float* __restrict__ sample, int64_t ld_sample, int64_t q_start, int64_t n_pools,
    int shift, int k, uint32_t* __restrict__ t_est, uint32_t* __restrict__ cnt,
    int32_t* __restrict__ any_fail) {
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t wave_tmp[2 * kTopkWaves + 1];
  __shared__ uint32_t pick[3];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  if (tid == 0) {
    cnt[r] = 0u;
    if (r == 0) *any_fail = 0;
  }
  const int64_t vis = visible_pools(q_start + r, n_pools);
  if (vis <= kCand) {
    if (tid == 0) t_est[r] = 0u;
    return;
  }
  const int vs = static_cast<int>((vis + (int64_t{1} << shift) - 1) >> shift);
  const int vs4 = (vs + 3) >> 2;
  const float* srow = sample + r * ld_sample;
  const int64_t target = k + k / 2;
  uint32_t rank = static_cast<uint32_t>((target * vs + vis / 2) / vis);
  rank = rank < 1u ? 1u : (rank > static_cast<uint32_t>(vs) ? static_cast<uint32_t>(vs) : rank);
  for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
  if (vs4 <= 4 * kTopkThreads) {
    // The whole sample row in registers (four float4 per thread, loaded at once).  Its
    // smallest and largest keys share their bits above bit hb; the two 10-bit digit windows
    // start right below that common prefix, so the keys spread over the histogram instead of
    // piling into the few bins of their shared exponent.
    uint32_t key[16];
    uint32_t kmax = 0u, kmin = ~0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i4 = u * kTopkThreads + tid;
      const f32x4 v = i4 < vs4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = 4 * i4 + e < vs;
        const uint32_t kk = float_order_key(v[e]);
        key[4 * u + e] = kk;
        kmax = ok && kk > kmax ? kk : kmax;
        kmin = ok && kk < kmin ? kk : kmin;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t omax = __shfl_xor(kmax, off, 64), omin = __shfl_xor(kmin, off, 64);
      kmax = omax > kmax ? omax : kmax;
      kmin = omin < kmin ? omin : kmin;
    }
    if (tid == 0) {
      pick[0] = 0u;
      pick[1] = ~0u;
    }
    __syncthreads();
    if ((tid & 63) == 0) {
      atomicMax(&pick[0], kmax);
      atomicMin(&pick[1], kmin);
    }
    __syncthreads();
    kmax = pick[0];
    kmin = pick[1];
    __syncthreads();  // pick is reused by pick_bin
    const uint32_t diff = kmax ^ kmin;
    if (diff == 0u) {  // every sample key equal
      if (tid == 0) t_est[r] = kmax;
      return;
    }
    const int hb = 31 - __builtin_clz(diff);
    const uint32_t common = kmax & ~((2u << hb) - 1u);  // bits above hb (2u << 31 == 0)
    const int sh1 = hb >= 9 ? hb - 9 : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * (u * kTopkThreads + tid) + e < vs)
          atomicAdd(&hist[(key[4 * u + e] >> sh1) & 0x3FFu], 1u);
    __syncthreads();
    uint32_t above1, in1;
    const uint32_t bin1 = pick_bin(hist, 1024, rank, wave_tmp, pick, &above1, &in1);
    const uint32_t mask1 = ~((1u << sh1) - 1u);
    const uint32_t prefix1 = (common | (bin1 << sh1)) & mask1;
    if (sh1 == 0) {
      if (tid == 0) t_est[r] = prefix1;
      return;
    }
    for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
    __syncthreads();
    const int sh2 = sh1 >= 10 ? sh1 - 10 : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * (u * kTopkThreads + tid) + e < vs && (key[4 * u + e] & mask1) == prefix1)
          atomicAdd(&hist[(key[4 * u + e] >> sh2) & 0x3FFu], 1u);
    __syncthreads();
    uint32_t above2, in2;
    const uint32_t bin2 = pick_bin(hist, 1024, rank - above1, wave_tmp, pick, &above2, &in2);
    if (tid == 0) t_est[r] = (prefix1 | (bin2 << sh2)) & ~((1u << sh2) - 1u);
    return;
  }
  __syncthreads();
  // Longer sample rows: two streamed passes over fixed windows (the top 10 key bits, then
  // the next 10).
  auto each_key = [&](auto&& f) {
    for (int base = 0; base < vs4; base += 4 * kTopkThreads) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i4 = base + u * kTopkThreads + tid;
        v[u] = i4 < vs4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i4 = base + u * kTopkThreads + tid;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * i4 + e < vs) f(float_order_key(v[u][e]));
      }
    }
  };
  each_key([&](uint32_t key) { atomicAdd(&hist[key >> 22], 1u); });
  __syncthreads();
  uint32_t above1, in1;
  const uint32_t bin1 = pick_bin(hist, 1024, rank, wave_tmp, pick, &above1, &in1);
  for (int b = tid; b < 1024; b += kTopkThreads) hist[b] = 0u;
  __syncthreads();
  each_key([&](uint32_t key) {
    if ((key >> 22) == bin1) atomicAdd(&hist[(key >> 12) & 0x3FFu], 1u);
  });
  __syncthreads();
  uint32_t above2, in2;
  const uint32_t bin2 = pick_bin(hist, 1024, rank - above1, wave_tmp, pick, &above2, &in2);
  if (tid == 0) t_est[r] = (bin1 << 22) | (bin2 << 12);
}

}  // namespace

int topk_max_k() { return kMaxK; }

int topk_cand_cap() { return kCand; }

bool topk_fused_supported(int k) { return k >= 1 && 3 * k <= 2 * kCand; }

size_t topk_workspace_bytes(int64_t, int64_t, int) { return 0; }

hipError_t launch_topk(const float* scores, int64_t ld, int64_t q_start, int64_t nq,
                       int64_t n_pools, int k, int32_t* idx, void*, size_t,
                       hipStream_t stream, const int32_t* gate) {
  if (nq <= 0) return hipSuccess;
  if (nq >= (int64_t{1} << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_kernel<false>, dim3(static_cast<unsigned>(nq)), dim3(kTopkThreads), 0,
                     stream, scores, ld, q_start, n_pools, k, idx, gate, TopkCand());
  return hipGetLastError();
}

hipError_t launch_topk_threshold(const float* sample, int64_t ld_sample, int64_t q_start,
                                 int64_t nq, int64_t n_pools, int shift, int k, uint32_t* t_est,
                                 uint32_t* cnt, int32_t* any_fail, hipStream_t stream) {
  if (nq <= 0) return hipSuccess;
  if (nq >= (int64_t{1} << 31) || ld_sample % 4 != 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(threshold_kernel, dim3(static_cast<unsigned>(nq)), dim3(kTopkThreads), 0,
                     stream, sample, ld_sample, q_start, n_pools, shift, k, t_est, cnt, any_fail);
  return hipGetLastError();
}

hipError_t launch_topk_from_cand(const TopkCand& cs, int64_t q_start, int64_t nq,
                                 int64_t n_pools, int k, int32_t* idx, hipStream_t stream) {
  if (nq <= 0) return hipSuccess;
  if (nq >= (int64_t{1} << 31) || cs.cap < kCand || !topk_fused_supported(k))
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_kernel<true>, dim3(static_cast<unsigned>(nq)), dim3(kTopkThreads), 0,
                     stream, nullptr, int64_t{0}, q_start, n_pools, k, idx, nullptr, cs);
  return hipGetLastError();
}

}  // namespace dsa
