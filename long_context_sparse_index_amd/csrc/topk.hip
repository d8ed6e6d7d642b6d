// Per-query top-k selection of pooled keys by indexer score on gfx950.
//
// Page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens", section "Model and
// bottleneck": each query keeps about 2048 pooled keys; section "Four optimizations", item 1:
// the selected pool indices are int32.  Output order: score descending, lower pool index
// first among equal scores, -1 in the slots beyond the visible count.
//
// One 1024-thread block per query row.  Scores are mapped to order-preserving 32-bit keys.
// Every path ends in one LDS list of at most 4096 (~key, pool) entries that holds the row's
// k winners; the list is sorted whole and its first k entries written:
//   * rows of at most 4096 visible pools list every visible pool;
//   * rows of up to 16384 pools are read once into registers; their smallest and largest
//     keys set the window of a 12-bit LDS histogram, a block-wide suffix scan picks the bin
//     holding the k-th largest key, and the keys in that bin or above it are listed;
//   * longer rows histogram a 1/16 sample of the row the same way, take the lower edge of
//     the bin holding the sample key ranked 1.5 k (scaled to the sample), and stream the
//     row once more, listing every score at or above that edge.
// Appends reserve their slots with one LDS atomic per wave.  The list is sorted by rank:
// entries go to 2048 buckets by a monotone map of their key, a block scan of the bucket
// counts gives each bucket's start, and each entry's position is its bucket's start plus
// the number of its bucket's entries that precede it in (~key, pool) order; a bucket of
// more than 64 entries (heavy ties) sends the list to a bitonic network in registers
// instead.  Ties therefore resolve as a stable full sort.  A row whose list does not hold
// k..4096 entries is marked in its first output slot and selected by a second, persistent
// launch with the exact two-pass select: a 12-bit histogram of the whole row picks the bin
// of the k-th largest key; the bin's keys are listed, or, when it holds more than the list,
// its remaining bits are resolved over the row by 10-bit digit histograms and a
// pool-ordered pass (block-wide prefix scans) gives the last slots to the threshold-equal
// keys of lowest pool.  A third form selects from the candidate lists of the fused
// indexer select.

#include <type_traits>

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
constexpr int kListF4 = 4;    // float4 per thread of a row read whole (list select)
constexpr int kRefineBin = 512;  // expected row keys in a sample bin that call for a second round
constexpr int kRankBuckets = 2048;    // buckets of the ranking sort of the winners
constexpr int kRankMaxBucket = 64;    // a fuller bucket (heavy ties) takes the bitonic network
constexpr int64_t kMarkedRowsGrid = 256;  // blocks of the pass over marked rows (1 per CU)

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t index) {
  return (static_cast<uint64_t>(~key) << 32) | index;  // ascending = key desc, index asc
}

// Order-preserving uint32 key of a score (larger score -> larger key, -0 as +0) in four
// VALU operations: adding +0 turns -0 into +0 and leaves every other value as it is, then
// negative values have all their bits flipped and the others their sign bit set.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

// Inclusive scan of one uint32 per lane over the wave: DPP row shifts by 1, 2, 4 and 8 within
// each row of 16 lanes (lanes without a source add 0), then the totals of the lower rows,
// read from lanes 15, 31 and 47 into scalar registers.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xF, 0xF, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xF, 0xF, false));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 15));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 31));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 47));
  const int lane = threadIdx.x & 63;
  x += lane >= 16 ? r0 : 0u;
  x += lane >= 32 ? r1 : 0u;
  x += lane >= 48 ? r2 : 0u;
  return x;
}

// Block-wide exclusive scan of one uint32 per thread; returns the exclusive prefix and
// writes the block total to *total.  All threads call it, and the block is synchronised
// again before the next call (wave_tmp is rewritten).  Each wave scans its own values; wave
// 0 then scans the wave totals (wave_tmp holds 2 * kTopkWaves + 1 words).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tmp,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) wave_tmp[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const uint32_t t = lane < kTopkWaves ? wave_tmp[lane] : 0u;
    const uint32_t ti = wave_inclusive_scan(t);
    if (lane < kTopkWaves) wave_tmp[kTopkWaves + lane] = ti - t;  // exclusive wave offsets
    if (lane == kTopkWaves - 1) wave_tmp[2 * kTopkWaves] = ti;
  }
  __syncthreads();
  *total = wave_tmp[2 * kTopkWaves];
  return wave_tmp[kTopkWaves + wid] + incl - v;
}

// Reserves for each lane cnt consecutive slots of a list whose length is the LDS counter
// *len, with one atomic per wave, and returns the lane's first slot.  Every lane of the
// wave calls it.
__device__ __forceinline__ uint32_t wave_append(uint32_t cnt, uint32_t* len) {
  const uint32_t incl = wave_inclusive_scan(cnt);
  const uint32_t total =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  uint32_t base = 0u;
  if (total != 0u && (threadIdx.x & 63) == 63) base = atomicAdd(len, total);
  base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), 63));
  return base + incl - cnt;
}

// As above, and also returns in *end the end of the wave's reservation (wave-uniform).
__device__ __forceinline__ uint32_t wave_append(uint32_t cnt, uint32_t* len, uint32_t* end) {
  const uint32_t incl = wave_inclusive_scan(cnt);
  const uint32_t total =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  uint32_t base = 0u;
  if (total != 0u && (threadIdx.x & 63) == 63) base = atomicAdd(len, total);
  base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), 63));
  *end = base + total;
  return base + incl - cnt;
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

// Wave-wide minimum and maximum of one uint32 per lane (a butterfly of VALU lane exchanges;
// every lane gets the result).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  uint32_t o;
  o = lane_xor<1>(x); x = o < x ? o : x;
  o = lane_xor<2>(x); x = o < x ? o : x;
  o = lane_xor<4>(x); x = o < x ? o : x;
  o = lane_xor<8>(x); x = o < x ? o : x;
  o = lane_xor<16>(x); x = o < x ? o : x;
  o = lane_xor<32>(x); x = o < x ? o : x;
  return x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  uint32_t o;
  o = lane_xor<1>(x); x = o > x ? o : x;
  o = lane_xor<2>(x); x = o > x ? o : x;
  o = lane_xor<4>(x); x = o > x ? o : x;
  o = lane_xor<8>(x); x = o > x ? o : x;
  o = lane_xor<16>(x); x = o > x ? o : x;
  o = lane_xor<32>(x); x = o > x ? o : x;
  return x;
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

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Picks, from a histogram of nbins bins (nbins / 1024 consecutive bins per thread, counted
// from the top), the bin holding the need-th largest key: returns it and writes the count
// of keys in higher bins and in the bin.  All threads call it; the histogram may be
// rewritten as soon as it returns.
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
  // The next call rewrites pick only after its scan's barrier, which every thread reaches
  // after these reads; any other writer of pick synchronises the block first.
  return bin;
}

// What one launch of topk_kernel does with its rows.
enum TopkMode {
  kTopkScoreRows = 0,  // score rows: the list paths, rows they cannot finish are marked
  kTopkCandLists = 1,  // candidate lists written by the candidate-emitting indexer
  kTopkMarkedRows = 2,  // the exact two-pass select on the marked rows (persistent grid)
  kTopkScoreRowsAhead = 3  // score rows of at most three listing rounds: the first round's
                           // loads go out with the sample's
};
constexpr int32_t kRowMarked = -2;  // first output slot of a row left to the two-pass select

// kTopkScoreRows: one block per row; a non-null gate skips rows whose gate is 0.  A row the
// list paths cannot finish (the sampled list out of range: heavy ties or adversarial
// layouts; k above the sampled path's limit) gets kRowMarked in its first output slot, and
// the kTopkMarkedRows launch that follows on the same stream selects it exactly.
// kTopkCandLists: the row's candidates come from a list written by the indexer (TopkCand);
// the row is flagged for the exact fallback when the list does not hold between k and
// kCand entries.
template <int MODE>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(
    MODE == kTopkMarkedRows ? 4 : 8, MODE == kTopkMarkedRows ? 4 : 8))) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t q_start, int64_t nq, int64_t n_pools,
    int k, int32_t* __restrict__ idx, const int32_t* __restrict__ gate, TopkCand cs) {
  // The first-digit histogram is dead before the candidate list is written: they share LDS.
  __shared__ uint64_t cand[kCand];  // (key << 32) | pool; the ranking sort's grouped entries
  __shared__ uint32_t hist[1024];   // 10-bit digit histograms
  __shared__ uint64_t buf[kMaxK];   // entries to sort: (~key << 32) | pool
  uint32_t* const hist0 = reinterpret_cast<uint32_t*>(cand);  // kBins0 counters
  static_assert(kBins0 * 4 <= kCand * 8, "first histogram fits the candidate list");
  __shared__ uint32_t wave_tmp[2 * kTopkWaves + 1];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t fill[3];  // slots taken in buf and in cand; sample size
  __shared__ uint32_t cand_max;  // largest key of a collected list
  __shared__ uint32_t rbin[kRankBuckets + 1];  // ranking sort: bucket counts, then starts
  __shared__ uint32_t rrange[3];  // ranking sort: smallest and largest ~key, fullest bucket
  __shared__ uint32_t rcut;  // ranking sort: end of the bucket holding the last written position
  __shared__ uint64_t marks[kTopkWaves];  // marked rows of a batch, one ballot per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  int64_t r = blockIdx.x;
  int vis = 0, n4 = 0;
  const float* srow = nullptr;
  int32_t* orow = nullptr;
  auto set_row = [&](int64_t row) {
    r = row;
    vis = static_cast<int>(visible_pools(q_start + row, n_pools));
    n4 = (vis + 3) >> 2;  // float4 groups; the row is padded to ld (a multiple of 4)
    srow = scores + row * ld;
    orow = idx + row * k;
  };

  // Exact resolution among the candidates cand[0, nc): the keys are known to hold every
  // key of the row that can still be selected above the current prefix (mask, prefix),
  // krem slots remain.  10-bit digit windows at `shift` and then shift - 10 ... 0 (a last
  // window may overlap bits already fixed); a prefix held by more candidates than slots
  // after all 32 bits is an exact tie, resolved by pool.  Winners (keys above the prefix,
  // or on it and among the lowest pools) go to buf through fill[0].
  auto resolve_candidates = [&](int nc, uint32_t prefix, uint32_t mask, int krem,
                                int shift) __attribute__((always_inline)) {
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

  // Ranking sort of the n entries of buf[0, n) (distinct composites (~key << 32) | pool)
  // into ascending order, i.e. score descending, lower pool first among equal scores.
  // nlo <= nhi span the entries' ~key: nhi bounds it from above, and entries below nlo
  // share the first bucket.  Each entry goes to one of kRankBuckets buckets by a function
  // of ~key that never decreases as ~key grows (0 below nlo, then a linear map of
  // ~key - nlo in fp32, truncated), so every entry of a lower bucket sorts before every
  // entry of a higher one; a block scan of the bucket counts gives each bucket's first
  // position, and an entry's position is its bucket's start plus the number of entries of
  // its bucket below it (exact 64-bit compares).  Scores near a selection threshold spread
  // a few entries per bucket, so this costs a few LDS reads per entry instead of a sorting
  // network's 66 compare-exchange steps.  The pools of the first min(n, k) positions are left, in
  // order, in the first words of buf.  Returns false, with buf untouched, when a bucket
  // holds more than kRankMaxBucket entries (heavy ties).  rbin and rrange[2] are zero on
  // entry; cand is free.
  auto rank_sort = [&](int n, uint32_t nlo, uint32_t nhi, bool raw) __attribute__((always_inline)) -> bool {
    constexpr int kR = kMaxK / kTopkThreads;
    uint32_t* const out32 = reinterpret_cast<uint32_t*>(buf);
    uint64_t* const grp = cand;
    const float inv = nhi > nlo ? static_cast<float>(kRankBuckets - 1) /
                                      static_cast<float>(nhi - nlo)
                                : 0.f;
    auto bucket = [&](uint64_t x) {
      const uint32_t nk = static_cast<uint32_t>(x >> 32);
      const uint32_t b =
          nk > nlo ? static_cast<uint32_t>(static_cast<float>(nk - nlo) * inv) : 0u;
      return b < static_cast<uint32_t>(kRankBuckets - 1) ? b
                                                         : static_cast<uint32_t>(kRankBuckets - 1);
    };
    const int nr = (n + kTopkThreads - 1) / kTopkThreads;  // uniform
    uint32_t ds[kR];  // bucket << 16 | slot in the bucket
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int i = tid + j * kTopkThreads;
      ds[j] = 0u;
      if (j < nr && i < n) {
        uint64_t x = buf[i];
        if (raw) {  // (score bits << 32) | pool -> composite, written back
          x = composite(score_key(__uint_as_float(static_cast<uint32_t>(x >> 32))),
                        static_cast<uint32_t>(x));
          buf[i] = x;
        }
        const uint32_t d = bucket(x);
        ds[j] = (d << 16) | atomicAdd(&rbin[d], 1u);
      }
    }
    __syncthreads();
    // Bucket starts: two buckets per thread, one block scan; the fullest bucket's count.
    static_assert(kRankBuckets == 2 * kTopkThreads, "two buckets per thread");
    const uint32_t c0 = rbin[2 * tid], c1 = rbin[2 * tid + 1];
    const uint32_t cmax = wave_max_u32(c0 > c1 ? c0 : c1);
    if (lane == 0) atomicMax(&rrange[2], cmax);
    uint32_t total;
    const uint32_t start = block_exclusive_scan(c0 + c1, wave_tmp, &total);
    rbin[2 * tid] = start;
    rbin[2 * tid + 1] = start + c0;
    if (tid == 0) rbin[kRankBuckets] = static_cast<uint32_t>(n);
    // Only the first n_out positions are written out: entries of buckets that start at or
    // past n_out are neither grouped nor ranked, and the grouped positions below `cut`, the
    // end of the bucket holding position n_out - 1, are the ones ranked.
    const uint32_t n_out = static_cast<uint32_t>(n < k ? n : k);
    if (start < n_out && start + c0 >= n_out) rcut = start + c0;
    if (start + c0 < n_out && start + c0 + c1 >= n_out) rcut = start + c0 + c1;
    __syncthreads();
    if (rrange[2] > static_cast<uint32_t>(kRankMaxBucket)) return false;  // uniform
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int i = tid + j * kTopkThreads;
      if (j < nr && i < n) {
        const uint32_t st = rbin[ds[j] >> 16];
        if (st < n_out) grp[st + (ds[j] & 0xFFFFu)] = buf[i];
      }
    }
    const int cut = static_cast<int>(rcut);
    __syncthreads();
    // Rank within the bucket; consecutive threads take consecutive grouped entries, so the
    // lanes of a wave mostly scan the same bucket (broadcast LDS reads, even loop counts).
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int p = tid + j * kTopkThreads;
      if (j < nr && p < cut) {
        const uint64_t x = grp[p];
        const uint32_t d = bucket(x);
        const uint32_t s = rbin[d], c = rbin[d + 1] - s;
        uint32_t rk = 0u;
        for (uint32_t q = 0; q < c; ++q) rk += grp[s + q] < x ? 1u : 0u;
        out32[s + rk] = static_cast<uint32_t>(x);
      }
    }
    __syncthreads();
    return true;
  };

  // Writes the first min(k, n) of the n entries of buf[0, n) (n <= kMaxK) to the output row
  // in sorted order, -1 in the slots past n.  nlo <= nhi span the entries' ~key (as in the
  // ranking sort), or nlo > nhi to have them found here.  The ranking sort, or for heavy
  // ties the bitonic network over buf padded with ~0 to a power of two.  All threads call
  // it after writing buf.
  auto sort_and_store = [&](int n, uint32_t nlo, uint32_t nhi, bool raw = false)
                            __attribute__((always_inline)) {
    if (n == 0) {
      for (int i = tid; i < k; i += kTopkThreads) orow[i] = -1;
      return;
    }
    const bool find = nlo > nhi;
    for (int b = tid; b <= kRankBuckets; b += kTopkThreads) rbin[b] = 0u;
    if (tid == 0) {
      rrange[2] = 0u;
      if (find) {
        rrange[0] = ~0u;
        rrange[1] = 0u;
      }
    }
    __syncthreads();  // buf written; rbin and rrange initialised
    if (find) {
      uint32_t lo = ~0u, hi = 0u;
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t nk = static_cast<uint32_t>(buf[i] >> 32);
        lo = nk < lo ? nk : lo;
        hi = nk > hi ? nk : hi;
      }
      lo = wave_min_u32(lo);
      hi = wave_max_u32(hi);
      if (lane == 0 && lo <= hi) {
        atomicMin(&rrange[0], lo);
        atomicMax(&rrange[1], hi);
      }
      __syncthreads();
      nlo = rrange[0];
      nhi = rrange[1];
    }
    if (rank_sort(n, nlo, nhi, raw)) {
      const uint32_t* out32 = reinterpret_cast<const uint32_t*>(buf);
      for (int i = tid; i < k; i += kTopkThreads)
        orow[i] = i < n ? static_cast<int32_t>(out32[i]) : -1;
      return;
    }
    const int n2 = max(next_pow2(n), kTopkThreads);
    for (int i = n + tid; i < n2; i += kTopkThreads) buf[i] = ~0ull;
    __syncthreads();
    sort_keys(buf, cand, n2);
    for (int i = tid; i < k; i += kTopkThreads)
      orow[i] = i < n ? static_cast<int32_t>(buf[i] & 0xFFFFFFFFu) : -1;
  };

  if constexpr (MODE == kTopkCandLists) {
    set_row(blockIdx.x);
    // The list holds every visible entry whose key is >= the row's threshold (all visible
    // entries when the threshold is 0).  With at least k (or all vis <= k) and at most kCand
    // of them it holds the k winners: the whole list is sorted and its first k written.  Any
    // other count leaves the row to the fallback (indexer scores + the score-row select).
    // Every list has room for kCand entries: all of it is requested before the count
    // arrives (entries past the count are ignored), so the loads take one round trip.
    static_assert(kCand == 4 * kTopkThreads, "four list entries per thread");
    const uint64_t* crow = cs.cand + r * cs.cap;
    uint64_t pre[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pre[u] = crow[u * kTopkThreads + tid];
    const uint32_t n = cs.cnt[r];
    const uint32_t t_est = cs.t_est[r];
    const bool usable = vis <= k ? n == static_cast<uint32_t>(vis)
                                 : (n >= static_cast<uint32_t>(k) &&
                                    n <= static_cast<uint32_t>(kCand));
    if (tid == 0) {
      cs.fail[r] = usable ? 0 : 1;
      if (!usable) atomicOr(cs.any_fail, 1);
      cand_max = 0u;
    }
    if (!usable) return;
    __syncthreads();  // cand_max cleared
    uint32_t my_max = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = u * kTopkThreads + tid;
      if (i < static_cast<int>(n)) {
        const uint32_t key = static_cast<uint32_t>(pre[u] >> 32);
        buf[i] = composite(key, static_cast<uint32_t>(pre[u]));
        my_max = key > my_max ? key : my_max;
      }
    }
    my_max = wave_max_u32(my_max);
    if (lane == 0 && my_max) atomicMax(&cand_max, my_max);
    __syncthreads();
    // Keys lie in [t_est, cand_max]; a zero threshold gives no useful bound.
    if (t_est == 0u)
      sort_and_store(static_cast<int>(n), 1u, 0u);
    else
      sort_and_store(static_cast<int>(n), ~cand_max, ~t_est);
    return;
  }

  // Calls f(i4, v) for every float4 group of the row, kLoads loads in flight per thread.
  // Groups past the row end carry keys with index >= vis, which f must skip.
  auto stream_row_with = [&](auto loads, auto&& f) {
    constexpr int kNL = decltype(loads)::value;
    for (int base = 0; base < n4; base += kNL * kTopkThreads) {
      f32x4 v[kNL];
#pragma unroll
      for (int u = 0; u < kNL; ++u) {
        const int i4 = base + u * kTopkThreads + tid;
        v[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kNL; ++u) f(base + u * kTopkThreads + tid, v[u]);
    }
  };
  auto stream_row = [&](auto&& f) {
    stream_row_with(std::integral_constant<int, kLoads>(), f);
  };

  // Rows longer than kCand.  Rows of up to kListVis pools are read whole into registers
  // (kListF4 float4 per thread); longer rows read a 1/16 sample (256-byte pieces, one every
  // 4 KB of the row, or sparser past 2^18 keys: at most 256 pieces, four per group of 16
  // threads).  A 12-bit histogram of those keys, its window starting at the highest bit
  // where their smallest and largest keys differ (so they spread over the bins instead of
  // piling into the few bins of a shared exponent), picks the bin holding the k-th largest
  // key of a whole row, or for a sample the key ranked 1.5 k scaled to the sample.  A whole
  // row then lists, from registers, every key in that bin or above it (k plus the bin's
  // few keys); a sampled row is streamed once more and every key at or above the bin's
  // lower edge listed (about 1.5 k).  The list (at most kMaxK entries, and at least k for a
  // sampled row) holds the k winners and is sorted whole, its first k written.  Any other
  // list size (heavy ties, layouts that fool the sample) returns false.
  auto list_select = [&](auto whole_c) __attribute__((always_inline)) -> bool {
    constexpr bool kWhole = decltype(whole_c)::value;
    const int piece_stride = 256 * ((n4 + 65535) / 65536);
    // Rounds of groups held: a whole row nu rounds of 1024 float4, a sample nu rounds of 64
    // pieces.  Slots past the row hold key 0, below the key of every score.
    int nu = 0;
    if constexpr (kWhole) {
      nu = (n4 + kTopkThreads - 1) / kTopkThreads;
    } else {
      while (nu < kListF4 && piece_stride * 64 * nu < n4) ++nu;
    }
    auto index4 = [&](int u) {  // float4 group of round u
      if constexpr (kWhole) return u * kTopkThreads + tid;
      else return piece_stride * ((tid >> 4) + 64 * u) + (tid & 15);
    };
    // Groups past the row are read at the row's last group (the values are not used), so
    // the loads need no branch.
    f32x4 x[kListF4];
#pragma unroll
    for (int u = 0; u < kListF4; ++u)
      if (u < nu)  // uniform
        x[u] = *reinterpret_cast<const f32x4*>(srow + 4 * min(index4(u), n4 - 1));
    // Launches whose sampled rows take at most three listing rounds load the first round
    // here, so that its latency hides behind the threshold work, and keep the next round's
    // loads in flight while one round is listed (62 instead of 42 VGPRs, still eight waves
    // per SIMD; 4-9% faster on such launches).  Longer rows keep the plain kernel, which
    // measured 1-2% faster there.
    constexpr bool kAhead = MODE == kTopkScoreRowsAhead && !kWhole;
    f32x4 ahead[kListF4];  // the listing round loaded ahead
    if constexpr (kAhead) {
#pragma unroll
      for (int u = 0; u < kListF4; ++u) {
        const int i4 = u * kTopkThreads + tid;
        ahead[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    for (int b = tid; b < kBins0; b += kTopkThreads) hist0[b] = 0u;
    if (tid == 0) {
      fill[0] = 0u;
      fill[1] = 0u;
      fill[2] = 0u;
      cand_max = 0u;
      rrange[0] = ~0u;
      rrange[1] = 0u;
    }
    uint32_t key[4 * kListF4];
    uint32_t lo1 = ~0u, hi = 0u, n_local = 0u;  // lo1: smallest key - 1 (key 0 is neutral)
#pragma unroll
    for (int u = 0; u < kListF4; ++u) {
      if (u < nu) {  // uniform
        const int nv = min(max(vis - 4 * index4(u), 0), 4);
        n_local += static_cast<uint32_t>(nv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          key[4 * u + e] = e < nv ? score_key(x[u][e]) : 0u;
          lo1 = min(lo1, key[4 * u + e] - 1u);
          hi = max(hi, key[4 * u + e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * u + e] = 0u;
      }
    }
    lo1 = wave_min_u32(lo1);
    hi = wave_max_u32(hi);
    __syncthreads();  // histogram, counters and range cleared
    if (lane == 0) {
      atomicMin(&rrange[0], lo1);
      atomicMax(&rrange[1], hi);
    }
    if (!kWhole && n_local) atomicAdd(&fill[2], n_local);
    __syncthreads();
    const uint32_t klo = rrange[0] + 1u, khi = rrange[1];
    const uint32_t n_keys = kWhole ? static_cast<uint32_t>(vis) : fill[2];
    const uint32_t diff = klo ^ khi;
    const int hb = diff != 0u ? 31 - __builtin_clz(diff) : 0;
    const int shift = hb >= 11 ? hb - 11 : 0;
#pragma unroll
    for (int u = 0; u < kListF4; ++u)
      if (u < nu)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key[4 * u + e] != 0u) atomicAdd(&hist0[(key[4 * u + e] >> shift) & 0xFFFu], 1u);
    __syncthreads();
    uint32_t rank = static_cast<uint32_t>(k);
    if constexpr (!kWhole) {  // 1.5 k scaled to the sample (an estimate: fp32 will do)
      rank = static_cast<uint32_t>(static_cast<float>(k + k / 2) * static_cast<float>(n_keys) /
                                       static_cast<float>(vis) +
                                   0.5f);
      rank = rank < 1u ? 1u : (rank > n_keys ? n_keys : rank);
    }
    uint32_t above0, in0;
    const uint32_t b0 = pick_bin(hist0, kBins0, rank, wave_tmp, pick, &above0, &in0);
    // Lower edge of bin b0: the bits above the window as in the largest key, the window b0.
    uint32_t lower = (khi & ~((0x1000u << shift) - 1u)) | (b0 << shift);
    if constexpr (kWhole) {
      const uint32_t n = above0 + in0;
      if (n > static_cast<uint32_t>(kMaxK)) return false;  // uniform
      // Key 0 (no score) never reaches a bin edge.
      uint32_t cnt = 0u;
#pragma unroll
      for (int u = 0; u < kListF4; ++u)
        if (u < nu)
#pragma unroll
          for (int e = 0; e < 4; ++e) cnt += key[4 * u + e] >= lower ? 1u : 0u;
      uint32_t slot = wave_append(cnt, &fill[0]);
#pragma unroll
      for (int u = 0; u < kListF4; ++u)
        if (u < nu)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key[4 * u + e] >= lower) {
              if (slot < static_cast<uint32_t>(kMaxK))
                buf[slot] = composite(key[4 * u + e], static_cast<uint32_t>(4 * index4(u) + e));
              ++slot;
            }
      sort_and_store(static_cast<int>(n), ~khi, ~lower);
      return true;
    } else {
      // A sample bin expected to hold many of the row's keys (a window spanning several
      // exponents): a second 12-bit round over the sample keys inside it.
      if (shift > 0 && static_cast<uint64_t>(in0) * static_cast<uint64_t>(vis) >
                           static_cast<uint64_t>(kRefineBin) * n_keys) {
        const int shift2 = shift >= 12 ? shift - 12 : 0;
        const uint32_t fixed = ~((1u << shift) - 1u);
        for (int b = tid; b < kBins0; b += kTopkThreads) hist0[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kListF4; ++u)
          if (u < nu)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if ((key[4 * u + e] & fixed) == lower)
                atomicAdd(&hist0[(key[4 * u + e] >> shift2) & 0xFFFu], 1u);
        __syncthreads();
        uint32_t above1, in1;
        const uint32_t b1 = pick_bin(hist0, kBins0, rank - above0, wave_tmp, pick, &above1, &in1);
        lower = (lower & ~(0xFFFu << shift2)) | (b1 << shift2);
      }
      // One pass over the row: every score whose key is at or above lower is listed as
      // (score bits << 32) | pool, kListF4 float4 per thread in flight, one list reservation
      // per wave and pass.  Scores are compared as floats against the smallest float of key
      // lower (-inf when lower is below the key of -inf).  A wave whose groups of a round all
      // lie inside the row (every round but the one holding the row's end) skips the
      // per-element visibility test, and a wave whose reservation ends past the list's
      // capacity stores nothing (the row then fails the size test below).
      const float f_lower =
          lower <= 0x007FFFFFu ? -__builtin_inff()
                               : __uint_as_float((lower & 0x80000000u) ? lower ^ 0x80000000u : ~lower);
      const int wfirst = __builtin_amdgcn_readfirstlane(tid & ~63);
      uint32_t* const buf32 = reinterpret_cast<uint32_t*>(buf);
      for (int base = 0; base < n4; base += kListF4 * kTopkThreads) {
        f32x4 v[kListF4];
        if constexpr (kAhead) {
#pragma unroll
          for (int u = 0; u < kListF4; ++u) v[u] = ahead[u];
          if (base + kListF4 * kTopkThreads < n4) {  // uniform: the next round's loads
#pragma unroll
            for (int u = 0; u < kListF4; ++u) {
              const int i4 = base + (kListF4 + u) * kTopkThreads + tid;
              ahead[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < kListF4; ++u) {
            const int i4 = base + u * kTopkThreads + tid;
            v[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(srow + 4 * i4)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        // Visible elements of this lane's group in round u (4 when the wave's round is whole).
        auto n_visible = [&](int u) {
          return min(max(vis - 4 * (base + u * kTopkThreads + tid), 0), 4);
        };
        auto whole = [&](int u) { return 4 * (base + u * kTopkThreads + wfirst + 64) <= vis; };
        auto present = [&](int u) { return base + u * kTopkThreads + wfirst < n4; };
        uint32_t cnt = 0u;
#pragma unroll
        for (int u = 0; u < kListF4; ++u) {
          if (!present(u)) continue;  // uniform
          if (whole(u)) {             // uniform
#pragma unroll
            for (int e = 0; e < 4; ++e) cnt += v[u][e] >= f_lower ? 1u : 0u;
          } else {
            const int nv = n_visible(u);
#pragma unroll
            for (int e = 0; e < 4; ++e) cnt += e < nv && v[u][e] >= f_lower ? 1u : 0u;
          }
        }
        uint32_t end;
        const uint32_t slot = wave_append(cnt, &fill[1], &end);
        if (end > static_cast<uint32_t>(kCand)) continue;  // uniform
        uint32_t* a = buf32 + 2u * slot;  // the lane's next entry: pool, then score bits
        auto put = [&](uint32_t pool, float x) {
          a[0] = pool;
          a[1] = __float_as_uint(x);
          a += 2;
        };
#pragma unroll
        for (int u = 0; u < kListF4; ++u) {
          if (!present(u)) continue;
          const uint32_t i0 = static_cast<uint32_t>(4 * (base + u * kTopkThreads + tid));
          if (whole(u)) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (v[u][e] >= f_lower) put(i0 + e, v[u][e]);
          } else {
            const int nv = n_visible(u);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (e < nv && v[u][e] >= f_lower) put(i0 + e, v[u][e]);
          }
        }
      }
      __syncthreads();
      const uint32_t n_cand = fill[1];
      if (n_cand < static_cast<uint32_t>(k) || n_cand > static_cast<uint32_t>(kCand))
        return false;
      // The listed keys are at least lower; the sample's largest key bounds all but a few
      // of them from above (the ranking sort puts any larger key in its first bucket).  The
      // entries hold raw scores.
      sort_and_store(static_cast<int>(n_cand), ~khi, ~lower, true);
      return true;
    }
  };

  // The exact two-pass select; the k winners end in buf.
  auto two_pass_select = [&]() __attribute__((always_inline)) {
    // Pass A: the top 12 bits of every visible key.
    for (int b = tid; b < kBins0; b += kTopkThreads) hist0[b] = 0u;
    if (tid < 2) fill[tid] = 0u;
    __syncthreads();
    stream_row([&](int i4, const f32x4& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * i4 + e < vis) atomicAdd(&hist0[score_key(v[e]) >> 20], 1u);
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
          const uint32_t key = score_key(v[e]);
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
            const uint32_t key = score_key(v[e]);
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
          const uint32_t mk = score_key(cur[e >> 2][e & 3]) & mask;
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
        __syncthreads();  // wave_tmp is rewritten by the next group's scan
        if (flags != 0u) {
          uint32_t pos_gt = run_gt + (pre & 0xFFFFu);
          uint32_t rank_eq = run_eq + (pre >> 16);
#pragma unroll
          for (int e = 0; e < 4 * kU; ++e) {
            const uint32_t i = static_cast<uint32_t>(4 * (base4 + kU * tid) + e);
            const uint32_t key = score_key(cur[e >> 2][e & 3]);
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
  };

  if constexpr (MODE == kTopkScoreRows || MODE == kTopkScoreRowsAhead) {
    if (gate && gate[blockIdx.x] == 0) return;
    set_row(blockIdx.x);
    if (vis <= kCand) {
      // Every visible key fits the list (rows with at most k visible pools included): the
      // row is sorted whole and its first k entries written.
      for (int i = tid; i < vis; i += kTopkThreads)
        buf[i] = composite(score_key(srow[i]), static_cast<uint32_t>(i));
      sort_and_store(vis, 1u, 0u);
      return;
    }
    if (3 * k <= 2 * kCand) {
      const bool done = n4 <= kListF4 * kTopkThreads ? list_select(std::true_type())
                                                     : list_select(std::false_type());
      if (done) return;
    }
    if (tid == 0) orow[0] = kRowMarked;
  } else if constexpr (MODE == kTopkMarkedRows) {
    // Block b looks at rows b, b + G, b + 2 G, ... (G blocks), 1024 of them per batch: one
    // load of each row's first slot, the marked ones collected as wave ballots, then each
    // selected in turn by the whole block.
    const int64_t g = gridDim.x;
    for (int64_t base = blockIdx.x; base < nq; base += g * kTopkThreads) {
      const int64_t row = base + static_cast<int64_t>(tid) * g;
      const bool marked =
          row < nq && (gate == nullptr || gate[row] != 0) && idx[row * k] == kRowMarked;
      const uint64_t m = __ballot(marked);
      if (lane == 0) marks[tid >> 6] = m;
      __syncthreads();
      for (int w = 0; w < kTopkWaves; ++w) {
        uint64_t mm = marks[w];
        while (mm != 0ull) {  // uniform
          const int b = __builtin_ctzll(mm);
          mm &= mm - 1ull;
          set_row(base + static_cast<int64_t>(w * 64 + b) * g);
          two_pass_select();
          sort_and_store(k, 1u, 0u);
        }
      }
      __syncthreads();  // marks is rewritten by the next batch
    }
  }
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
        const uint32_t kk = score_key(v[e]);
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
          if (4 * i4 + e < vs) f(score_key(v[u][e]));
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
  // Rows of more than one register load per thread take the sampled path, whose listing
  // streams kListF4 float4 per thread per round.
  constexpr int64_t kRoundPools = 4 * kListF4 * kTopkThreads;
  const int64_t vis_max = (q_start + nq) / 4 < n_pools ? (q_start + nq) / 4 : n_pools;
  if (vis_max > kRoundPools && vis_max <= 3 * kRoundPools)
    hipLaunchKernelGGL(topk_kernel<kTopkScoreRowsAhead>, dim3(static_cast<unsigned>(nq)),
                       dim3(kTopkThreads), 0, stream, scores, ld, q_start, nq, n_pools, k, idx,
                       gate, TopkCand());
  else
    hipLaunchKernelGGL(topk_kernel<kTopkScoreRows>, dim3(static_cast<unsigned>(nq)),
                       dim3(kTopkThreads), 0, stream, scores, ld, q_start, nq, n_pools, k, idx,
                       gate, TopkCand());
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Rows marked by the launch above (rare), one block per compute unit of the chip.
  const int64_t grid = nq < kMarkedRowsGrid ? nq : kMarkedRowsGrid;
  hipLaunchKernelGGL(topk_kernel<kTopkMarkedRows>, dim3(static_cast<unsigned>(grid)),
                     dim3(kTopkThreads), 0, stream, scores, ld, q_start, nq, n_pools, k, idx,
                     gate, TopkCand());
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
  hipLaunchKernelGGL(topk_kernel<kTopkCandLists>, dim3(static_cast<unsigned>(nq)),
                     dim3(kTopkThreads), 0, stream, nullptr, int64_t{0}, q_start, nq, n_pools, k,
                     idx, nullptr, cs);
  return hipGetLastError();
}

}  // namespace dsa
