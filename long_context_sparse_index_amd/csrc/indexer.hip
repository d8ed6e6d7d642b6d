// Lightning-indexer scores on gfx950 MFMA.
//
// Page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens", section "Model and
// bottleneck": every query scores every visible pooled key (one pool per 4 tokens), which is
// the quadratic part of the layer.  Score I[t,s] = sum_j w[t,j] * max(0, q[t,j,:] . k[s,:]).
//
// Tiling.  A block owns a tile of BQ queries x 256 pools; each of its 4 waves owns 64 pools
// and keeps their key rows in registers as MFMA A operands for the whole head loop, since
// the pooled key is shared by all indexer heads.  The queries of one head are gathered into
// LDS by asynchronous global->LDS loads issued three heads ahead (four stages, one barrier
// per head), so their memory latency hides behind three heads of MFMA work, and read by all
// waves as B operands.  Each head's
// 16x16 products are ReLU'd and added with the head weight into fp32 score registers, so
// the per-head products never leave the register file.  Products are laid out
// pool-major (MFMA rows = pools, columns = queries), which puts one query per lane column:
// the head weight is one value per lane and the finished scores go out as 16-byte rows.
// With few heads a block keeps its key rows for several consecutive query tiles, the
// staging running on from one tile's last head to the next tile's first.
//
// The grid covers the causal trapezoid: tiles whose first pool lies beyond the visible
// prefix of the tile's last query exit at once.  Block ids are remapped so that the pool
// tiles of one query tile (or group of tiles) run on the same XCD (blocks are dealt to the
// 8 XCDs round-robin) and share the queries through that XCD's L2.

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kIdxWaves = 4;
constexpr int kIdxThreads = kIdxWaves * kWave;
constexpr int kPoolsPerWave = 64;
constexpr int kMB = kPoolsPerWave / 16;
constexpr int kPoolsPerBlock = kIdxWaves * kPoolsPerWave;
constexpr int kMaxHeads = 64;
// Few-head score launches (at most kMaxGroupHeads heads): (query tile, head) passes per
// block's key-row load at most, and the grid size below which blocks take fewer query tiles.
constexpr int kMaxGroupHeads = 16;
constexpr int kPassesPerKeyLoad = 256;
constexpr int kMinBlocks = 2048;

template <bool FP8>
struct FragT;
template <>
struct FragT<false> {
  using type = bf16x8;
};
template <>
struct FragT<true> {
  using type = i32x8;
};

template <bool FP8>
__device__ __forceinline__ typename FragT<FP8>::type load_frag(const uint8_t* p) {
  if constexpr (FP8) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  } else {
    return *reinterpret_cast<const bf16x8*>(p);
  }
}

template <bool FP8>
__device__ __forceinline__ typename FragT<FP8>::type zero_frag() {
  typename FragT<FP8>::type z;
  if constexpr (FP8) {
    for (int i = 0; i < 8; ++i) z[i] = 0;
  } else {
    z = bf16x8_zero();
  }
  return z;
}

template <bool FP8>
__device__ __forceinline__ f32x4 mfma_frag(typename FragT<FP8>::type a,
                                           typename FragT<FP8>::type b, f32x4 c) {
  if constexpr (FP8)
    return mfma16x16x128_e4m3(a, b, c);
  else
    return mfma16x16x32_bf16(a, b, c);
}

// max(x, 0) as one integer max on the bit pattern: an IEEE float with the sign bit set is
// a negative int32 (-0 included) and becomes +0.  A float max would first spend an
// instruction quieting signalling NaNs.
__device__ __forceinline__ float relu_bits(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// One asynchronous 16-byte-per-lane global -> LDS load (lane l's 16 bytes land at LDS byte
// address lds_addr + 16 l).  Written as inline assembly so that the compiler does not drain
// every outstanding load before the next LDS read; the head loop waits for exactly the
// loads it needs.
__device__ __forceinline__ void idx_dma_16b(const void* src, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr) : "memory");
}

// Waits until at most `n` vector-memory operations of this wave are outstanding (n < 64).
#define IDX_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

// D: d_i; NB: 16-query column blocks per tile (BQ = 16 * NB); FP8: e4m3 operands; EMIT:
// instead of storing scores, append the (key, pool) pairs whose order key reaches the row's
// threshold to the row's candidate list (IndexerOpts); MULTI: a block takes group_tiles
// consecutive query tiles (else one).
template <int D, int NB, bool FP8, bool EMIT, bool MULTI>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(
    const uint8_t* __restrict__ q, int64_t q_stride_b, const uint8_t* __restrict__ k,
    int64_t k_stride_b, const float* __restrict__ w, int64_t w_stride,
    float* __restrict__ scores, int64_t ld, int64_t q_start, int64_t nq, int64_t n_pools,
    int h_i, int accumulate, int n_pool_tiles, int n_query_groups, int group_tiles,
    IndexerOpts opt) {
  using Frag = typename FragT<FP8>::type;
  constexpr int kRowBytes = D * (FP8 ? 1 : 2);
  constexpr int kFragBytes = FP8 ? 32 : 16;        // bytes of one row per lane group
  constexpr int kStepBytes = 4 * kFragBytes;       // bytes of one row per MFMA
  constexpr int kKS = kRowBytes / kStepBytes;      // MFMAs per head per tile
  constexpr int kBQ = 16 * NB;
  constexpr int kCpr = kRowBytes / 16;             // 16-byte chunks per query row
  constexpr int kHeadBytes = kBQ * kRowBytes;      // one head's query tile in LDS
  constexpr int kDmaPerHead = kHeadBytes / 1024;   // 1 KB global->LDS loads per head
  // Loads are dealt to the waves round-robin; a wave issues at most kDmaPerWave per head.
  constexpr int kDmaPerWave = (kDmaPerHead + kIdxWaves - 1) / kIdxWaves;
  constexpr int kStages = 4;                       // heads staged ahead
  static_assert(kRowBytes % kStepBytes == 0, "d_i must fill whole MFMA steps");
  static_assert(kHeadBytes % 1024 == 0, "query tile of whole 1 KB loads");
  // Every wave that issues loads issues exactly kDmaPerWave per head (the waits count them).
  static_assert(kDmaPerHead % kIdxWaves == 0 || kDmaPerHead < kIdxWaves, "even split");
  static_assert(kDmaPerWave * (kStages - 1) < 64, "vmcnt range");

  // Query tile of a head in LDS: row r, chunk c at chunk position c ^ swz(r), so that the 16
  // rows read by one lane group at the same chunk hit 16 different 16-byte bank groups
  // (rows are not padded: the global->LDS loads fill 1 KB contiguously).
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kStages * kHeadBytes];
  __shared__ float w_lds[kBQ * (MULTI ? kPassesPerKeyLoad : kMaxHeads)];
  auto swz = [](int r) {
    if constexpr (kCpr >= 16) return r & 15;
    else return (r / (16 / kCpr)) & (kCpr - 1);
  };

  if (opt.gate && *opt.gate == 0) return;  // gated launch with nothing to do
  static_assert(!(EMIT && MULTI), "the candidate pass takes one query tile per block");
  // With pool_shift s the key table is read at every 2^s-th pool (the caller scales the key
  // stride): column c is pool c * 2^s, visible to t iff c * 2^s < V(t).
  const int sh = opt.pool_shift;
  auto vis_of = [&](int64_t t) {
    return (visible_pools(t, n_pools) + (int64_t{1} << sh) - 1) >> sh;
  };
  const int64_t n_cols = (n_pools + (int64_t{1} << sh) - 1) >> sh;
  // XCD-aware remap: consecutive logical tiles (same query group) land on one XCD.
  const int n_tiles = n_pool_tiles * n_query_groups;
  const int per_xcd = (n_tiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= n_tiles) return;
  const int qg = logical / n_pool_tiles;
  const int pt = logical - qg * n_pool_tiles;
  const int64_t p0 = static_cast<int64_t>(pt) * kPoolsPerBlock;
  // The block's query tiles [qt_first, qt_first + n_qt): tile qg alone, or (MULTI) the
  // tiles of group qg that see some of the block's pools.  Visible prefixes grow with the
  // query, so the tiles that see none come first and are skipped.
  auto vis_last_of = [&](int64_t qt) {  // visible columns of the tile's last row
    const int64_t last = (qt + 1) * kBQ < nq ? (qt + 1) * kBQ - 1 : nq - 1;
    return vis_of(q_start + last);
  };
  int64_t qt_first = qg;
  int n_qt = 1;
  if constexpr (MULTI) {
    const int64_t n_query_tiles = (nq + kBQ - 1) / kBQ;
    const int64_t qt_end = (static_cast<int64_t>(qg) + 1) * group_tiles < n_query_tiles
                               ? (static_cast<int64_t>(qg) + 1) * group_tiles
                               : n_query_tiles;
    if (p0 >= vis_last_of(qt_end - 1)) return;  // every tile above the causal boundary
    qt_first = static_cast<int64_t>(qg) * group_tiles;
    while (p0 >= vis_last_of(qt_first)) ++qt_first;  // stops at qt_end - 1 at the latest
    n_qt = static_cast<int>(qt_end - qt_first);
  }
  // Visible columns of the block's last row.
  const int64_t vis_last = vis_last_of(qt_first + n_qt - 1);
  if constexpr (!MULTI) {
    if (p0 >= vis_last) return;  // whole tile above the causal boundary
  }
  const int n_pass = n_qt * h_i;  // (query tile, head) passes, head-minor

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t pw0 = p0 + wid * kPoolsPerWave;
  // The wave's pools are visible to some row of the block (its last row).
  const bool keys_live = pw0 < vis_last;

  if (opt.gate_rows) {
    // Only query tiles holding a flagged row (one tile per block here): wave 0 checks the
    // tile's rows (kBQ <= 64) and passes the verdict through the weight array's first word
    // before the weights land.
    static_assert(kBQ <= kWave, "one wave checks the tile");
    const int64_t q0 = qt_first * kBQ;
    uint32_t* const verdict = reinterpret_cast<uint32_t*>(w_lds);
    if (tid < kWave) {
      const bool flagged = tid < kBQ && q0 + tid < nq && opt.gate_rows[q0 + tid] != 0;
      const uint64_t b = __ballot(flagged);
      if (tid == 0) *verdict = b != 0 ? 1u : 0u;
    }
    __syncthreads();
    const bool any_row = *verdict != 0u;
    __syncthreads();  // the weights overwrite the verdict next
    if (!any_row) return;
  }

  // Head weights of the block's queries, pass-major ([tile][head][query]) so that the 16
  // lanes of a group read 16 consecutive words; consecutive threads write consecutive words
  // (walking the rows of one head first avoids 32-way bank conflicts on the transposing
  // stores).  The host keeps n_qt * h_i <= kPassesPerKeyLoad (MULTI) or h_i <= kMaxHeads.
  for (int i = tid; i < n_pass * kBQ; i += kIdxThreads) {
    const int jj = i / kBQ;
    const int row = i - jj * kBQ;
    const int qi = MULTI ? jj / h_i : 0;
    const int j = jj - qi * h_i;
    const int64_t t = (qt_first + qi) * kBQ + row;
    w_lds[i] = t < nq ? w[t * w_stride + j] : 0.0f;
  }
  // Candidate counters of the tile's rows: past the weights when they leave room, zeroed
  // here (the head loop's barriers order this before the epilogue's LDS atomics), else on
  // the weights once the last head has read them.
  const bool counters_apart = h_i <= kMaxHeads - 2;
  if constexpr (EMIT) {
    if (counters_apart && tid < kBQ) reinterpret_cast<uint32_t*>(w_lds)[h_i * kBQ + tid] = 0u;
  }

  // This wave's pooled key rows, resident for all of the block's passes.
  Frag kf[kMB][kKS];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int64_t pool = pw0 + mb * 16 + r16;
    const bool ok = keys_live && pool < n_cols;
    const uint8_t* kp = k + (ok ? pool : 0) * k_stride_b + g * kFragBytes;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      kf[mb][ks] = ok ? load_frag<FP8>(kp + ks * kStepBytes) : zero_frag<FP8>();
  }

  // This lane's share of a pass's query-tile loads: the wave's load i is the pass's 1 KB load
  // L = wid + 4 i (if L < kDmaPerHead); lane slot s = 64 L + lane -> row s / kCpr, position
  // s % kCpr.
  // One tile: the loads' source rows are fixed, so their addresses are formed once.
  auto dma_row = [&](int i) {  // loads past the tile (not issued) stay in range
    return ((64 * (wid + kIdxWaves * i) + lane) / kCpr) % kBQ;
  };
  auto dma_chunk = [&](int i) {
    return ((64 * (wid + kIdxWaves * i) + lane) % kCpr) ^ swz(dma_row(i));
  };
  // Several tiles: with a short row stride, a whole tile's loads sit at fixed 32-bit lane
  // offsets from the tile's first row (dma_off), so that a pass adds only a wave-uniform
  // base; the last, partial tile of the range (or a long stride) clamps its rows instead.
  const bool short_stride = q_stride_b * kBQ < (int64_t{1} << 31);
  const uint8_t* dma_src[kDmaPerWave];
  uint32_t dma_off[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int64_t t = qt_first * kBQ + dma_row(i);
    dma_src[i] = q + (t < nq ? t : nq - 1) * q_stride_b + dma_chunk(i) * 16;  // any valid row
    dma_off[i] = static_cast<uint32_t>(short_stride ? dma_row(i) * q_stride_b : 0) +
                 dma_chunk(i) * 16;
  }
  const uint32_t q_lds_a = lds_addr_of(q_lds);
  // Loads of pass jj = qi * h_i + j (query tile qi of the block, head j).
  auto issue = [&](int jj, int qi, int j) {
    const int64_t t0 = (qt_first + qi) * kBQ;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i)
      if (wid + kIdxWaves * i < kDmaPerHead) {
        const uint32_t dst = q_lds_a + (jj % kStages) * kHeadBytes + (wid + kIdxWaves * i) * 1024;
        if constexpr (MULTI) {
          if (short_stride && t0 + kBQ <= nq) {  // wave-uniform: every row of the tile exists
            idx_dma_16b(q + (t0 * q_stride_b + j * kRowBytes) + dma_off[i], dst);
          } else {
            const int64_t t = t0 + dma_row(i);
            idx_dma_16b(
                q + (t < nq ? t : nq - 1) * q_stride_b + j * kRowBytes + dma_chunk(i) * 16, dst);
          }
        } else {
          idx_dma_16b(dma_src[i] + static_cast<int64_t>(j) * kRowBytes, dst);
        }
      }
  };

  f32x4 sc[kMB][NB];
  for (int jj = 0; jj < kStages - 1 && jj < n_pass; ++jj)
    issue(jj, MULTI ? jj / h_i : 0, MULTI ? jj % h_i : jj);
  // Tile and head of the next pass to issue, advanced one pass at a time.
  int ia_q = MULTI ? (kStages - 1) / h_i : 0;
  int ia_j = MULTI ? (kStages - 1) % h_i : kStages - 1;
  // The key rows and the first passes' loads land together.  Waiting for them here, once,
  // also tells the compiler that the key registers are complete before the pass loop;
  // otherwise it would wait for every outstanding load (the prefetched passes included) at
  // their first use in each iteration.
  IDX_WAIT_VMCNT(0);
  // B-operand rows of this lane: query nb * 16 + r16 of the tile.
  const lds_ptr qb = lds_ptr_of(q_lds);
  for (int qi = 0; qi < n_qt; ++qi) {
    const int64_t q0 = (qt_first + qi) * kBQ;
    const bool wave_live = MULTI ? pw0 < vis_last_of(qt_first + qi) : keys_live;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int jj = qi * h_i; jj < (qi + 1) * h_i; ++jj) {
      // Pass jj's loads (and the key rows before them) have landed for this wave.  A
      // finished tile's score stores are younger than some of the loads waited for, so
      // those waits also wait for them (the counter counts in order).
      const int ahead = n_pass - 1 - jj < kStages - 2 ? n_pass - 1 - jj : kStages - 2;
      if (ahead >= 2) {
        IDX_WAIT_VMCNT(2 * kDmaPerWave);
      } else if (ahead == 1) {
        IDX_WAIT_VMCNT(kDmaPerWave);
      } else {
        IDX_WAIT_VMCNT(0);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();  // pass jj's tile is in LDS for every wave; jj - 1 read
      asm volatile("" ::: "memory");
      if (jj + kStages - 1 < n_pass) {
        issue(jj + kStages - 1, ia_q, ia_j);
        if (MULTI && ++ia_j == h_i) {
          ia_j = 0;
          ++ia_q;
        }
        if (!MULTI) ++ia_j;
      }
      if (wave_live) {
        const lds_ptr stage = qb + (jj % kStages) * kHeadBytes;
        // Query fragment of step ks, column block nb (B operand: query nb * 16 + r16).
        auto read_q = [&](int ks, int nb) {
          const int row = nb * 16 + r16;
          const int c0 = (ks * kStepBytes + g * kFragBytes) / 16;
          Frag f;
          if constexpr (FP8) {
            const u32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                stage + row * kRowBytes + ((c0 ^ swz(row)) * 16));
            const u32x4 hi = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                stage + row * kRowBytes + (((c0 + 1) ^ swz(row)) * 16));
            for (int e = 0; e < 4; ++e) {
              f[e] = lo[e];
              f[4 + e] = hi[e];
            }
          } else {
            f = lds_load_bf16x8(stage + row * kRowBytes + ((c0 ^ swz(row)) * 16));
          }
          return f;
        };
        f32x4 acc[kMB][NB];
        auto head_epilogue = [&](int mb, int nb, float wv) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[mb][nb][i] = __builtin_fmaf(wv, relu_bits(acc[mb][nb][i]), sc[mb][nb][i]);
        };
        if constexpr ((MULTI && NB > 1) || FP8) {
          // All pool blocks advance together, one contraction step at a time (the step's
          // query fragments live only through it).  On fp8 every MFMA of the pass issues
          // before the first epilogue value is read (scheduling fences): left to itself the
          // compiler reuses three accumulator sets and waits on each MFMA's result right after
          // the next one issues; grouped, a wave's MFMAs run back to back while the other
          // waves' epilogues fill the SIMD's VALU (2-3% faster on the 256k fp8 workload; with
          // four column blocks the 16 live accumulators would cost a wave per SIMD).
          float wv[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) wv[nb] = w_lds[jj * kBQ + nb * 16 + r16];
          if constexpr (FP8 && NB <= 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) {
            Frag qf[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) qf[nb] = read_q(ks, nb);
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)  // the first step starts from a literal zero
                acc[mb][nb] = mfma_frag<FP8>(kf[mb][ks], qf[nb],
                                             ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mb][nb]);
          }
          if constexpr (FP8 && NB <= 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) head_epilogue(mb, nb, wv[nb]);
        } else {
          // bf16, single tiles and 16-row tile groups: pool blocks in pairs.  A pair's
          // products finish after its own MFMAs (2 NB independent chains), so its ReLU +
          // weight epilogue overlaps the next pair's MFMAs (2-3% faster with 32 heads).  The
          // query fragments of every step stay live through the pass, which 32-row tile
          // groups cannot afford (a wave per SIMD); on fp8 (one step per head) the order
          // measured 1-2% slower.
          static_assert(kMB % 2 == 0, "pool blocks in pairs");
          Frag qf[kKS][NB];
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) qf[ks][nb] = read_q(ks, nb);
          float wv[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) wv[nb] = w_lds[jj * kBQ + nb * 16 + r16];
#pragma unroll
          for (int mp = 0; mp < kMB; mp += 2) {
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
              for (int mb = mp; mb < mp + 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                  acc[mb][nb] = mfma_frag<FP8>(kf[mb][ks], qf[ks][nb],
                                               ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mb][nb]);
#pragma unroll
            for (int mb = mp; mb < mp + 2; ++mb)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) head_epilogue(mb, nb, wv[nb]);
          }
        }
      }
    }
    // The tile's scores are complete.  With several tiles per block, the lane coordinates
    // pass through an empty asm statement first, so that no address or bound of the
    // epilogue (all invariant across tiles) is computed before the tile loop and held in
    // registers through it (that costs a wave per SIMD).
    int r16e = r16, ge = g;
    int64_t pw0e = pw0;
    if constexpr (MULTI) asm volatile("" : "+v"(r16e), "+v"(ge), "+s"(pw0e));
    if constexpr (EMIT) {
      // Candidates: visible entries whose order key reaches the row's threshold, i.e. whose
      // score is >= the threshold's float (one compare each; a threshold key of 0 takes
      // every finite score).  Each lane marks its candidates in a bit mask per row, takes
      // its offset in the tile's share of the row with one LDS atomic, one thread per row
      // reserves that share in the row's list, and the marked entries are written.
      static_assert(2 * kBQ <= kBQ * kMaxHeads, "counters fit the weight array");
      static_assert(kMB * 4 <= 32, "one 32-bit mask per row");
      uint32_t* const c_cnt =
          reinterpret_cast<uint32_t*>(w_lds) + (counters_apart ? h_i * kBQ : 0);
      uint32_t* const c_base = c_cnt + kBQ;
      if (!counters_apart) {
        __syncthreads();
        if (tid < kBQ) c_cnt[tid] = 0u;
        __syncthreads();
      }
      uint32_t mask[NB], off[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t row = q0 + nb * 16 + r16e;
        const bool live = wave_live && row < nq;
        const int64_t vis = live ? vis_of(q_start + row) : 0;
        const uint32_t tk = live ? opt.t_est[row] : 0u;
        // float at the lower edge of the threshold key (keys with the top bit set are the
        // non-negative floats)
        const float thr =
            tk == 0u ? -__builtin_inff()
                     : __uint_as_float((tk & 0x80000000u) ? (tk & 0x7FFFFFFFu) : ~tk);
        uint32_t m = 0u;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            m |= sc[mb][nb][i] >= thr ? (1u << (mb * 4 + i)) : 0u;
        if (pw0e + kPoolsPerWave > vis) {  // tile on the causal boundary: drop invisible pools
          const int64_t lim = vis - (pw0e + ge * 4);  // lane's pools: pw0 + g*4 + 16 mb + i
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (mb * 16 + i >= lim) m &= ~(1u << (mb * 4 + i));
        }
        mask[nb] = m;
        off[nb] = m ? atomicAdd(&c_cnt[nb * 16 + r16e],
                                static_cast<uint32_t>(__builtin_popcount(m)))
                    : 0u;
      }
      __syncthreads();
      if (tid < kBQ && q0 + tid < nq) {
        const uint32_t c = c_cnt[tid];
        c_base[tid] = c ? atomicAdd(&opt.cand_cnt[q0 + tid], c) : 0u;
      }
      __syncthreads();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (!mask[nb]) continue;
        const int64_t row = q0 + nb * 16 + r16e;
        uint32_t slot = c_base[nb * 16 + r16e] + off[nb];
        uint64_t* const dst = opt.cand + row * opt.cand_cap;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          if (!((mask[nb] >> (mb * 4)) & 0xFu)) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (mask[nb] & (1u << (mb * 4 + i))) {
              if (slot < static_cast<uint32_t>(opt.cand_cap))
                dst[slot] = (static_cast<uint64_t>(float_order_key(sc[mb][nb][i])) << 32) |
                            static_cast<uint32_t>(pw0e + mb * 16 + ge * 4 + i);
              ++slot;
            }
          }
        }
      }
    } else if (wave_live) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t row = q0 + nb * 16 + r16e;
        if (row >= nq) continue;
        const int64_t vis = vis_of(q_start + row);
        float* dst_row = scores + row * ld;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          const int64_t p = pw0e + mb * 16 + ge * 4;
          f32x4 val = sc[mb][nb];
          float* dst = dst_row + p;
          if (p + 4 <= vis) {
            if (accumulate) val += *reinterpret_cast<const f32x4*>(dst);
            *reinterpret_cast<f32x4*>(dst) = val;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (p + i < vis) dst[i] = accumulate ? dst[i] + val[i] : val[i];
          }
        }
      }
    }
  }
}

template <int D, int NB, bool FP8, bool MULTI>
hipError_t launch_indexer_nb(const void* q, int64_t q_row_stride, const void* k,
                             int64_t k_row_stride, const float* w, int64_t w_row_stride,
                             float* scores, int64_t ld, int64_t q_start, int64_t nq,
                             int64_t n_pools, int h_i, int accumulate, const IndexerOpts& opt,
                             int64_t n_query_tiles, int64_t n_pool_tiles, int group_tiles,
                             hipStream_t stream) {
  const int64_t elt = FP8 ? 1 : 2;
  const int64_t step = int64_t{1} << opt.pool_shift;
  const int64_t n_query_groups = (n_query_tiles + group_tiles - 1) / group_tiles;
  const int64_t n_tiles = n_query_groups * n_pool_tiles;
  if (n_tiles >= (int64_t{1} << 31) - 8) return hipErrorInvalidConfiguration;
  const int64_t grid = ((n_tiles + 7) / 8) * 8;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kIdxThreads), 0, stream,
                       static_cast<const uint8_t*>(q), q_row_stride * elt,
                       static_cast<const uint8_t*>(k), k_row_stride * elt * step, w,
                       w_row_stride, scores, ld, q_start, nq, n_pools, h_i, accumulate,
                       static_cast<int>(n_pool_tiles), static_cast<int>(n_query_groups),
                       group_tiles, opt);
  };
  if constexpr (MULTI) {
    args(indexer_kernel<D, NB, FP8, false, true>);
  } else {
    if (opt.cand)
      args(indexer_kernel<D, NB, FP8, true, false>);
    else
      args(indexer_kernel<D, NB, FP8, false, false>);
  }
  return hipGetLastError();
}

// Tiles.  With few heads a block's key rows serve little MFMA work per load, so for score
// output a block walks several consecutive 16-row query tiles (MULTI) with its key rows
// resident and the query staging running on across tiles: up to kPassesPerKeyLoad (tile,
// head) passes per key load, fewer tiles while the grid would hold fewer than kMinBlocks
// blocks.  Measured at 8 heads against 64-row single tiles (with 32-row tiles): 5-6% faster
// with 32 passes per load, 12% with 64, 15% with 128; at 32 heads 6-8% slower (so up to 16
// heads only).  16-row tiles (128 VGPRs: four waves per SIMD, and the pool-pair MFMA order
// fits) with 256 passes per load are another 2-3% faster at 1M than 32-row tiles with 128
// (384 passes: 2% slower again).  Otherwise a block owns one tile of 64 rows when few heads
// (at most 8) leave each block little MFMA work per key-row load (the larger tile doubles
// the queries each key row serves: 5% faster at 8 heads, 3% slower at 32), else one tile of
// 16 rows for bf16 scores (120 VGPRs, four waves per SIMD: 2-3% faster at 32 heads than 32
// rows at three waves; tile groups of them are 3-7% slower there) and of 32 rows for fp8
// and the candidate pass.  The 64-row tile and MULTI are kept to d_i <= 128, whose
// key, score and product registers still fit.  The candidate pass (its epilogue holds more
// registers across a tile loop), the sampled pass of the fused select (1% slower with tile
// groups) and launches that compute only flagged tiles take single tiles.
template <int D, bool FP8>
hipError_t launch_indexer_t(const void* q, int64_t q_row_stride, const void* k,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            float* scores, int64_t ld, int64_t q_start, int64_t nq,
                            int64_t n_pools, int h_i, int accumulate, const IndexerOpts& opt,
                            hipStream_t stream) {
  const int64_t step = int64_t{1} << opt.pool_shift;
  const int64_t vis_pools = n_pools < (q_start + nq) / 4 ? n_pools : (q_start + nq) / 4;
  const int64_t vis_max = (vis_pools + step - 1) / step;
  if (nq <= 0 || vis_max <= 0) return hipSuccess;
  const int64_t n_pool_tiles = (vis_max + kPoolsPerBlock - 1) / kPoolsPerBlock;
  const int64_t tiles32 = (nq + 31) / 32;
  const int64_t tiles16 = (nq + 15) / 16;
  if constexpr (D <= 128) {
    const bool single = opt.gate_rows || opt.cand || opt.pool_shift != 0;
    int group_tiles = (single || h_i > kMaxGroupHeads) ? 1 : kPassesPerKeyLoad / h_i;
    while (group_tiles > 1 &&
           ((tiles16 + group_tiles - 1) / group_tiles) * n_pool_tiles < kMinBlocks)
      group_tiles /= 2;
    if (group_tiles > 1)
      return launch_indexer_nb<D, 1, FP8, true>(q, q_row_stride, k, k_row_stride, w,
                                                w_row_stride, scores, ld, q_start, nq, n_pools,
                                                h_i, accumulate, opt, tiles16, n_pool_tiles,
                                                group_tiles, stream);
    if (h_i <= 8)
      return launch_indexer_nb<D, 4, FP8, false>(q, q_row_stride, k, k_row_stride, w,
                                                 w_row_stride, scores, ld, q_start, nq, n_pools,
                                                 h_i, accumulate, opt, (nq + 63) / 64,
                                                 n_pool_tiles, 1, stream);
  }
  if (!FP8 && !opt.cand)  // bf16 scores: 16-row tiles (four waves per SIMD), 2-3% faster
    return launch_indexer_nb<D, 1, FP8, false>(q, q_row_stride, k, k_row_stride, w, w_row_stride,
                                               scores, ld, q_start, nq, n_pools, h_i, accumulate,
                                               opt, tiles16, n_pool_tiles, 1, stream);
  return launch_indexer_nb<D, 2, FP8, false>(q, q_row_stride, k, k_row_stride, w, w_row_stride,
                                             scores, ld, q_start, nq, n_pools, h_i, accumulate,
                                             opt, tiles32, n_pool_tiles, 1, stream);
}

}  // namespace

bool indexer_supported(int d_i, int dtype) {
  if (dtype == 0) return d_i == 32 || d_i == 64 || d_i == 128 || d_i == 256;
  if (dtype == 1) return d_i == 128 || d_i == 256;
  return false;
}

int indexer_max_heads() { return kMaxHeads; }

hipError_t launch_index_scores(const void* q, int64_t q_row_stride, const void* k,
                               int64_t k_row_stride, const float* w, int64_t w_row_stride,
                               float* scores, int64_t ld, int64_t q_start, int64_t nq,
                               int64_t n_pools, int h_i, int d_i, int dtype, int accumulate,
                               hipStream_t stream, const IndexerOpts& opt) {
  if (opt.pool_shift < 0 || opt.pool_shift > 8) return hipErrorInvalidValue;
#define DSA_IDX_CASE(DD, F8)                                                                 \
  return launch_indexer_t<DD, F8>(q, q_row_stride, k, k_row_stride, w, w_row_stride, scores, \
                                  ld, q_start, nq, n_pools, h_i, accumulate, opt, stream)
  if (dtype == 0) {
    switch (d_i) {
      case 32: DSA_IDX_CASE(32, false);
      case 64: DSA_IDX_CASE(64, false);
      case 128: DSA_IDX_CASE(128, false);
      case 256: DSA_IDX_CASE(256, false);
    }
  } else if (dtype == 1) {
    switch (d_i) {
      case 128: DSA_IDX_CASE(128, true);
      case 256: DSA_IDX_CASE(256, true);
    }
  }
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
