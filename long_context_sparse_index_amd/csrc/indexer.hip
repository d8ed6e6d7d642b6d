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
//
// The grid covers the causal trapezoid: tiles whose first pool lies beyond the visible
// prefix of the tile's last query exit at once.  Block ids are remapped so that the pool
// tiles of one query tile run on the same XCD (blocks are dealt to the 8 XCDs round-robin)
// and share the query tile through that XCD's L2.

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

// D: d_i; NB: 16-query column blocks per tile (BQ = 16 * NB); FP8: e4m3 operands.
template <int D, int NB, bool FP8>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(
    const uint8_t* __restrict__ q, int64_t q_stride_b, const uint8_t* __restrict__ k,
    int64_t k_stride_b, const float* __restrict__ w, int64_t w_stride,
    float* __restrict__ scores, int64_t ld, int64_t q_start, int64_t nq, int64_t n_pools,
    int h_i, int accumulate, int n_pool_tiles, int n_query_tiles) {
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
  __shared__ float w_lds[kBQ * kMaxHeads];
  auto swz = [](int r) {
    if constexpr (kCpr >= 16) return r & 15;
    else return (r / (16 / kCpr)) & (kCpr - 1);
  };

  // XCD-aware remap: consecutive logical tiles (same query tile) land on one XCD.
  const int n_tiles = n_pool_tiles * n_query_tiles;
  const int per_xcd = (n_tiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= n_tiles) return;
  const int qt = logical / n_pool_tiles;
  const int pt = logical - qt * n_pool_tiles;
  const int64_t q0 = static_cast<int64_t>(qt) * kBQ;
  const int64_t p0 = static_cast<int64_t>(pt) * kPoolsPerBlock;
  const int64_t rows_here = (nq - q0) < kBQ ? (nq - q0) : kBQ;
  const int64_t vis_last = visible_pools(q_start + q0 + rows_here - 1, n_pools);
  if (p0 >= vis_last) return;  // whole tile above the causal boundary

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t pw0 = p0 + wid * kPoolsPerWave;
  const bool wave_live = pw0 < vis_last;

  // Head weights of the tile's queries, stored [head][query] so that the 16 lanes of a group
  // read 16 consecutive words.
  for (int i = tid; i < kBQ * h_i; i += kIdxThreads) {
    const int row = i / h_i;
    const int j = i - row * h_i;
    w_lds[j * kBQ + row] = (q0 + row < nq) ? w[(q0 + row) * w_stride + j] : 0.0f;
  }

  // This wave's pooled key rows, resident for all heads.
  Frag kf[kMB][kKS];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int64_t pool = pw0 + mb * 16 + r16;
    const bool ok = wave_live && pool < n_pools;
    const uint8_t* kp = k + (ok ? pool : 0) * k_stride_b + g * kFragBytes;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      kf[mb][ks] = ok ? load_frag<FP8>(kp + ks * kStepBytes) : zero_frag<FP8>();
  }

  // This lane's source rows for the query-tile loads: the wave's load i is the head's 1 KB
  // load L = wid + 4 i (if L < kDmaPerHead); lane slot s = 64 L + lane -> row s / kCpr,
  // position s % kCpr.
  const uint8_t* dma_src[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int slot = 64 * (wid + kIdxWaves * i) + lane;
    const int row = (slot / kCpr) % kBQ;  // loads past the tile (not issued) stay in range
    const int chunk = (slot % kCpr) ^ swz(row);
    const int64_t qrow = q0 + row < nq ? q0 + row : nq - 1;  // rows past nq: any valid row
    dma_src[i] = q + qrow * q_stride_b + chunk * 16;
  }
  const uint32_t q_lds_a = lds_addr_of(q_lds);
  auto issue = [&](int j) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i)
      if (wid + kIdxWaves * i < kDmaPerHead)
        idx_dma_16b(dma_src[i] + static_cast<int64_t>(j) * kRowBytes,
                    q_lds_a + (j % kStages) * kHeadBytes + (wid + kIdxWaves * i) * 1024);
  };

  f32x4 sc[kMB][NB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < kStages - 1 && j < h_i; ++j) issue(j);
  // The key rows and the first heads' loads land together.  Waiting for them here, once,
  // also tells the compiler that the key registers are complete before the head loop;
  // otherwise it would wait for every outstanding load (the prefetched heads included) at
  // their first use in each iteration.
  IDX_WAIT_VMCNT(0);
  // B-operand rows of this lane: query nb * 16 + r16 of the tile.
  const lds_ptr qb = lds_ptr_of(q_lds);
  for (int j = 0; j < h_i; ++j) {
    // Head j's loads (and the key rows before them) have landed for this wave.
    const int ahead = h_i - 1 - j < kStages - 2 ? h_i - 1 - j : kStages - 2;
    if (ahead >= 2) {
      IDX_WAIT_VMCNT(2 * kDmaPerWave);
    } else if (ahead == 1) {
      IDX_WAIT_VMCNT(kDmaPerWave);
    } else {
      IDX_WAIT_VMCNT(0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // head j's tile is in LDS for every wave; j - 1 consumed
    asm volatile("" ::: "memory");
    if (j + kStages - 1 < h_i) issue(j + kStages - 1);
    if (wave_live) {
      const lds_ptr stage = qb + (j % kStages) * kHeadBytes;
      f32x4 acc[kMB][NB];
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        Frag qf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int row = nb * 16 + r16;
          const int c0 = (ks * kStepBytes + g * kFragBytes) / 16;
          if constexpr (FP8) {
            const u32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                stage + row * kRowBytes + ((c0 ^ swz(row)) * 16));
            const u32x4 hi = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                stage + row * kRowBytes + (((c0 + 1) ^ swz(row)) * 16));
            for (int e = 0; e < 4; ++e) {
              qf[nb][e] = lo[e];
              qf[nb][4 + e] = hi[e];
            }
          } else {
            qf[nb] = lds_load_bf16x8(stage + row * kRowBytes + ((c0 ^ swz(row)) * 16));
          }
        }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)  // the first step starts from a literal zero
            acc[mb][nb] = mfma_frag<FP8>(kf[mb][ks], qf[nb],
                                         ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mb][nb]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float wv = w_lds[j * kBQ + nb * 16 + r16];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[mb][nb][i] = __builtin_fmaf(wv, relu_bits(acc[mb][nb][i]), sc[mb][nb][i]);
      }
    }
  }
  if (!wave_live) return;

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t row = q0 + nb * 16 + r16;
    if (row >= nq) continue;
    const int64_t vis = visible_pools(q_start + row, n_pools);
    float* dst_row = scores + row * ld;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int64_t p = pw0 + mb * 16 + g * 4;
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

template <int D, int NB, bool FP8>
hipError_t launch_indexer_nb(const void* q, int64_t q_row_stride, const void* k,
                             int64_t k_row_stride, const float* w, int64_t w_row_stride,
                             float* scores, int64_t ld, int64_t q_start, int64_t nq,
                             int64_t n_pools, int h_i, int accumulate, hipStream_t stream) {
  constexpr int kBQ = 16 * NB;
  const int64_t elt = FP8 ? 1 : 2;
  const int64_t vis_max = n_pools < (q_start + nq) / 4 ? n_pools : (q_start + nq) / 4;
  if (nq <= 0 || vis_max <= 0) return hipSuccess;
  const int64_t n_query_tiles = (nq + kBQ - 1) / kBQ;
  const int64_t n_pool_tiles = (vis_max + kPoolsPerBlock - 1) / kPoolsPerBlock;
  const int64_t n_tiles = n_query_tiles * n_pool_tiles;
  if (n_tiles >= (int64_t{1} << 31) - 8) return hipErrorInvalidConfiguration;
  const int64_t grid = ((n_tiles + 7) / 8) * 8;
  hipLaunchKernelGGL((indexer_kernel<D, NB, FP8>), dim3(static_cast<unsigned>(grid)),
                     dim3(kIdxThreads), 0, stream, static_cast<const uint8_t*>(q),
                     q_row_stride * elt, static_cast<const uint8_t*>(k), k_row_stride * elt, w,
                     w_row_stride, scores, ld, q_start, nq, n_pools, h_i, accumulate,
                     static_cast<int>(n_pool_tiles), static_cast<int>(n_query_tiles));
  return hipGetLastError();
}

// Query tile of 32 rows, or of 64 rows when few heads (at most 8) leave each block little
// MFMA work per key-row load: the larger tile doubles the queries each key row serves
// (measured 5% faster at 8 heads, 3% slower at 32).  The 64-row tile is kept to d_i <= 128,
// whose key, score and product registers still fit.
template <int D, bool FP8>
hipError_t launch_indexer_t(const void* q, int64_t q_row_stride, const void* k,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            float* scores, int64_t ld, int64_t q_start, int64_t nq,
                            int64_t n_pools, int h_i, int accumulate, hipStream_t stream) {
  if constexpr (D <= 128) {
    if (h_i <= 8)
      return launch_indexer_nb<D, 4, FP8>(q, q_row_stride, k, k_row_stride, w, w_row_stride,
                                          scores, ld, q_start, nq, n_pools, h_i, accumulate,
                                          stream);
  }
  return launch_indexer_nb<D, 2, FP8>(q, q_row_stride, k, k_row_stride, w, w_row_stride, scores,
                                      ld, q_start, nq, n_pools, h_i, accumulate, stream);
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
                               hipStream_t stream) {
#define DSA_IDX_CASE(DD, F8)                                                                 \
  return launch_indexer_t<DD, F8>(q, q_row_stride, k, k_row_stride, w, w_row_stride, scores, \
                                  ld, q_start, nq, n_pools, h_i, accumulate, stream)
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
