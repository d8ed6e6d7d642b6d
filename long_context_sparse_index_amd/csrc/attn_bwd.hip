// Backward of the sparse MQA attention, on gfx950 MFMA with fp32 atomics for dK/dV.
//
// The pages train the layer (page "SkyRL extends GLM-5.3-Flash training context to 1 million
// tokens", from the title on) but print no backward; this is the exact gradient of the
// forward in attn_fwd.hip.  With P = exp(scale q.K - LSE), dP = dO.V, D = dO.O and
// dS = P (dP - D):
//     dQ = scale dS K,   dK[idx] += scale dS^T q,   dV[idx] += P^T dO.
//
// Three launches on the caller's stream:
//   1. delta: D[t, h] = dO[t, h, :] . O[t, h, :], one wave per (token, head) row.
//   2. dq: per token, one wave per 16 heads, over 32-key tiles of the gathered latent rows:
//      recompute S^T and P^T as the forward does, dP^T = V_tile . dO^T (A: value rows from
//      LDS, B: the wave's dO, held in registers) and dS^T in registers; dS^T of all heads is
//      exchanged through LDS and each wave accumulates dQ^T += K_tile^T . dS^T for a quarter
//      of the columns and all heads, K^T from LDS transpose reads; dQ stays in registers.
//   3. dkv: per token, the same recomputation, then P^T and dS^T of all 64 heads go to LDS
//      and each wave forms its quarter of the tile's columns of
//          dK_tile = dS^T . Q (contraction over the 64 heads),  dV_tile = P^T . dO
//      so every (selected row, column) gets one fp32 atomic add per token, with the head
//      sum already done in the MFMA.  The Q and dO operands for that product (heads along
//      the contraction) are built once per token from LDS-staged copies with transpose
//      reads.  With V aliased to the first d_v columns of the latent row and no separate
//      dV buffer, the two contributions are added before the single atomic.
// Probabilities and dS enter the MFMAs as bf16 hi + lo pairs (about 16 significant bits).
// Summation order of the atomics varies from run to run.
//
// Deterministic variant: no atomics.  Query rows go in chunks; for each chunk the dkv kernel
// writes every (row, slot) pair's head-summed dK (and dV) row to a staging buffer, then
// bwd_reduce.hip sorts the chunk's selection by pool (stable, so pairs keep their row-major
// order) and one workgroup per pool adds that pool's staged rows in that order into dkv (and
// dv).  Chunks are reduced one after another, so every sum has a fixed order.

#include <mutex>

#include "attn_common.hpp"
#include "launch.hpp"

// Static scratch of the allocation-free backward entry point: the per-row deltas
// D[t, h] = dO . O of one call, at most kBwdScratchFloats of them (16 MiB).  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): it uses the device address
// that hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr long long kBwdScratchFloats = 1ll << 22;
static __device__ __align__(256) float scratch[kBwdScratchFloats];

namespace dsa {
namespace {

// ---------------------------------------------------------------- 1. D = rowsum(dO * O)
template <int DV, bool O_F32>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const void* __restrict__ o,
                                                             const uint16_t* __restrict__ d_o,
                                                             float* __restrict__ delta,
                                                             int64_t n_rows) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int lane = threadIdx.x & 63;
  float acc = 0.0f;
  for (int e = lane * 8; e < DV; e += 512) {
    const u32x4 dv4 = *reinterpret_cast<const u32x4*>(d_o + r * DV + e);
    float ov[8];
    if constexpr (O_F32) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + r * DV + e);
      const f32x4 b =
          *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + r * DV + e + 4);
      for (int i = 0; i < 4; ++i) ov[i] = a[i], ov[4 + i] = b[i];
    } else {
      const u32x4 a =
          *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o) + r * DV + e);
      for (int i = 0; i < 4; ++i) {
        ov[2 * i] = __uint_as_float(a[i] << 16);
        ov[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      }
    }
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(dv4[i] << 16) * ov[2 * i];
      acc += __uint_as_float(dv4[i] & 0xFFFF0000u) * ov[2 * i + 1];
    }
  }
  for (int m = 32; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
  if (lane == 0) delta[r] = acc;
}

// Per-tile recomputation shared by the dq and dkv kernels: S^T, P^T, dP^T and dS^T of the
// wave's 16 heads for the 32 keys of the tile.  Probabilities and dS come back as bf16
// hi/lo operand pairs in the S^T slot order (slot 4 mb + i <-> key 16 mb + 4 g + i).
struct TileGrads {
  bf16x8 p_hi, p_lo, ds_hi, ds_lo;
  float p[2][4], ds[2][4];
};

template <int DQK, int DV, int VBASE>
__device__ __forceinline__ void tile_grads(lds_ptr tile, const bf16x8* qf,
                                           const bf16x8* dof, int slot0, int n_valid,
                                           bool head_ok, float scale_log2, float lse2,
                                           float dh, int g, int r16, TileGrads& out) {
  constexpr int kKS = DQK / 32;
  constexpr int kVS = DV / 32;
  f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  // With V aliased to the key row's first DV columns, one LDS read feeds both products.
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 a = lds_load_bf16x8(tile + tile_off(4 * ks + g, mb * 16 + r16));
      s[mb] = mfma16x16x32_bf16(a, qf[ks], s[mb]);
      if (VBASE == 0 && ks < kVS) dp[mb] = mfma16x16x32_bf16(a, dof[ks], dp[mb]);
    }
  if constexpr (VBASE != 0) {
#pragma unroll
    for (int ks = 0; ks < kVS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        dp[mb] = mfma16x16x32_bf16(
            lds_load_bf16x8(tile + tile_off(VBASE + 4 * ks + g, mb * 16 + r16)), dof[ks],
            dp[mb]);
  }
  f32x8 pv, dv;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = head_ok && slot0 + mb * 16 + 4 * g + i < n_valid;
      const float p = ok ? __builtin_exp2f(s[mb][i] * scale_log2 - lse2) : 0.0f;
      const float d = p * (dp[mb][i] - dh);
      out.p[mb][i] = p;
      out.ds[mb][i] = d;
      pv[mb * 4 + i] = p;
      dv[mb * 4 + i] = d;
    }
  // hi = RNE(x), lo = RNE(x - hi) with the hardware packed conversion
  split_bf16x8(pv, out.p_hi, out.p_lo);
  split_bf16x8(dv, out.ds_hi, out.ds_lo);
}

// The wave's B operands for S^T (queries) and dP^T (dO): lane column = head.
template <int DQK, int DV>
__device__ __forceinline__ void load_head_operands(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ d_o,
                                                   int64_t row, int h, int head, bool head_ok,
                                                   int g, bf16x8* qf, bf16x8* dof) {
  const uint16_t* qrow = q + (row * h + (head_ok ? head : 0)) * DQK + g * 8;
  const uint16_t* drow = d_o + (row * h + (head_ok ? head : 0)) * DV + g * 8;
#pragma unroll
  for (int ks = 0; ks < DQK / 32; ++ks)
    qf[ks] = head_ok ? *reinterpret_cast<const bf16x8*>(qrow + ks * 32) : bf16x8_zero();
#pragma unroll
  for (int ks = 0; ks < DV / 32; ++ks)
    dof[ks] = head_ok ? *reinterpret_cast<const bf16x8*>(drow + ks * 32) : bf16x8_zero();
}

// ---------------------------------------------------------------- 2. dQ
// dS^T of all heads is exchanged through LDS so that each wave forms a quarter of the columns
// of dQ^T = K^T . dS^T for all heads: every transposed key block is read by one wave instead
// of four.  Exchange layout: [hi/lo][head][position] bf16 with the tile's keys at position
// 8 g + 4 mb + i for key 16 mb + 4 g + i (the operand slot order of lane group g), so a lane
// writes its 8 values with one 16-byte store and reads an operand with one 16-byte load;
// rows of 40 bf16 (80 bytes) keep the 16 lanes of a group on distinct banks.  Two buffers
// alternate between tiles.
constexpr int kDsRow = 40;
constexpr int kDsBuf = 2 * 64 * kDsRow;  // bf16 per buffer (hi and lo)
constexpr int kDqXchgBytes = 2 * kDsBuf * 2;

template <int DQK, int DV, bool SEPARATE_V>
__global__ __launch_bounds__(kAttnThreads) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t ld_kv,
    const uint16_t* __restrict__ v, int64_t ld_v, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ lse, const uint16_t* __restrict__ d_o,
    const float* __restrict__ delta, float* __restrict__ dq, int64_t n_pools, int h,
    float scale_log2, float scale) {
  constexpr int kTileBytes = TileDma<DQK, DV, SEPARATE_V, 1>::kTileBytes;
  using Dma = TileDma<DQK, DV, SEPARATE_V,
                      pick_depth(kTileBytes, kMaxTopK * 4 + 64 + kDqXchgBytes)>;
  constexpr int kNBW = DQK / 64;  // 16-column blocks of dQ per wave (a quarter of DQK)
  static_assert(DQK % 64 == 0, "column quarters of whole 16-column blocks");
  __shared__ __attribute__((aligned(16))) uint8_t tiles[Dma::kLdsBytes];
  __shared__ __attribute__((aligned(16))) uint16_t dsx[2 * kDsBuf];
  __shared__ int32_t sel[kMaxTopK];
  __shared__ int wave_tmp[kAttnThreads / 64];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t row = blockIdx.x;
  const int head = wid * 16 + r16;
  const bool head_ok = head < h;
  const bool wave_has_heads = wid * 16 < h;
  const int nb0 = wid * kNBW;  // this wave's first column block

  const int n_valid = compact_selection(idx + row * k, k, n_pools, sel, wave_tmp);
  bf16x8 qf[DQK / 32], dof[DV / 32];
  load_head_operands<DQK, DV>(q, d_o, row, h, head, head_ok, g, qf, dof);
  const float lse2 = head_ok && n_valid > 0 ? lse[row * h + head] * kLog2e : 0.0f;
  const float dh = head_ok ? delta[row * h + head] : 0.0f;
  DSA_WAIT_VMCNT(0);  // operands in registers before the tile pipeline starts

  f32x4 acc[4][kNBW];  // [head block][column block]
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) acc[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_tiles = (n_valid + kKeysPerTile - 1) / kKeysPerTile;
  Dma::for_each_tile(tiles, n_tiles, sel, n_valid, kv, ld_kv, v, ld_v,
                     [&](lds_ptr tile, int t) {
    uint16_t* const xb = dsx + (t & 1) * kDsBuf;
    bf16x8 ds_hi = bf16x8_zero(), ds_lo = bf16x8_zero();
    if (wave_has_heads) {
      TileGrads tg;
      tile_grads<DQK, DV, Dma::kVBase>(tile, qf, dof, t * kKeysPerTile, n_valid, head_ok,
                                       scale_log2, lse2, dh, g, r16, tg);
      ds_hi = tg.ds_hi;
      ds_lo = tg.ds_lo;
    }
    *reinterpret_cast<bf16x8*>(xb + head * kDsRow + 8 * g) = ds_hi;
    *reinterpret_cast<bf16x8*>(xb + 64 * kDsRow + head * kDsRow + 8 * g) = ds_lo;
    DSA_WAIT_LGKMCNT0();
    tile_barrier();  // every head's dS^T of tile t is in the exchange buffer
    bf16x8 b_hi[4], b_lo[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      b_hi[hb] = *reinterpret_cast<const bf16x8*>(xb + (hb * 16 + r16) * kDsRow + 8 * g);
      b_lo[hb] =
          *reinterpret_cast<const bf16x8*>(xb + 64 * kDsRow + (hb * 16 + r16) * kDsRow + 8 * g);
    }
    // dQ^T += K^T . dS^T over the tile's keys, this wave's columns, all heads.
    const lds_ptr kt_base = tile + tile_tr_lane_off(0, g, r16);
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) {
      const bf16x8 kt = tile_tr_block(kt_base, nb0 + nb);
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        acc[hb][nb] = mfma16x16x32_bf16(kt, b_hi[hb], acc[hb][nb]);
        acc[hb][nb] = mfma16x16x32_bf16(kt, b_lo[hb], acc[hb][nb]);
      }
    }
  });
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int hh = hb * 16 + r16;
    if (hh >= h) continue;
    float* out = dq + (row * h + hh) * DQK + nb0 * 16 + 4 * g;
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
      *reinterpret_cast<f32x4*>(out + nb * 16) = acc[hb][nb] * scale;
  }
}

// ---------------------------------------------------------------- 3. dK, dV
constexpr int kHeadsPad = 64;       // heads of the LDS-staged operands (zero beyond h)
constexpr int kPsRow = kHeadsPad + 8;  // bf16 per key row of the P / dS arrays (padded)

template <int DQK, int DV, bool SEPARATE_V>
struct DkvLds {
  static constexpr int kStageQ = kHeadsPad * (DQK + 8) * 2;
  static constexpr int kStageO = kHeadsPad * (DV + 8) * 2;
  static constexpr int kStage = kStageQ > kStageO ? kStageQ : kStageO;
  static constexpr int kOther = 4 * kKeysPerTile * kPsRow * 2 + kMaxTopK * 6 + 64;
  static constexpr int kTileBytes = TileDma<DQK, DV, SEPARATE_V, 1>::kTileBytes;
  // Tile stages share the staging region; deepest pipeline that fits beside the rest.
  static constexpr int kDepth = 3 * kTileBytes + kOther <= 160 * 1024 - 256   ? 3
                                : 2 * kTileBytes + kOther <= 160 * 1024 - 256 ? 2
                                                                              : 1;
  using Dma = TileDma<DQK, DV, SEPARATE_V, kDepth>;
  static constexpr int kShared = kStage > Dma::kLdsBytes ? kStage : Dma::kLdsBytes;
};

// B operand for a product contracting over heads: lane (g, r) gets X[32 ks + 8 g + s][col0 + r]
// for s = 0..7 from a row-major LDS copy X[head][col] with row stride `ld` elements.
__device__ __forceinline__ bf16x8 heads_operand(const uint16_t* x, int ld, int ks, int col0,
                                                int g, int r16) {
  const int hrow = 32 * ks + 8 * g + (r16 >> 2);
  const int col = col0 + 4 * (r16 & 3);
  const i16x4 lo = lds_read_tr16(x + hrow * ld + col);
  const i16x4 hi = lds_read_tr16(x + (hrow + 4) * ld + col);
  return join_tr(lo, hi);
}

// How the dK/dV kernel delivers its per-token tile results.
enum DkvMode {
  kDkvAtomic = 0,     // fp32 atomic adds into dkv [n_pools, DQK] (and dv [n_pools, DV], or
                      // dV folded into dkv when dv is null)
  kDkvStageFold = 1,  // staging rows (see below) of DQK: dK with dV added into its first DV
  kDkvStageSplit = 2  // staging rows of DQK (dK) and, in dv, of DV (dV)
};

// Staging modes: dkv (and dv) hold one row per (query row, slot) of this launch, row index
// row * k + slot, written (not added) for every valid slot; row `junk` receives the stores of
// the invalid slots of a partial last tile (and, for dv, of the columns past DV), so that
// every tile issues the same number of stores and the tile pipeline can leave them in flight.
template <int DQK, int DV, bool SEPARATE_V, int MODE>
__global__ __launch_bounds__(kAttnThreads) void attn_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t ld_kv,
    const uint16_t* __restrict__ v, int64_t ld_v, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ lse, const uint16_t* __restrict__ d_o,
    const float* __restrict__ delta, float* __restrict__ dkv, float* __restrict__ dv,
    int64_t n_pools, int h, float scale_log2, float scale, int64_t junk) {
  constexpr bool STAGE = MODE != kDkvAtomic;
  using Lds = DkvLds<DQK, DV, SEPARATE_V>;
  using Dma = typename Lds::Dma;
  constexpr int kCols = DQK / 4;     // output columns owned by each wave
  constexpr int kNBW = kCols / 16;
  static_assert(kCols % 16 == 0, "column split");
  __shared__ __attribute__((aligned(16))) uint8_t shared[Lds::kShared];  // staging, then tiles
  __shared__ __attribute__((aligned(16))) uint16_t ps[4][kKeysPerTile * kPsRow];
  __shared__ int32_t sel[kMaxTopK];
  __shared__ int16_t slot_of[kMaxTopK];
  __shared__ int wave_tmp[kAttnThreads / 64];
  uint16_t* stage = reinterpret_cast<uint16_t*>(shared);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t row = blockIdx.x;
  const int head = wid * 16 + r16;
  const bool head_ok = head < h;
  const bool wave_has_heads = wid * 16 < h;
  const int col_base = wid * kCols;

  const int n_valid =
      compact_selection(idx + row * k, k, n_pools, sel, wave_tmp, STAGE ? slot_of : nullptr);
  if (n_valid == 0) return;  // uniform: no selected row receives anything from this token

  // Operands with heads along the contraction, for this wave's columns: Q, then dO.
  bf16x8 qb[kNBW][2], db[kNBW][2];
  {
    constexpr int ld = DQK + 8;
    for (int i = tid; i < kHeadsPad * (DQK / 8); i += kAttnThreads) {
      const int hh = i / (DQK / 8), c = i - hh * (DQK / 8);
      u32x4 val = {0u, 0u, 0u, 0u};
      if (hh < h) val = *reinterpret_cast<const u32x4*>(q + (row * h + hh) * DQK + 8 * c);
      *reinterpret_cast<u32x4*>(stage + hh * ld + 8 * c) = val;
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        qb[nb][ks] = heads_operand(stage, ld, ks, col_base + 16 * nb, g, r16);
    __syncthreads();
  }
  {
    constexpr int ld = DV + 8;
    for (int i = tid; i < kHeadsPad * (DV / 8); i += kAttnThreads) {
      const int hh = i / (DV / 8), c = i - hh * (DV / 8);
      u32x4 val = {0u, 0u, 0u, 0u};
      if (hh < h) val = *reinterpret_cast<const u32x4*>(d_o + (row * h + hh) * DV + 8 * c);
      *reinterpret_cast<u32x4*>(stage + hh * ld + 8 * c) = val;
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        db[nb][ks] = col_base + 16 * nb < DV
                         ? heads_operand(stage, ld, ks, col_base + 16 * nb, g, r16)
                         : bf16x8_zero();
  }

  bf16x8 qf[DQK / 32], dof[DV / 32];
  load_head_operands<DQK, DV>(q, d_o, row, h, head, head_ok, g, qf, dof);
  const float lse2 = head_ok ? lse[row * h + head] * kLog2e : 0.0f;
  const float dh = head_ok ? delta[row * h + head] : 0.0f;
  const bool fold_v = dv == nullptr;  // V aliased and its gradient folded into dkv
  DSA_WAIT_VMCNT(0);  // operands in registers before the tile pipeline starts

  const int n_tiles = (n_valid + kKeysPerTile - 1) / kKeysPerTile;
  // Stores of one tile in each wave (staging modes): one 16-byte store per (row block,
  // column block), twice with separate dV rows.
  constexpr int kTileStores = MODE == kDkvAtomic ? 0 : 2 * kNBW * (MODE == kDkvStageSplit ? 2 : 1);
  __syncthreads();  // the staging copies are fully read before tiles overwrite them
  Dma::template for_each_tile<kTileStores>(shared, n_tiles, sel, n_valid, kv, ld_kv, v, ld_v,
                                           [&](lds_ptr tile, int t) {
    const int slot0 = t * kKeysPerTile;
    TileGrads tg;
    if (wave_has_heads) {
      tile_grads<DQK, DV, Dma::kVBase>(tile, qf, dof, slot0, n_valid, head_ok, scale_log2,
                                       lse2, dh, g, r16, tg);
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tg.p[mb][i] = tg.ds[mb][i] = 0.0f;
    }
    // P^T and dS^T of this wave's heads into the [key][head] arrays (hi, lo parts).
    {
      f32x8 pv, dv8;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[mb * 4 + i] = tg.p[mb][i], dv8[mb * 4 + i] = tg.ds[mb][i];
      bf16x8 parts[4];
      split_bf16x8(pv, parts[0], parts[1]);
      split_bf16x8(dv8, parts[2], parts[3]);
#pragma unroll
      for (int arr = 0; arr < 4; ++arr) {
        const i16x8 bits = __builtin_bit_cast(i16x8, parts[arr]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ps[arr][(mb * 16 + 4 * g + i) * kPsRow + head] =
                static_cast<uint16_t>(bits[mb * 4 + i]);
      }
    }
    DSA_WAIT_LGKMCNT0();
    tile_barrier();
    // This wave's columns of dK_tile = dS^T . Q and dV_tile = P^T . dO (64-head contraction).
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      bf16x8 a[4][2];
#pragma unroll
      for (int arr = 0; arr < 4; ++arr)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          a[arr][ks] = *reinterpret_cast<const bf16x8*>(
              &ps[arr][(mb * 16 + r16) * kPsRow + 32 * ks + 8 * g]);
      if constexpr (STAGE) {
        // Transposed products dK^T = Q^T . dS, dV^T = dO^T . P: lane (g, r) ends with columns
        // col0 + 4 g .. col0 + 4 g + 3 of key 16 mb + r, one 16-byte store per block.
        const int slot = slot0 + mb * 16 + r16;
        const int64_t srow = slot < n_valid ? row * k + slot_of[slot] : junk;
#pragma unroll
        for (int nb = 0; nb < kNBW; ++nb) {
          const int col0 = col_base + 16 * nb;
          f32x4 ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            ak = mfma16x16x32_bf16(qb[nb][ks], a[2][ks], ak);
            ak = mfma16x16x32_bf16(qb[nb][ks], a[3][ks], ak);
          }
          f32x4 av = {0.f, 0.f, 0.f, 0.f};
          if (col0 < DV) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              av = mfma16x16x32_bf16(db[nb][ks], a[0][ks], av);
              av = mfma16x16x32_bf16(db[nb][ks], a[1][ks], av);
            }
          }
          const int c = col0 + 4 * g;
          if constexpr (MODE == kDkvStageFold) {
            *reinterpret_cast<f32x4*>(dkv + srow * DQK + c) = ak * scale + av;
          } else {
            *reinterpret_cast<f32x4*>(dkv + srow * DQK + c) = ak * scale;
            const bool in_v = col0 < DV;
            *reinterpret_cast<f32x4*>(dv + (in_v ? srow : junk) * DV + (in_v ? c : 4 * g)) = av;
          }
        }
        continue;
      }
      int64_t dst[4];  // gradient row (pool); -1: none
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = slot0 + mb * 16 + 4 * g + i;
        dst[i] = slot < n_valid ? sel[slot] : -1;
      }
#pragma unroll
      for (int nb = 0; nb < kNBW; ++nb) {
        const int col0 = col_base + 16 * nb;
        f32x4 ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          ak = mfma16x16x32_bf16(a[2][ks], qb[nb][ks], ak);
          ak = mfma16x16x32_bf16(a[3][ks], qb[nb][ks], ak);
        }
        f32x4 av = {0.f, 0.f, 0.f, 0.f};
        if (col0 < DV) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            av = mfma16x16x32_bf16(a[0][ks], db[nb][ks], av);
            av = mfma16x16x32_bf16(a[1][ks], db[nb][ks], av);
          }
        }
        const int col = col0 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (dst[i] < 0) continue;
          const int64_t kat = dst[i] * DQK + col;
          const float gk = fold_v ? ak[i] * scale + (col0 < DV ? av[i] : 0.0f) : ak[i] * scale;
          atomicAdd(dkv + kat, gk);
          if (!fold_v && col0 < DV) atomicAdd(dv + dst[i] * DV + col, av[i]);
        }
      }
    }
  });
}

// Query rows per chunk of the deterministic backward: its staging holds one dK (and dV) row
// per (row, slot) of a chunk, e.g. 4096 * 2048 * 576 floats (19.3 GB) for 576-wide rows.
constexpr int64_t kDetChunkRows = 4096;

struct DetLayout {
  size_t stage_k, stage_v, reduce, total;
};

size_t align256(size_t b) { return (b + 255) & ~size_t{255}; }

DetLayout det_layout(int64_t rows, int k, int64_t n_pools, int d_qk, int d_v, bool separate_dv) {
  DetLayout L{};
  // one staging row per (row, slot) pair, plus the row that takes the stores of invalid
  // slots
  const size_t pairs = static_cast<size_t>(rows > 0 ? rows : 0) * static_cast<size_t>(k) + 1;
  size_t off = 0;
  L.stage_k = off;
  off += align256(pairs * d_qk * sizeof(float));
  L.stage_v = off;
  if (separate_dv) off += align256(pairs * d_v * sizeof(float));
  L.reduce = off;
  off += pool_reduce_workspace_bytes(static_cast<int64_t>(pairs - 1), n_pools);
  L.total = off;
  return L;
}

template <int DQK, int DV, bool SEP>
hipError_t launch_bwd_t(const void* q, const void* kv, int64_t ld_kv, const void* v,
                        int64_t ld_v, const int32_t* idx, int k, const void* o, int o_f32,
                        const float* lse, const void* d_o, float* dq, float* dkv, float* dv,
                        int64_t nq, int64_t n_pools, int h, float scale, float* delta,
                        char* det_ws, hipStream_t stream) {
  const int64_t rows = nq * h;
  const unsigned dgrid = static_cast<unsigned>((rows + 3) / 4);
  if (o_f32)
    hipLaunchKernelGGL((attn_bwd_delta_kernel<DV, true>), dim3(dgrid), dim3(256), 0, stream, o,
                       static_cast<const uint16_t*>(d_o), delta, rows);
  else
    hipLaunchKernelGGL((attn_bwd_delta_kernel<DV, false>), dim3(dgrid), dim3(256), 0, stream, o,
                       static_cast<const uint16_t*>(d_o), delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = scale * kLog2e;
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kvb = static_cast<const uint16_t*>(kv);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  const uint16_t* dob = static_cast<const uint16_t*>(d_o);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, SEP>), dim3(static_cast<unsigned>(nq)),
                     dim3(kAttnThreads), 0, stream, qb, kvb, ld_kv, vb, ld_v, idx, k, lse, dob,
                     delta, dq, n_pools, h, sl2, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!det_ws) {
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<DQK, DV, SEP, kDkvAtomic>),
                       dim3(static_cast<unsigned>(nq)), dim3(kAttnThreads), 0, stream, qb, kvb,
                       ld_kv, vb, ld_v, idx, k, lse, dob, delta, dkv, dv, n_pools, h, sl2,
                       scale, int64_t{-1});
    return hipGetLastError();
  }
  // Deterministic: chunk by chunk, staged rows, then the ordered per-pool reduction.
  const int64_t chunk = nq < kDetChunkRows ? nq : kDetChunkRows;
  const DetLayout L = det_layout(chunk, k, n_pools, DQK, DV, dv != nullptr);
  float* stage_k = reinterpret_cast<float*>(det_ws + L.stage_k);
  float* stage_v = dv ? reinterpret_cast<float*>(det_ws + L.stage_v) : nullptr;
  void* red = det_ws + L.reduce;
  const int64_t junk = chunk * k;  // the staging row past the chunk's (row, slot) rows
  for (int64_t r0 = 0; r0 < nq; r0 += chunk) {
    const int64_t m = nq - r0 < chunk ? nq - r0 : chunk;
    if (dv)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<DQK, DV, SEP, kDkvStageSplit>),
                         dim3(static_cast<unsigned>(m)), dim3(kAttnThreads), 0, stream,
                         qb + r0 * h * DQK, kvb, ld_kv, vb, ld_v, idx + r0 * k, k, lse + r0 * h,
                         dob + r0 * h * DV, delta + r0 * h, stage_k, stage_v, n_pools, h, sl2,
                         scale, junk);
    else
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<DQK, DV, SEP, kDkvStageFold>),
                         dim3(static_cast<unsigned>(m)), dim3(kAttnThreads), 0, stream,
                         qb + r0 * h * DQK, kvb, ld_kv, vb, ld_v, idx + r0 * k, k, lse + r0 * h,
                         dob + r0 * h * DV, delta + r0 * h, stage_k, stage_v, n_pools, h, sl2,
                         scale, junk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_pool_reduce(idx + r0 * k, m, k, n_pools, stage_k, DQK, dkv, stage_v, DV, dv, red,
                           stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t nq, int h) {
  return static_cast<size_t>(nq > 0 ? nq : 0) * static_cast<size_t>(h > 0 ? h : 0) * sizeof(float);
}

int64_t attn_bwd_scratch_floats() { return kBwdScratchFloats; }

hipError_t attn_bwd_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

size_t attn_bwd_det_bytes(int64_t nq, int64_t n_pools, int k, int d_qk, int d_v,
                          bool separate_dv) {
  if (nq <= 0 || k <= 0 || d_qk <= 0 || d_v <= 0) return 0;
  const int64_t chunk = nq < kDetChunkRows ? nq : kDetChunkRows;
  return det_layout(chunk, k, n_pools > 0 ? n_pools : 0, d_qk, d_v, separate_dv).total;
}

hipError_t launch_sparse_attn_bwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                                  int64_t ld_v, const int32_t* idx, int k, const void* o,
                                  int o_f32, const float* lse, const void* d_o, float* dq,
                                  float* dkv, float* dv, int64_t nq, int64_t n_pools, int h,
                                  int d_qk, int d_v, float scale, void* ws,
                                  hipStream_t stream, void* det_ws) {
  if (nq <= 0) return hipSuccess;
  if (nq * h >= (int64_t{1} << 33)) return hipErrorInvalidConfiguration;
  if (det_ws && (nq < kDetChunkRows ? nq : kDetChunkRows) * k >= (int64_t{1} << 31))
    return hipErrorInvalidConfiguration;
  float* delta = static_cast<float*>(ws);
  char* det = static_cast<char*>(det_ws);
#define DSA_BWD(DQ, DVV)                                                                      \
  return v ? launch_bwd_t<DQ, DVV, true>(q, kv, ld_kv, v, ld_v, idx, k, o, o_f32, lse, d_o,   \
                                         dq, dkv, dv, nq, n_pools, h, scale, delta, det,      \
                                         stream)                                              \
           : launch_bwd_t<DQ, DVV, false>(q, kv, ld_kv, nullptr, 0, idx, k, o, o_f32, lse,    \
                                          d_o, dq, dkv, dv, nq, n_pools, h, scale, delta,     \
                                          det, stream)
  if (d_qk == 128 && d_v == 128) DSA_BWD(128, 128);
  if (d_qk == 576 && d_v == 512) DSA_BWD(576, 512);
  if (d_qk == 512 && d_v == 512) DSA_BWD(512, 512);
  if (d_qk == 256 && d_v == 256) DSA_BWD(256, 256);
#undef DSA_BWD
  return hipErrorInvalidValue;
}

}  // namespace dsa
