// Pieces shared by the sparse-attention kernels (forward and backward): the compaction of a
// selection row, the gather of 32 selected latent KV rows into an LDS tile, and the join of
// two LDS transpose reads into one MFMA operand.  Internal to libdsa.
#pragma once

#include "common.hpp"

namespace dsa {

constexpr int kKeysPerTile = 32;
constexpr int kAttnThreads = 256;  // 4 waves gather every tile; waves without heads only gather
constexpr int kMaxTopK = 4096;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Joins two transpose reads into one 8-slot bf16 MFMA operand (slots 0..3, then 4..7).
__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Compacts the valid slots of one selection row (0 <= idx < n_pools; -1 marks an empty
// slot, and any other value is skipped the same way so that no gather leaves the table)
// into sel[], in slot order, and returns their count.  All threads of the block call it.
__device__ inline int compact_selection(const int32_t* __restrict__ irow, int k,
                                        int64_t n_pools, int32_t* sel, int* wave_tmp) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  constexpr int kWaves = kAttnThreads / 64;
  int base = 0;
  for (int s0 = 0; s0 < k; s0 += kAttnThreads) {
    const int s = s0 + threadIdx.x;
    const int32_t v = s < k ? irow[s] : -1;
    const bool valid = v >= 0 && v < n_pools;
    const uint64_t ballot = __ballot(valid);
    const int before = __popcll(ballot & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tmp[wid] = __popcll(ballot);
    __syncthreads();
    int off = base;
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wave_tmp[w];
      if (w < wid) off += c;
      tot += c;
    }
    if (valid) sel[off + before] = v;
    base += tot;
    __syncthreads();
  }
  return base;
}

// Gather of one tile of 32 selected rows into LDS, laid out [16-byte chunk c][key]: chunks
// [0, DQK/8) are the key row, then (separate V only) DV/8 chunks of the value row.  Thread t
// loads key t % 32, chunk columns t / 32 + 8 i, into registers (load), then writes them to
// LDS (store), so the next tile's loads can be in flight while the current one is used.
template <int DQK, int DV, bool SEPARATE_V>
struct TileGather {
  static constexpr int kChunksQK = DQK / 8;
  static constexpr int kChunksRow = kChunksQK + (SEPARATE_V ? DV / 8 : 0);
  static constexpr int kTileChunks = kChunksRow * kKeysPerTile;
  static constexpr int kTileBytes = kTileChunks * 16;
  static constexpr int kVBase = SEPARATE_V ? kChunksQK : 0;  // first chunk of V in a row
  static constexpr int kColStep = kAttnThreads / kKeysPerTile;
  static constexpr int kPerThread = (kTileChunks + kAttnThreads - 1) / kAttnThreads;
  u32x4 pre[kPerThread];

  __device__ __forceinline__ void load(int t, const int32_t* sel, int n_valid,
                                       const uint16_t* __restrict__ kv, int64_t ld_kv,
                                       const uint16_t* __restrict__ v, int64_t ld_v) {
    const int tid = threadIdx.x;
    const int slot = t * kKeysPerTile + (tid & (kKeysPerTile - 1));
    const int32_t p = slot < n_valid ? sel[slot] : -1;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      u32x4 val = {0u, 0u, 0u, 0u};
      const int c = (tid >> 5) + i * kColStep;
      if (c < kChunksRow && p >= 0) {
        const uint16_t* src = (!SEPARATE_V || c < kChunksQK)
                                  ? kv + static_cast<int64_t>(p) * ld_kv + c * 8
                                  : v + static_cast<int64_t>(p) * ld_v + (c - kChunksQK) * 8;
        val = *reinterpret_cast<const u32x4*>(src);
      }
      pre[i] = val;
    }
  }

  __device__ __forceinline__ void store(uint8_t* tile) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = (tid >> 5) + i * kColStep;
      if (c < kChunksRow)
        *reinterpret_cast<u32x4*>(&tile[(c * kKeysPerTile + (tid & (kKeysPerTile - 1))) * 16]) =
            pre[i];
    }
  }
};

// Byte offset in a tile of the 16-byte chunk holding columns [8c, 8c + 8) of tile key `key`.
__device__ __forceinline__ int tile_off(int c, int key) { return (c * kKeysPerTile + key) * 16; }

// MFMA operand "X^T" for columns [16 nb, 16 nb + 16) of a tile, contraction over the tile's
// 32 keys: lane (g, r) gets X[key][16 nb + r] for keys 4g + e (slots 0..3) and 16 + 4g + e
// (slots 4..7), the slot order in which an S^T accumulator holds its probabilities.
// `cbase` is the first chunk of X in a tile row.
__device__ __forceinline__ bf16x8 tile_cols_transposed(const uint8_t* tile, int cbase, int nb,
                                                       int g, int r16) {
  const int key = 4 * g + (r16 >> 2);
  const int col = nb * 16 + 4 * (r16 & 3);
  const int c = cbase + (col >> 3);
  const int byte = (col & 7) * 2;
  const i16x4 lo = lds_read_tr16(&tile[tile_off(c, key) + byte]);
  const i16x4 hi = lds_read_tr16(&tile[tile_off(c, 16 + key) + byte]);
  return join_tr(lo, hi);
}

}  // namespace dsa
