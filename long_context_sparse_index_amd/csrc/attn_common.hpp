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
// Thread i takes the m = ceil(k / threads) consecutive slots [i m, i m + m), all loaded in
// one memory round trip; a block prefix sum over the per-thread counts places them.  When
// slot_of is given, slot_of[j] receives the original slot of compacted entry j.
__device__ inline int compact_selection(const int32_t* __restrict__ irow, int k,
                                        int64_t n_pools, int32_t* sel, int* wave_tmp,
                                        int16_t* slot_of = nullptr) {
  constexpr int kMaxPer = kMaxTopK / kAttnThreads;
  constexpr int kWaves = kAttnThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int m = (k + kAttnThreads - 1) / kAttnThreads;
  const int s0 = threadIdx.x * m;
  int32_t v[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) v[i] = (i < m && s0 + i < k) ? irow[s0 + i] : -1;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) cnt += (v[i] >= 0 && v[i] < n_pools) ? 1 : 0;
  int incl = cnt;  // inclusive prefix over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tmp[wid] = incl;
  __syncthreads();
  int off = incl - cnt;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = wave_tmp[w];
    if (w < wid) off += c;
    total += c;
  }
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i)
    if (v[i] >= 0 && v[i] < n_pools) {
      if (slot_of) slot_of[off] = static_cast<int16_t>(s0 + i);
      sel[off++] = v[i];
    }
  __syncthreads();
  return total;
}

// Waits until at most `n` vector-memory operations of this wave are outstanding (n < 64).
#define DSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

// Waits until this wave's LDS operations (ds_read / ds_write) have completed.
#define DSA_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Deepest tile pipeline (<= 3 stages) whose LDS fits next to `other_bytes` of LDS.
constexpr int pick_depth(int tile_bytes, int other_bytes) {
  return 3 * tile_bytes + other_bytes <= 160 * 1024 - 256   ? 3
         : 2 * tile_bytes + other_bytes <= 160 * 1024 - 256 ? 2
                                                            : 1;
}

// Workgroup barrier that is also a compiler barrier for memory operations but does not
// wait for outstanding vector-memory operations (the tile pipeline below waits for exactly
// the loads it needs with DSA_WAIT_VMCNT).  LDS writes made with ds_write must be waited
// for (lgkmcnt) by the caller before it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One asynchronous 16-byte-per-lane global -> LDS load: lane l's 16 bytes at `src` land at
// LDS byte address lds_addr + 16 l (lds_addr wave-uniform).  Written as inline assembly so
// that the compiler's wait insertion does not treat it as an LDS store and drain every
// outstanding load before the next LDS read; the tile pipeline below waits for exactly
// the loads it needs (the compiler's own waits only count more operations, never fewer).
__device__ __forceinline__ void dma_16b(const void* src, uint32_t lds_addr) {
  // m0 (the LDS base of the load) is an input operand, so the compiler sets it and knows
  // it is in use.
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr) : "memory");
}


// Asynchronous gather of tiles of 32 selected rows straight into LDS (global_load_lds,
// 16 bytes per lane), `DEPTH` tiles deep.  A tile is laid out [16-byte chunk c][key]:
// chunks [0, DQK/8) are the key row, then (separate V only) DV/8 chunks of the value row.
// One load instruction fills 1 KB of LDS (64 lanes x 16 bytes) = chunk columns 2j, 2j+1 of
// all 32 keys; the tile's instructions are split evenly over the 4 waves.  Keys past the
// last valid slot repeat the last valid row (their probabilities are masked to zero).
template <int DQK, int DV, bool SEPARATE_V, int DEPTH>
struct TileDma {
  static constexpr int kChunksQK = DQK / 8;
  static constexpr int kChunksRow = kChunksQK + (SEPARATE_V ? DV / 8 : 0);
  static constexpr int kTileBytes = kChunksRow * kKeysPerTile * 16;
  static constexpr int kVBase = SEPARATE_V ? kChunksQK : 0;  // first chunk of V in a row
  static constexpr int kInstr = kChunksRow / 2;
  static constexpr int kPerWave = kInstr / (kAttnThreads / 64);
  static constexpr int kLdsBytes = DEPTH * kTileBytes;
  static_assert(kChunksRow % 2 == 0 && kInstr % (kAttnThreads / 64) == 0, "tile split");
  static_assert(DEPTH >= 1 && DEPTH <= 3 && kPerWave * (DEPTH - 1) < 64, "vmcnt range");

  // The table row this lane gathers for tile t (keys past the last valid slot repeat the
  // last valid row).
  __device__ __forceinline__ static int32_t row_of(int t, const int32_t* sel, int n_valid) {
    int slot = t * kKeysPerTile + (threadIdx.x & (kKeysPerTile - 1));
    slot = slot < n_valid ? slot : n_valid - 1;
    return sel[slot];
  }

  // Issues the loads of tile t into stage `stage` of `tiles`.
  __device__ __forceinline__ static void issue(uint8_t* tiles, int stage, int t,
                                               const int32_t* sel, int n_valid,
                                               const uint16_t* __restrict__ kv, int64_t ld_kv,
                                               const uint16_t* __restrict__ v, int64_t ld_v) {
    issue_row(tiles, stage, row_of(t, sel, n_valid), kv, ld_kv, v, ld_v);
  }

  // Issues the loads of the tile whose rows (one per lane, see row_of) are `p` into stage
  // `stage` of `tiles`.
  __device__ __forceinline__ static void issue_row(uint8_t* tiles, int stage, int64_t p,
                                                   const uint16_t* __restrict__ kv,
                                                   int64_t ld_kv,
                                                   const uint16_t* __restrict__ v,
                                                   int64_t ld_v) {
    const int lane = threadIdx.x & 63;
    // Wave-uniform: keeps the LDS destinations (M0) in scalar registers.
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t base = lds_addr_of(tiles) + stage * kTileBytes;
    if constexpr (!SEPARATE_V) {
      // One row pointer; the wave's loads are at constant column offsets from it.
      const uint16_t* rowp = kv + p * ld_kv + (2 * wid * kPerWave + (lane >> 5)) * 8;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i)
        dma_16b(rowp + i * 16, base + (wid * kPerWave + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int j = wid * kPerWave + i;
        const int c = 2 * j + (lane >> 5);
        const uint16_t* src =
            c < kChunksQK ? kv + p * ld_kv + c * 8 : v + p * ld_v + (c - kChunksQK) * 8;
        dma_16b(src, base + j * 1024);
      }
    }
  }

  // Waits until at most N (at most 63) vector-memory operations of this wave are pending.
  template <int N>
  __device__ __forceinline__ static void wait_at_most() {
    DSA_WAIT_VMCNT(N < 63 ? N : 63);
  }

  // Runs body(tile, t) for every tile t in order with DEPTH - 1 tiles prefetched; `tile` is
  // an LDS pointer to the tile.
  // All threads of the block must call it (it contains barriers).  kBodyOps: the number of
  // vector-memory operations (e.g. stores) every call of body issues in each wave, exactly;
  // those issued after a tile's loads are allowed to stay in flight while the pipeline waits
  // for that tile (vector-memory operations complete in issue order for the wait counter).
  template <int kBodyOps = 0, class Body>
  __device__ __forceinline__ static void for_each_tile(uint8_t* tiles, int n_tiles,
                                                       const int32_t* sel, int n_valid,
                                                       const uint16_t* __restrict__ kv,
                                                       int64_t ld_kv,
                                                       const uint16_t* __restrict__ v,
                                                       int64_t ld_v, Body&& body) {
    if constexpr (DEPTH == 1) {
      for (int t = 0; t < n_tiles; ++t) {
        tile_barrier();  // the previous tile is consumed
        issue(tiles, 0, t, sel, n_valid, kv, ld_kv, v, ld_v);
        DSA_WAIT_VMCNT(0);
        tile_barrier();
        body(lds_ptr_of(tiles), t);
      }
    } else {
      for (int s = 0; s < DEPTH - 1 && s < n_tiles; ++s)
        issue(tiles, s, s, sel, n_valid, kv, ld_kv, v, ld_v);
      for (int t = 0; t < n_tiles; ++t) {
        // Operations issued after tile t's loads: with DEPTH 3, tile t + 1's loads (issued at
        // iteration t - 1, if that tile exists) and the bodies of tiles t - 2 and t - 1; with
        // DEPTH 2, the body of tile t - 1.  (The memory clobber keeps the previous body's
        // stores ahead of the wait, where the count assumes them.)
        asm volatile("" ::: "memory");
        if constexpr (DEPTH == 2) {
          if (t == 0)
            wait_at_most<0>();
          else
            wait_at_most<kBodyOps>();
        } else {
          const bool next = t + 1 < n_tiles;
          if (t == 0) {
            if (next) wait_at_most<kPerWave>(); else wait_at_most<0>();
          } else if (t == 1) {
            if (next) wait_at_most<kPerWave + kBodyOps>(); else wait_at_most<kBodyOps>();
          } else {
            if (next) wait_at_most<kPerWave + 2 * kBodyOps>(); else wait_at_most<2 * kBodyOps>();
          }
        }
        tile_barrier();  // tile t is in LDS for every wave; tile t-1 is consumed
        if (t + DEPTH - 1 < n_tiles)
          issue(tiles, (t + DEPTH - 1) % DEPTH, t + DEPTH - 1, sel, n_valid, kv, ld_kv, v,
                ld_v);
        body(lds_ptr_of(tiles) + (t % DEPTH) * kTileBytes, t);
      }
    }
  }
};

// Gather of 32 selected rows in 128-byte bands: wave w loads the rows of tile keys
// 8w .. 8w + 7 (lane l: key 8w + l / 8), one load per 128-byte band of the row, so each load
// instruction covers 8 rows x 128 contiguous bytes (eight whole cache lines of the 1152-byte
// latent rows) instead of 32 rows x 32 bytes.  Layout of a tile:
//   [key / 8][band][key % 8][position] x 16 bytes, chunk c of a band at position
//   (c % 8) ^ swz(key), swz(key) = 2 ((key >> 1) % 4) + (key >> 3) % 2.
// Rows key and key + 1 sit 128 bytes apart, i.e. in the two halves of the 256-byte window of
// the 64 LDS banks, and the swizzle takes the 8 even (or odd) keys of an aligned 16 onto 8
// distinct 16-byte positions: the 16 keys of a key-row operand load (one chunk each) hit 16
// distinct slots.  The transposed value reads take two adjacent chunks (32 bytes) of each of
// 8 consecutive keys per 256 bytes of data; their swizzles differ in bits 1-2 among the 4
// even (or odd) keys of an aligned 8, so the chunk pairs are disjoint and those reads are
// conflict-free too (with (key >> 1) & 7 keys k and k + 2 shared a pair: two-way conflicts).
// DEPTH tiles are staged (see TileDma for the waits).
template <int DQK, int DV, bool SEPARATE_V, int DEPTH>
struct TileDmaBands {
  static constexpr int kChunksQK = DQK / 8;
  static constexpr int kChunksRow = kChunksQK + (SEPARATE_V ? DV / 8 : 0);
  static constexpr int kBands = kChunksRow / 8;
  static constexpr int kTileBytes = kChunksRow * kKeysPerTile * 16;
  static constexpr int kGroupBytes = kBands * 1024;  // one key group of 8 rows
  static constexpr int kVChunk = SEPARATE_V ? kChunksQK : 0;  // first chunk of V in a row
  static constexpr int kPerWave = kBands;
  static constexpr int kLdsBytes = DEPTH * kTileBytes;
  static_assert(kChunksRow % 8 == 0 && kChunksQK % 8 == 0, "whole bands");
  static_assert(kAttnThreads == 256, "four waves of 8 keys");
  static_assert(DEPTH >= 1 && DEPTH <= 3 && kPerWave * (DEPTH - 1) < 64, "vmcnt range");

  __device__ __forceinline__ static int swz(int key) {
    return (((key >> 1) & 3) << 1) | ((key >> 3) & 1);
  }

  // Byte offset in a tile of chunk `c` (columns [8c, 8c + 8)) of tile key `key`.
  __device__ __forceinline__ static int offset(int key, int c) {
    return (key >> 3) * kGroupBytes + (c >> 3) * 1024 + (key & 7) * 128 +
           (((c & 7) ^ swz(key)) << 4);
  }

  // The table row this lane gathers for tile t (keys past the last valid slot repeat the
  // last valid row).
  __device__ __forceinline__ static int32_t row_of(int t, const int32_t* sel, int n_valid) {
    const int key = 8 * (threadIdx.x >> 6) + ((threadIdx.x & 63) >> 3);
    int slot = t * kKeysPerTile + key;
    slot = slot < n_valid ? slot : n_valid - 1;
    return sel[slot];
  }

  // Issues the load of band `b` (columns [64 b, 64 b + 64) of the row) of the tile whose row
  // for this lane is `p` into stage `stage`: one instruction, 1 KB of LDS per wave.
  __device__ __forceinline__ static void issue_band(uint8_t* tiles, int stage, int64_t p, int b,
                                                    const uint16_t* __restrict__ kv,
                                                    int64_t ld_kv,
                                                    const uint16_t* __restrict__ v,
                                                    int64_t ld_v) {
    const int lane = threadIdx.x & 63;
    // Wave-uniform: keeps the LDS destinations (M0) in scalar registers.
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int key = 8 * wid + (lane >> 3);
    const int pos = (lane & 7) ^ swz(key);  // chunk of each band this lane loads
    const uint32_t base = lds_addr_of(tiles) + stage * kTileBytes + wid * kGroupBytes;
    const int c = 8 * b + pos;
    const uint16_t* src;
    if constexpr (!SEPARATE_V)
      src = kv + p * ld_kv + c * 8;
    else
      src = c < kChunksQK ? kv + p * ld_kv + c * 8 : v + p * ld_v + (c - kChunksQK) * 8;
    dma_16b(src, base + b * 1024);
  }

  // Issues all loads of the tile whose row for this lane is `p` into stage `stage`.
  __device__ __forceinline__ static void issue_row(uint8_t* tiles, int stage, int64_t p,
                                                   const uint16_t* __restrict__ kv,
                                                   int64_t ld_kv,
                                                   const uint16_t* __restrict__ v,
                                                   int64_t ld_v) {
#pragma unroll
    for (int b = 0; b < kBands; ++b) issue_band(tiles, stage, p, b, kv, ld_kv, v, ld_v);
  }

  __device__ __forceinline__ static void issue(uint8_t* tiles, int stage, int t,
                                               const int32_t* sel, int n_valid,
                                               const uint16_t* __restrict__ kv, int64_t ld_kv,
                                               const uint16_t* __restrict__ v, int64_t ld_v) {
    issue_row(tiles, stage, row_of(t, sel, n_valid), kv, ld_kv, v, ld_v);
  }
};

// Byte offset in a tile of the 16-byte chunk holding columns [8c, 8c + 8) of tile key `key`.
__device__ __forceinline__ int tile_off(int c, int key) { return (c * kKeysPerTile + key) * 16; }

// Lane part of the LDS address of a transposed tile operand (see tile_tr_block):
// the operand for column block nb is then at offset nb * 1024 (keys 4g + e) and
// nb * 1024 + 256 (keys 16 + 4g + e), so one base address serves every block.
__device__ __forceinline__ int tile_tr_lane_off(int cbase, int g, int r16) {
  const int key = 4 * g + (r16 >> 2);
  return tile_off(cbase + ((r16 & 3) >> 1), key) + (r16 & 1) * 8;
}

__device__ __forceinline__ bf16x8 tile_tr_block(lds_ptr lane_base, int nb) {
  const i16x4 lo = lds_read_tr16_at(lane_base + nb * 1024);
  const i16x4 hi = lds_read_tr16_at(lane_base + nb * 1024 + 16 * 16);
  return join_tr(lo, hi);
}

}  // namespace dsa
