// Sparse MQA attention forward over the selected pooled KV rows, on gfx950 MFMA.
//
// Page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens", section "Model and
// bottleneck": attention reads only about 2048 selected entries per query; section "Four
// optimizations", item 1: the kernel works on DeepSeek-V3.2-shaped tensors, where all query
// heads share one 576-wide latent KV row whose first 512 columns are the value.
//
// One block per query token, one wave per 16 query heads.  Because the heads share the KV
// row, each gathered tile of 32 selected rows is an MFMA operand for all heads at once:
//   S^T[key, head] = K_tile . Q^T   (A: key rows from LDS, B: the wave's queries, held in
//                                    registers for the whole row of selections)
//   O^T[dim, head] += V_tile^T . P^T
// Computing the transposed products puts one head in each lane column, so the running max,
// the running sum and the output rescale of the online softmax stay in the lane (two
// cross-group shuffles per tile for the max), and the probabilities come out of the S^T
// accumulator already in the B-operand layout of the P.V product.  V^T is read from the
// same row-major LDS tile with the LDS transpose read, so V costs no second gather or copy.
// The selection row is first compacted in LDS (valid slots in slot order), so tiles of
// empty (-1) slots are never visited; only the last tile can be partial.  Tiles are
// gathered with asynchronous global->LDS loads, up to three tiles deep, so the gather of
// the next tiles overlaps the MFMA work on the current one without staging registers.
//
// LDS tile layout: [16-byte column chunk c][key] so that both the key-row reads for S^T and
// the transposed value reads touch contiguous 256-byte spans.

#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

// Largest log2 excess of a logit over the softmax reference that the fp32/bf16 arithmetic
// of the P.V product tolerates (probabilities up to 2^64, sums far below fp32 overflow).
constexpr float kRefHeadroomLog2 = 64.0f;

// Rows with fewer valid slots than this feed the P.V product each probability as a bf16
// pair hi + lo (about 16 significant bits); rows with more feed one bf16 (8 bits, half the
// P.V MFMAs).  The rounding of p to bf16 is a relative error of at most 2^-8 per key, random
// in sign, so O of a row with c keys carries a relative error of about 1.6e-3 of its own
// magnitude, which is about sqrt(e / c) for N(0, 1) logits: at c >= 512 that stays far
// inside 2e-2 of the RMS of O over any set of rows (whose RMS is at least that of the
// many-key rows); rows with few keys (|O| up to the size of one value row) need the pair.
constexpr int kSplitBelow = 512;

template <int DQK, int DV, bool SEPARATE_V, bool OUT_F32>
__global__ __launch_bounds__(kAttnThreads) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t ld_kv,
    const uint16_t* __restrict__ v, int64_t ld_v, const int32_t* __restrict__ idx, int k,
    void* __restrict__ o, float* __restrict__ lse, int64_t n_pools, int h,
    float scale_log2) {
  constexpr int kTileBytes = TileDma<DQK, DV, SEPARATE_V, 1>::kTileBytes;
  using Dma = TileDma<DQK, DV, SEPARATE_V, pick_depth(kTileBytes, kMaxTopK * 4 + 64)>;
  constexpr int kKS = DQK / 32;  // MFMA steps of q . k
  constexpr int kNB = DV / 16;   // 16-dim output blocks
  static_assert(DQK % 32 == 0 && DV % 16 == 0, "tile shapes");

  __shared__ __attribute__((aligned(16))) uint8_t tiles[Dma::kLdsBytes];
  __shared__ int32_t sel[kMaxTopK];
  __shared__ int wave_tmp[kAttnThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t row = blockIdx.x;
  const int head = wid * 16 + r16;
  const bool head_ok = head < h;
  const bool wave_has_heads = wid * 16 < h;

  const int n_valid = compact_selection(idx + row * k, k, n_pools, sel, wave_tmp);

  // The wave's queries as B operands: lane column = head, 8 contraction values per group.
  bf16x8 qf[kKS];
  {
    const uint16_t* qrow = q + (row * h + (head_ok ? head : 0)) * DQK + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[ks] = head_ok ? *reinterpret_cast<const bf16x8*>(qrow + ks * 32) : bf16x8_zero();
  }
  // Land the operand loads before the tile pipeline starts: the pipeline's own waits count
  // only its tile loads, and an operand load still pending inside the loop would make the
  // compiler wait for every outstanding load there.
  DSA_WAIT_VMCNT(0);

  // Softmax reference per head (log2 domain): the first tile's maximum.  O = sum p V / sum p
  // does not depend on the reference, so no accumulator is ever rescaled in the loop; a
  // logit more than 2^64 above the reference (fp32 headroom) raises `overflow` and the
  // token is redone after an exact max pass.
  f32x4 oacc[kNB];
  float m_ref = -__builtin_inff();
  float l_run = 0.0f;
  bool overflow = false;
  const int n_tiles = (n_valid + kKeysPerTile - 1) / kKeysPerTile;

  // S^T = K . Q^T for the 32 keys of a tile (two 16-key row blocks), in log2 units, with
  // slots past the last valid one at -inf; also returns the tile max of the lane's head.
  auto tile_logits = [&](lds_ptr tile, int t, f32x8& x) {
    // Key rows 16 mb + r of chunk column 4 ks + g.  Four independent accumulation chains
    // (row block x parity of ks) keep back-to-back MFMAs free of dependences.
    const lds_ptr k_base0 = tile + tile_off(g, r16);
    const lds_ptr k_base1 = tile + tile_off(g, 16 + r16);
    f32x4 s[2][2] = {};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      s[0][ks & 1] = mfma16x16x32_bf16(lds_load_bf16x8(k_base0 + ks * 2048), qf[ks], s[0][ks & 1]);
      s[1][ks & 1] = mfma16x16x32_bf16(lds_load_bf16x8(k_base1 + ks * 2048), qf[ks], s[1][ks & 1]);
    }
    const int slot0 = t * kKeysPerTile;
    float mt = -__builtin_inff();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = slot0 + mb * 16 + g * 4 + i < n_valid;
        x[mb * 4 + i] = ok ? (s[mb][0][i] + s[mb][1][i]) * scale_log2 : -__builtin_inff();
        mt = __builtin_fmaxf(mt, x[mb * 4 + i]);
      }
    mt = __builtin_fmaxf(mt, shfl_xor(mt, 16));
    return __builtin_fmaxf(mt, shfl_xor(mt, 32));
  };

  // One pass of P.V over all tiles against the reference m_ref (taken from tile 0 when
  // `ref_from_first` is set).
  auto pv_pass = [&](bool ref_from_first) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.0f;
    Dma::for_each_tile(tiles, n_tiles, sel, n_valid, kv, ld_kv, v, ld_v,
                       [&](lds_ptr tile, int t) {
      if (!wave_has_heads) return;
      f32x8 x;
      const float mt = tile_logits(tile, t, x);
      if (ref_from_first && t == 0) m_ref = mt;
      overflow |= mt > m_ref + kRefHeadroomLog2;
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_exp2f(x[e] - m_ref);
      l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // Each probability goes to the MFMA as a bf16 pair hi + lo, so the P.V product sees
      // p to about 16 significant bits instead of 8.
      bf16x8 pf_hi, pf_lo;
      split_bf16x8(p, pf_hi, pf_lo);
      // O^T += V^T . P^T, contraction over the tile's keys in the S^T slot order.
      const lds_ptr vt_base = tile + tile_tr_lane_off(Dma::kVBase, g, r16);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const bf16x8 vt = tile_tr_block(vt_base, nb);
        oacc[nb] = mfma16x16x32_bf16(vt, pf_hi, oacc[nb]);
        oacc[nb] = mfma16x16x32_bf16(vt, pf_lo, oacc[nb]);
      }
    });
  };

  pv_pass(true);
  if (__syncthreads_or(overflow)) {
    // Rare: some logit far above the first tile's maximum.  Take the exact maximum first.
    m_ref = -__builtin_inff();
    Dma::for_each_tile(tiles, n_tiles, sel, n_valid, kv, ld_kv, v, ld_v,
                       [&](lds_ptr tile, int t) {
      if (!wave_has_heads) return;
      f32x8 x;
      m_ref = __builtin_fmaxf(m_ref, tile_logits(tile, t, x));
    });
    pv_pass(false);
  }
  const float m_run = m_ref;

  // Finish: combine the four lane groups' partial sums of each head.
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  if (!head_ok) return;
  const float inv = n_valid > 0 ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int dim = nb * 16 + 4 * g;
    if constexpr (OUT_F32) {
      float* orow = static_cast<float*>(o) + (row * h + head) * DV;
      *reinterpret_cast<f32x4*>(orow + dim) = oacc[nb] * inv;
    } else {
      uint16_t* orow = static_cast<uint16_t*>(o) + (row * h + head) * DV;
      const uint32_t w0 = static_cast<uint32_t>(float_to_bf16_bits(oacc[nb][0] * inv)) |
                          (static_cast<uint32_t>(float_to_bf16_bits(oacc[nb][1] * inv)) << 16);
      const uint32_t w1 = static_cast<uint32_t>(float_to_bf16_bits(oacc[nb][2] * inv)) |
                          (static_cast<uint32_t>(float_to_bf16_bits(oacc[nb][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + dim) = make_uint2(w0, w1);
    }
  }
  if (g == 0)
    lse[row * h + head] =
        n_valid > 0 ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------------------------------
// Head-pair kernel, used wherever three tiles fit in LDS next to its exchange buffers.
//
// The kernel above makes every wave read the whole tile (its keys for S^T, its values for
// O^T) for 16 heads and run the softmax of 16 heads x 32 keys per tile.  Here wave
// w = (head half hh = w / 2, half kh = w % 2) serves 32 heads (two 16-head groups):
//   * it computes the logits of both head groups for the 16 keys 16 kh .. 16 kh + 15 of
//     each tile (full contraction; one key fragment read feeds both head groups) and their
//     probabilities.  In the B-operand layout of the P.V product those 16 keys are exactly
//     slots 4 kh .. 4 kh + 3 of every lane, so the two waves of a pair each write their
//     half of the 16-byte operand into one shared LDS slot per lane and read back the
//     whole operand after the tile barrier;
//   * it accumulates O^T of the 32 heads over value-column half kh, so each transpose
//     read of V feeds four MFMAs (two head groups x the hi/lo halves of P), or two on rows
//     with at least kSplitBelow valid slots, whose P is one bf16 value.
// Per tile and block this halves the transpose reads and the key reads of the kernel
// above, and no softmax work is done twice.  The pair shares one softmax reference per
// head (the maximum of tile 0 over both key halves, exchanged once per pass) and adds its
// two partial row sums at the end.  Loop body for tile t: logits and probabilities of
// tile t + 1 and the whole P.V product of tile t (all independent, so the MFMA work of one
// overlaps the vector work of the other), then one barrier, at which tile t is consumed,
// the probabilities of tile t + 1 are exchanged and the tile two ahead has landed; the
// load of the tile three ahead then reuses tile t's buffer.

constexpr int kPairXchgBytes = 2 * 2 * 2 * 2 * 64 * 16;  // [buf][hh][hg][hi/lo][lane] x 16 B
constexpr int kPairRedBytes = 4 * 64 * 8;                 // [wave][lane] x 2 floats

template <int DQK, int DV, bool SEPARATE_V>
constexpr bool pair_fits() {
  return 3 * TileDma<DQK, DV, SEPARATE_V, 1>::kTileBytes + kPairXchgBytes + kPairRedBytes +
             kMaxTopK * 4 + 64 <=
         160 * 1024;
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;

template <int DQK, int DV, bool SEPARATE_V, bool OUT_F32>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t ld_kv,
    const uint16_t* __restrict__ v, int64_t ld_v, const int32_t* __restrict__ idx, int k,
    void* __restrict__ o, float* __restrict__ lse, int64_t n_pools, int h,
    float scale_log2) {
  using Dma = TileDmaBands<DQK, DV, SEPARATE_V, 3>;
  constexpr int kKS = DQK / 32;   // q . k MFMA steps
  constexpr int kNBH = DV / 32;   // 16-column output blocks per value half
  static_assert(DQK % 64 == 0 && DV % 32 == 0, "tile shapes");
  static_assert(pair_fits<DQK, DV, SEPARATE_V>(), "LDS budget");
  // P.V blocks of the current tile done in phase 1 of the loop body (next to the next tile's
  // logits); the rest go to phase 2, where they cover the softmax.  With 576/512 rows that
  // is 9 of the 16 blocks in phase 1 and 7 beside the softmax.
  constexpr int kPvPhase1 = 9;
  constexpr int kN1 = kPvPhase1 < kKS / 2 ? kPvPhase1 : kKS / 2;
  // With one bf16 per probability a block is two MFMAs: phase 1 takes one block per slot for
  // its first kPvPhase1Single slots, phase 2 the rest beside the softmax (12 of 16 blocks
  // with 576/512 rows: 2.79-2.88 ms per 8192-row 128k chunk on MI355X against 2.81-2.91
  // with 9, 2.86-2.91 with 16 and 2.90-2.99 with 6).
  constexpr int kPvPhase1Single = 12;

  __shared__ __attribute__((aligned(16))) uint8_t tiles[Dma::kLdsBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pxchg[kPairXchgBytes];
  __shared__ __attribute__((aligned(16))) f32x2 red[kPairRedBytes / 8];
  __shared__ int32_t sel[kMaxTopK];
  __shared__ int wave_tmp[kAttnThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = wid >> 1;
  const int kh = wid & 1;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t row = blockIdx.x;
  const bool compute = hh * 32 < h;  // wave-uniform; waves without heads only gather

  // Queries of the two head groups as B operands (lane column = head), loaded before the
  // selection row so that both loads share one memory round trip.
  bf16x8 qf[2][kKS];
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    const int head = hh * 32 + hg * 16 + r16;
    const bool ok = head < h;
    const uint16_t* qrow = q + (row * h + (ok ? head : 0)) * DQK + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[hg][ks] = ok ? *reinterpret_cast<const bf16x8*>(qrow + ks * 32) : bf16x8_zero();
  }
  const int n_valid = compact_selection(idx + row * k, k, n_pools, sel, wave_tmp);
  const int n_tiles = (n_valid + kKeysPerTile - 1) / kKeysPerTile;
  DSA_WAIT_VMCNT(0);  // the tile pipeline's waits count only tile loads

  f32x4 oacc[2][kNBH];
#pragma unroll
  for (int hg = 0; hg < 2; ++hg)
#pragma unroll
    for (int nb = 0; nb < kNBH; ++nb) oacc[hg][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_tot[2] = {0.f, 0.f};
  bool overflow = false;

  const uint32_t tiles_a = lds_addr_of(tiles);
  // Lane offsets in a tile.  Logits: key 16 kh + r, chunk 4 ks + g, i.e. band ks / 2 and
  // in-band chunk 4 (ks % 2) + g: one base for even and one for odd ks.  Transposed value
  // block nb of value half kh (columns 16 nb ..): lane i of group g reads key 4 g + i / 4,
  // chunk 2 nb + (i % 4) / 2, half i % 2; band nb / 4, in-band chunk 2 (nb % 4) + ..., so one
  // base per nb % 4; the keys 16 .. 31 of the second read sit two key groups further.
  const int k_lane[2] = {Dma::offset(16 * kh + r16, g), Dma::offset(16 * kh + r16, 4 + g)};
  int v_lane[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int key = 4 * g + (r16 >> 2);
    v_lane[m] = Dma::offset(key, Dma::kVChunk + 2 * kh * kNBH + 2 * m + ((r16 & 3) >> 1)) +
                (r16 & 1) * 8;
  }
  constexpr int kVHi = 2 * Dma::kGroupBytes;  // keys 16 + k vs k
  // Transposed V operand of block nb (relative to value half kh) from the four bases.
  auto vt_block = [&](const lds_ptr (&vb)[4], int nb) {
    const lds_ptr lo = vb[nb & 3] + (nb >> 2) * 1024;
    return join_tr(lds_read_tr16_at(lo), lds_read_tr16_at(lo + kVHi));
  };
  // Stage base plus lane offset as one opaque register, so that the constant offsets of
  // the individual reads fold into the LDS instructions.
  auto pinned = [&](int st, int lane_off) {
    uint32_t a = tiles_a + st * Dma::kTileBytes + lane_off;
    asm("" : "+v"(a));
    return (lds_ptr)(uintptr_t)(a);
  };
  // Probability exchange slot of (buffer, head group, hi/lo): 16 bytes per lane, of which
  // this wave owns bytes [8 kh, 8 kh + 8).
  auto pslot = [&](int buf, int hg, int hl) {
    return reinterpret_cast<__attribute__((address_space(3))) char*>(lds_addr_of(pxchg)) +
           ((((buf * 2 + hh) * 2 + hg) * 2 + hl) * 64 + lane) * 16;
  };
  lds_f32x2* const red_own = (lds_f32x2*)(lds_addr_of(red)) + wid * 64 + lane;
  lds_f32x2* const red_partner = (lds_f32x2*)(lds_addr_of(red)) + (wid ^ 1) * 64 + lane;

  // S^T of this wave's 16 keys of a tile for both head groups; two accumulation chains per
  // head group (even / odd contraction steps).
  auto logits = [&](int st, f32x4 (&s)[2][2]) {
    const lds_ptr kb[2] = {pinned(st, k_lane[0]), pinned(st, k_lane[1])};
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) s[hg][0] = s[hg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const bf16x8 a = lds_load_bf16x8(kb[ks & 1] + (ks >> 1) * 1024);
      s[0][ks & 1] = mfma16x16x32_bf16(a, qf[0][ks], s[0][ks & 1]);
      s[1][ks & 1] = mfma16x16x32_bf16(a, qf[1][ks], s[1][ks & 1]);
    }
  };
  // y = x - m with x = logit * log2(e) * scale rounded to fp32, for this lane's keys
  // 16 kh + 4 g + i of tile t (-inf past the last valid slot).  Rounding x before the
  // subtraction (the select between them keeps the two from being fused) makes y exactly
  // 0 for the key that defines the reference.
  auto shifted = [&](const f32x4 (&s)[2][2], int t, const float (&m)[2], f32x4 (&y)[2]) {
    const int slot0 = t * kKeysPerTile + 16 * kh + 4 * g;
#pragma unroll
    for (int hg = 0; hg < 2; ++hg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x =
            slot0 + i < n_valid ? (s[hg][0][i] + s[hg][1][i]) * scale_log2 : -__builtin_inff();
        y[hg][i] = x - m[hg];
      }
  };
  auto max4 = [](const f32x4& y) {
    return __builtin_fmaxf(__builtin_fmaxf(y[0], y[1]), __builtin_fmaxf(y[2], y[3]));
  };
  auto head_max = [](float m) {
    m = __builtin_fmaxf(m, shfl_xor(m, 16));
    return __builtin_fmaxf(m, shfl_xor(m, 32));
  };
  auto head_sum = [](float l) {
    l += shfl_xor(l, 16);
    return l + shfl_xor(l, 32);
  };
  // Probabilities p = 2^y of this wave's keys, summed into l_run, and written as bf16
  // hi + lo pairs into this wave's half of the exchange slots.
  // (SPLIT: the bf16 pair hi + lo; otherwise hi only.)
  auto probabilities = [&](const f32x4 (&y)[2], int buf, float (&l_run)[2], float (&ymax)[2],
                           auto split) {
    constexpr bool SPLIT = decltype(split)::value;
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) {
      ymax[hg] = __builtin_fmaxf(ymax[hg], max4(y[hg]));
      f32x4 p;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(y[hg][i]);
      l_run[hg] += (p[0] + p[1]) + (p[2] + p[3]);
      const bf16x4 hi = __builtin_convertvector(p, bf16x4);
      *(lds_i16x4*)(pslot(buf, hg, 0) + 8 * kh) = __builtin_bit_cast(i16x4, hi);
      if constexpr (SPLIT) {
        const bf16x4 lo =
            __builtin_convertvector(p - __builtin_convertvector(hi, f32x4), bf16x4);
        *(lds_i16x4*)(pslot(buf, hg, 1) + 8 * kh) = __builtin_bit_cast(i16x4, lo);
      }
    }
  };
  auto read_probabilities = [&](int buf, bf16x8 (&phi)[2], bf16x8 (&plo)[2], auto split) {
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) {
      phi[hg] = lds_load_bf16x8((lds_ptr)pslot(buf, hg, 0));
      if constexpr (decltype(split)::value) plo[hg] = lds_load_bf16x8((lds_ptr)pslot(buf, hg, 1));
    }
  };
  // O^T += V^T . P^T over the 32 keys of a tile, value half kh.
  auto pv_tile = [&](int st, const bf16x8 (&phi)[2], const bf16x8 (&plo)[2], auto split) {
    const lds_ptr vb[4] = {pinned(st, v_lane[0]), pinned(st, v_lane[1]), pinned(st, v_lane[2]),
                           pinned(st, v_lane[3])};
#pragma unroll
    for (int nb = 0; nb < kNBH; ++nb) {
      const bf16x8 vt = vt_block(vb, nb);
#pragma unroll
      for (int hg = 0; hg < 2; ++hg)
        oacc[hg][nb] = mfma16x16x32_bf16(vt, phi[hg], oacc[hg][nb]);
      if constexpr (decltype(split)::value) {
#pragma unroll
        for (int hg = 0; hg < 2; ++hg)
          oacc[hg][nb] = mfma16x16x32_bf16(vt, plo[hg], oacc[hg][nb]);
      }
    }
  };

  // Steady-state body of the P.V pass as an explicit software pipeline: the logits of tile
  // t1 (stage st_k) and the P.V product of the previous tile (stage st_v, operands phi/plo)
  // share the MFMA pipe.  Phase 1: one slot per contraction step, each with the two logit
  // MFMAs of that step and half of a P.V block; key fragments are read two slots ahead,
  // value fragments one block ahead.  Phase 2: the remaining P.V blocks, with the softmax
  // of tile t1 (whose inputs are complete after phase 1) in four pieces between them.
  // Scheduling fences keep the compiler from regrouping loads next to their uses.
  // The first fragments of a fused step, read ahead (right after the previous tile barrier)
  // so that their latency overlaps the barrier's other work.
  struct Ahead {
    bf16x8 k0, k1, v0;
  };
  auto read_ahead = [&](int st_k, int st_v, Ahead& ah) {
    ah.k0 = lds_load_bf16x8(pinned(st_k, k_lane[0]));
    ah.k1 = lds_load_bf16x8(pinned(st_k, k_lane[1]));
    const lds_ptr v0 = pinned(st_v, v_lane[0]);
    ah.v0 = join_tr(lds_read_tr16_at(v0), lds_read_tr16_at(v0 + kVHi));
  };
  auto fused_step = [&](int st_k, int st_v, int t1, const Ahead& ah, const bf16x8 (&phi)[2],
                        const bf16x8 (&plo)[2], float (&l_run)[2], float (&ymax)[2],
                        int st_d, int32_t row_d, auto split) {
    constexpr bool SPLIT = decltype(split)::value;
    static_assert(kKS % 2 == 0 && kKS / 2 <= kNBH, "pipeline shape");
    static_assert(Dma::kBands <= kKS, "one gather band per phase-1 slot");
    // P.V blocks in phase 1: SPLIT, half a block (two MFMAs) in each of the first 2 kN1
    // slots; otherwise one whole block (two MFMAs) in each of the first kN1s slots.
    constexpr int kN1s = kPvPhase1Single < kKS
                             ? (kPvPhase1Single < kNBH ? kPvPhase1Single : kNBH)
                             : (kKS < kNBH ? kKS : kNBH);
    constexpr int kP1 = SPLIT ? kN1 : kN1s;  // blocks done in phase 1
    const lds_ptr kb[2] = {pinned(st_k, k_lane[0]), pinned(st_k, k_lane[1])};
    const lds_ptr vb[4] = {pinned(st_v, v_lane[0]), pinned(st_v, v_lane[1]),
                           pinned(st_v, v_lane[2]), pinned(st_v, v_lane[3])};
    bf16x8 ka[3], vf[2];
    f32x4 s[2][2];
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) s[hg][0] = s[hg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    ka[0] = ah.k0;
    ka[1] = ah.k1;
    vf[0] = ah.v0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      // The gather of the tile two ahead (row row_d of this lane, stage st_d): band j in slot
      // j.  Issued as one burst after the barrier, its loads held up the wave (5-8% of the
      // kernel at 128k); one per slot, the memory pipeline works through them beside the
      // MFMA work.
      if (j < Dma::kBands) Dma::issue_band(tiles, st_d, row_d, j, kv, ld_kv, v, ld_v);
      if (j + 2 < kKS) ka[(j + 2) % 3] = lds_load_bf16x8(kb[j & 1] + ((j + 2) >> 1) * 1024);
      if constexpr (SPLIT) {
        const int n = j / 2;
        const bool pv = n < kN1;  // slots 0 .. 2 kN1 - 1 also carry half a P.V block
        if (pv && (j & 1) == 0 && n + 1 < kNBH) vf[(n + 1) & 1] = vt_block(vb, n + 1);
        s[0][j & 1] = mfma16x16x32_bf16(ka[j % 3], qf[0][j], s[0][j & 1]);
        s[1][j & 1] = mfma16x16x32_bf16(ka[j % 3], qf[1][j], s[1][j & 1]);
        if (pv) {
          const bf16x8(&pp)[2] = (j & 1) ? plo : phi;
          oacc[0][n] = mfma16x16x32_bf16(vf[n & 1], pp[0], oacc[0][n]);
          oacc[1][n] = mfma16x16x32_bf16(vf[n & 1], pp[1], oacc[1][n]);
        }
      } else {
        const bool pv = j < kN1s;
        if (pv && j + 1 < kNBH) vf[(j + 1) & 1] = vt_block(vb, j + 1);
        s[0][j & 1] = mfma16x16x32_bf16(ka[j % 3], qf[0][j], s[0][j & 1]);
        s[1][j & 1] = mfma16x16x32_bf16(ka[j % 3], qf[1][j], s[1][j & 1]);
        if (pv) {
          oacc[0][j] = mfma16x16x32_bf16(vf[j & 1], phi[0], oacc[0][j]);
          oacc[1][j] = mfma16x16x32_bf16(vf[j & 1], phi[1], oacc[1][j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Phase 2.
    f32x4 y[2], p[2];
    const int slot0 = t1 * kKeysPerTile + 16 * kh + 4 * g;
    auto piece = [&](int idx) {
      const int hg = idx >> 1;
      if ((idx & 1) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = slot0 + i < n_valid ? (s[hg][0][i] + s[hg][1][i]) * scale_log2
                                              : -__builtin_inff();
          y[hg][i] = x - m_ref[hg];
        }
        ymax[hg] = __builtin_fmaxf(ymax[hg], max4(y[hg]));
#pragma unroll
        for (int i = 0; i < 4; ++i) p[hg][i] = __builtin_amdgcn_exp2f(y[hg][i]);
        l_run[hg] += (p[hg][0] + p[hg][1]) + (p[hg][2] + p[hg][3]);
      } else {
        const bf16x4 hi = __builtin_convertvector(p[hg], bf16x4);
        *(lds_i16x4*)(pslot((t1 & 1), hg, 0) + 8 * kh) = __builtin_bit_cast(i16x4, hi);
        if constexpr (SPLIT) {
          const bf16x4 lo =
              __builtin_convertvector(p[hg] - __builtin_convertvector(hi, f32x4), bf16x4);
          *(lds_i16x4*)(pslot((t1 & 1), hg, 1) + 8 * kh) = __builtin_bit_cast(i16x4, lo);
        }
      }
    };
    // Pieces of the softmax go after phase-2 blocks n0 + 1, n0 + 1 + kSp, ... (kSp apart).
    constexpr int n0 = kP1;
    constexpr int kSp = (kNBH - n0 - 1) / 4 > 1 ? (kNBH - n0 - 1) / 4 : 1;
#pragma unroll
    for (int n = n0; n < kNBH; ++n) {
      if (n + 1 < kNBH) vf[(n + 1) & 1] = vt_block(vb, n + 1);
#pragma unroll
      for (int hg = 0; hg < 2; ++hg)
        oacc[hg][n] = mfma16x16x32_bf16(vf[n & 1], phi[hg], oacc[hg][n]);
      if constexpr (SPLIT) {
#pragma unroll
        for (int hg = 0; hg < 2; ++hg)
          oacc[hg][n] = mfma16x16x32_bf16(vf[n & 1], plo[hg], oacc[hg][n]);
      }
      const int rel = n - n0 - 1;
      if (rel >= 0 && rel % kSp == 0 && rel / kSp < 4) piece(rel / kSp);
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int kDone = kNBH - n0 - 1 <= 0 ? 0 : ((kNBH - n0 - 2) / kSp + 1 < 4 ? (kNBH - n0 - 2) / kSp + 1 : 4);
#pragma unroll
    for (int idx = kDone; idx < 4; ++idx) piece(idx);  // pieces that found no block
  };

  // One pass over all tiles.  DO_PV: accumulate O and the row sums against m_ref (taken
  // from tile 0 when REF_FIRST); otherwise take the exact maximum logit of every head into
  // m_ref.  Tile t lives in LDS stage t % 3.
  auto run_pass = [&](auto do_pv, auto ref_first, auto split) {
    constexpr bool DO_PV = decltype(do_pv)::value;
    constexpr bool REF_FIRST = decltype(ref_first)::value;
    const float zero_m[2] = {0.f, 0.f};
    float ymax[2] = {-__builtin_inff(), -__builtin_inff()};
    float l_run[2] = {0.f, 0.f};
    if constexpr (DO_PV) {
#pragma unroll
      for (int hg = 0; hg < 2; ++hg)
#pragma unroll
        for (int nb = 0; nb < kNBH; ++nb) oacc[hg][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    Dma::issue(tiles, 0, 0, sel, n_valid, kv, ld_kv, v, ld_v);
    if (n_tiles > 1) {
      Dma::issue(tiles, 1, 1, sel, n_valid, kv, ld_kv, v, ld_v);
      DSA_WAIT_VMCNT(Dma::kPerWave);
    } else {
      DSA_WAIT_VMCNT(0);
    }
    tile_barrier();  // tile 0 is in LDS
    f32x4 s[2][2], y[2];
    if (compute) logits(0, s);
    if constexpr (DO_PV && REF_FIRST) {
      // The pair's common reference: the maximum of tile 0 over both key halves.
      if (compute) {
        shifted(s, 0, zero_m, y);
        *red_own = f32x2{head_max(max4(y[0])), head_max(max4(y[1]))};
      }
      DSA_WAIT_LGKMCNT0();
      tile_barrier();
      if (compute) {
        const f32x2 other = *red_partner;
        m_ref[0] = __builtin_fmaxf(head_max(max4(y[0])), other.x);
        m_ref[1] = __builtin_fmaxf(head_max(max4(y[1])), other.y);
      }
    }
    if (compute) {
      if constexpr (DO_PV) {
        shifted(s, 0, m_ref, y);
        probabilities(y, 0, l_run, ymax, split);
      } else {
        shifted(s, 0, zero_m, y);
        ymax[0] = max4(y[0]);
        ymax[1] = max4(y[1]);
      }
    }
    DSA_WAIT_VMCNT(0);
    DSA_WAIT_LGKMCNT0();
    tile_barrier();  // tile 1 is in LDS; tile 0's probabilities are exchanged
    bf16x8 phi[2], plo[2];
    if constexpr (DO_PV) {
      if (compute) read_probabilities(0, phi, plo, split);
    }
    // The max pass gathers tile t + 3 after the barrier of tile t; the P.V pass gathers tile
    // t + 2 during the fused step of tile t, into the stage freed at the previous barrier.
    if (!DO_PV && n_tiles > 2) Dma::issue(tiles, 2, 2, sel, n_valid, kv, ld_kv, v, ld_v);
    int st_cur = 0, st_next = 1, st_after = 2;  // stages of tiles t, t + 1, t + 2
    Ahead ah;
    if constexpr (DO_PV) {
      if (compute && n_tiles > 1) read_ahead(st_next, st_cur, ah);
    }
    for (int t = 0; t + 1 < n_tiles; ++t) {
      // Row of the tile gathered in this iteration (clamped, so always a valid read; past the
      // last tile the P.V pass reloads a valid row into the free stage, which nothing reads).
      const int32_t row_g = Dma::row_of(t + (DO_PV ? 2 : 3), sel, n_valid);
      if constexpr (DO_PV) {
        if (!compute) Dma::issue_row(tiles, st_after, row_g, kv, ld_kv, v, ld_v);
      }
      if (compute) {
        if constexpr (DO_PV) {
          fused_step(st_next, st_cur, t + 1, ah, phi, plo, l_run, ymax, st_after, row_g, split);
        } else {
          logits(st_next, s);
          shifted(s, t + 1, zero_m, y);
          ymax[0] = __builtin_fmaxf(ymax[0], max4(y[0]));
          ymax[1] = __builtin_fmaxf(ymax[1], max4(y[1]));
        }
      }
      DSA_WAIT_VMCNT(0);  // tile t + 2 (if any) has landed
      DSA_WAIT_LGKMCNT0();
      tile_barrier();  // tile t is consumed; tile t + 2 and tile t + 1's probabilities are visible
      if constexpr (DO_PV) {
        if (compute) {
          read_probabilities((t + 1) & 1, phi, plo, split);
          if (t + 2 < n_tiles) read_ahead(st_after, st_next, ah);
        }
      }
      if (!DO_PV && t + 3 < n_tiles) Dma::issue_row(tiles, st_cur, row_g, kv, ld_kv, v, ld_v);
      const int st_free = st_cur;
      st_cur = st_next;
      st_next = st_after;
      st_after = st_free;
    }
    if constexpr (DO_PV) {
      if (compute) pv_tile(st_cur, phi, plo, split);  // the last tile
    }
    // Combine the pair's halves: row sums (P.V pass) or maxima (max pass) per head.
    if (compute) {
      if constexpr (DO_PV) {
        overflow |= __builtin_fmaxf(ymax[0], ymax[1]) > kRefHeadroomLog2;
        *red_own = f32x2{head_sum(l_run[0]), head_sum(l_run[1])};
      } else {
        *red_own = f32x2{head_max(ymax[0]), head_max(ymax[1])};
      }
    }
    DSA_WAIT_LGKMCNT0();
    tile_barrier();
    if (compute) {
      const f32x2 other = *red_partner;
      if constexpr (DO_PV) {
        l_tot[0] = head_sum(l_run[0]) + other.x;
        l_tot[1] = head_sum(l_run[1]) + other.y;
      } else {
        m_ref[0] = __builtin_fmaxf(head_max(ymax[0]), other.x);
        m_ref[1] = __builtin_fmaxf(head_max(ymax[1]), other.y);
      }
    }
  };

  // Block-uniform choice of the probability precision (see kSplitBelow).
  auto forward = [&](auto split) {
    run_pass(std::true_type{}, std::true_type{}, split);
    if (__syncthreads_or(overflow)) {
      // Rare: a logit far above tile 0's maximum.  Take the exact maximum, then redo.
      run_pass(std::false_type{}, std::false_type{}, split);
      __syncthreads();
      run_pass(std::true_type{}, std::false_type{}, split);
    }
  };
  if (n_tiles > 0) {
    if (n_valid < kSplitBelow)
      forward(std::true_type{});
    else
      forward(std::false_type{});
  }

#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    const int head = hh * 32 + hg * 16 + r16;
    if (head >= h) continue;
    const float inv = n_valid > 0 ? 1.0f / l_tot[hg] : 0.0f;
#pragma unroll
    for (int nb = 0; nb < kNBH; ++nb) {
      const int dim = (kh * kNBH + nb) * 16 + 4 * g;
      if constexpr (OUT_F32) {
        float* orow = static_cast<float*>(o) + (row * h + head) * DV;
        *reinterpret_cast<f32x4*>(orow + dim) = oacc[hg][nb] * inv;
      } else {
        uint16_t* orow = static_cast<uint16_t*>(o) + (row * h + head) * DV;
        const f32x4 yv = oacc[hg][nb] * inv;
        const uint32_t w0 = static_cast<uint32_t>(float_to_bf16_bits(yv[0])) |
                            (static_cast<uint32_t>(float_to_bf16_bits(yv[1])) << 16);
        const uint32_t w1 = static_cast<uint32_t>(float_to_bf16_bits(yv[2])) |
                            (static_cast<uint32_t>(float_to_bf16_bits(yv[3])) << 16);
        *reinterpret_cast<uint2*>(orow + dim) = make_uint2(w0, w1);
      }
    }
    if (kh == 0 && g == 0)
      lse[row * h + head] =
          n_valid > 0 ? (m_ref[hg] + __builtin_log2f(l_tot[hg])) * kLn2 : -__builtin_inff();
  }
}

template <int DQK, int DV, bool SEP, bool F32>
hipError_t launch_fwd_variant(const void* q, const void* kv, int64_t ld_kv, const void* v,
                              int64_t ld_v, const int32_t* idx, int k, void* o, float* lse,
                              int64_t nq, int64_t n_pools, int h, float scale,
                              hipStream_t stream) {
  if constexpr (pair_fits<DQK, DV, SEP>()) {
    hipLaunchKernelGGL((attn_fwd_pair_kernel<DQK, DV, SEP, F32>),
                       dim3(static_cast<unsigned>(nq)), dim3(kAttnThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), ld_kv,
                       static_cast<const uint16_t*>(v), ld_v, idx, k, o, lse, n_pools, h,
                       scale * kLog2e);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, SEP, F32>), dim3(static_cast<unsigned>(nq)),
                       dim3(kAttnThreads), 0, stream, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(kv), ld_kv, static_cast<const uint16_t*>(v),
                       ld_v, idx, k, o, lse, n_pools, h, scale * kLog2e);
  }
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_fwd_t(const void* q, const void* kv, int64_t ld_kv, const void* v,
                        int64_t ld_v, const int32_t* idx, int k, void* o, int o_f32,
                        float* lse, int64_t nq, int64_t n_pools, int h, float scale,
                        hipStream_t stream) {
  if (v)
    return o_f32 ? launch_fwd_variant<DQK, DV, true, true>(q, kv, ld_kv, v, ld_v, idx, k, o,
                                                           lse, nq, n_pools, h, scale, stream)
                 : launch_fwd_variant<DQK, DV, true, false>(q, kv, ld_kv, v, ld_v, idx, k, o,
                                                            lse, nq, n_pools, h, scale, stream);
  return o_f32 ? launch_fwd_variant<DQK, DV, false, true>(q, kv, ld_kv, nullptr, 0, idx, k, o,
                                                          lse, nq, n_pools, h, scale, stream)
               : launch_fwd_variant<DQK, DV, false, false>(q, kv, ld_kv, nullptr, 0, idx, k, o,
                                                           lse, nq, n_pools, h, scale, stream);
}

}  // namespace

// Latent row shapes with a kernel: 128/128; 576/512 (the DeepSeek-V3.2 shape: 512 value
// columns plus 64 rotary columns of the key); and the same latent rows without the rotary
// part (NoPE, V = the whole key row), full and half width: 512/512 and 256/256.
bool attn_shape_supported(int d_qk, int d_v) {
  return (d_qk == 128 && d_v == 128) || (d_qk == 576 && d_v == 512) ||
         (d_qk == 512 && d_v == 512) || (d_qk == 256 && d_v == 256);
}

int attn_max_k() { return kMaxTopK; }

hipError_t launch_sparse_attn_fwd(const void* q, const void* kv, int64_t ld_kv, const void* v,
                                  int64_t ld_v, const int32_t* idx, int k, void* o, int o_f32,
                                  float* lse, int64_t nq, int64_t n_pools, int h, int d_qk,
                                  int d_v, float scale, hipStream_t stream) {
  if (nq <= 0) return hipSuccess;
  if (nq >= (int64_t{1} << 31)) return hipErrorInvalidConfiguration;
  if (d_qk == 128 && d_v == 128)
    return launch_fwd_t<128, 128>(q, kv, ld_kv, v, ld_v, idx, k, o, o_f32, lse, nq, n_pools, h,
                                  scale, stream);
  if (d_qk == 576 && d_v == 512)
    return launch_fwd_t<576, 512>(q, kv, ld_kv, v, ld_v, idx, k, o, o_f32, lse, nq, n_pools, h,
                                  scale, stream);
  if (d_qk == 512 && d_v == 512)
    return launch_fwd_t<512, 512>(q, kv, ld_kv, v, ld_v, idx, k, o, o_f32, lse, nq, n_pools, h,
                                  scale, stream);
  if (d_qk == 256 && d_v == 256)
    return launch_fwd_t<256, 256>(q, kv, ld_kv, v, ld_v, idx, k, o, o_f32, lse, nq, n_pools, h,
                                  scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
