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

#include "attn_common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

// Largest log2 excess of a logit over the softmax reference that the fp32/bf16 arithmetic
// of the P.V product tolerates (probabilities up to 2^64, sums far below fp32 overflow).
constexpr float kRefHeadroomLog2 = 64.0f;

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

template <int DQK, int DV, bool SEP, bool F32>
hipError_t launch_fwd_variant(const void* q, const void* kv, int64_t ld_kv, const void* v,
                              int64_t ld_v, const int32_t* idx, int k, void* o, float* lse,
                              int64_t nq, int64_t n_pools, int h, float scale,
                              hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, SEP, F32>), dim3(static_cast<unsigned>(nq)),
                     dim3(kAttnThreads), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(kv), ld_kv, static_cast<const uint16_t*>(v),
                     ld_v, idx, k, o, lse, n_pools, h, scale * kLog2e);
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

bool attn_shape_supported(int d_qk, int d_v) {
  return (d_qk == 128 && d_v == 128) || (d_qk == 576 && d_v == 512);
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
  return hipErrorInvalidValue;
}

}  // namespace dsa
