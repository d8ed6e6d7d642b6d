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
// empty (-1) slots are never visited; only the last tile can be partial.
//
// LDS tile layout: [16-byte column chunk c][key] so that both the key-row reads for S^T and
// the transposed value reads touch contiguous 256-byte spans.

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kKeysPerTile = 32;
constexpr int kFwdThreads = 256;  // 4 waves gather every tile; waves without heads only gather
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
__device__ int compact_selection(const int32_t* __restrict__ irow, int k, int64_t n_pools,
                                 int32_t* sel, int* wave_tmp) {
  const int nthreads = kFwdThreads;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int nwaves = nthreads >> 6;
  int base = 0;
  for (int s0 = 0; s0 < k; s0 += nthreads) {
    const int s = s0 + threadIdx.x;
    const int32_t v = s < k ? irow[s] : -1;
    const bool valid = v >= 0 && v < n_pools;
    const uint64_t ballot = __ballot(valid);
    const int before = __popcll(ballot & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tmp[wid] = __popcll(ballot);
    __syncthreads();
    int off = base;
    int tot = 0;
    for (int w = 0; w < nwaves; ++w) {
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

template <int DQK, int DV, bool SEPARATE_V, bool OUT_F32>
__global__ __launch_bounds__(kFwdThreads) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t ld_kv,
    const uint16_t* __restrict__ v, int64_t ld_v, const int32_t* __restrict__ idx, int k,
    void* __restrict__ o, float* __restrict__ lse, int64_t n_pools, int h,
    float scale_log2) {
  constexpr int kChunksQK = DQK / 8;                       // 16-byte chunks of a key row
  constexpr int kChunksV = SEPARATE_V ? DV / 8 : 0;        // chunks of a separate value row
  constexpr int kChunksRow = kChunksQK + kChunksV;
  constexpr int kKS = DQK / 32;                            // MFMA steps of q . k
  constexpr int kNB = DV / 16;                             // 16-dim output blocks
  constexpr int kTileChunks = kChunksRow * kKeysPerTile;
  constexpr int kVBase = SEPARATE_V ? kChunksQK : 0;       // first chunk of V in a tile row
  static_assert(DQK % 32 == 0 && DV % 16 == 0, "tile shapes");

  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileChunks * 16];
  __shared__ int32_t sel[kMaxTopK];
  __shared__ int wave_tmp[kFwdThreads / 64];

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

  f32x4 oacc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  const int n_tiles = (n_valid + kKeysPerTile - 1) / kKeysPerTile;
  // Gather assignment: thread -> one key of the tile (tid % 32), chunk columns tid/32 + 8i.
  const int my_key = tid & (kKeysPerTile - 1);
  constexpr int kColStep = kFwdThreads / kKeysPerTile;
  constexpr int kChunksPerThread = (kTileChunks + kFwdThreads - 1) / kFwdThreads;
  u32x4 pre[kChunksPerThread];

  auto gather = [&](int t) {
    const int slot = t * kKeysPerTile + my_key;
    const int32_t p = slot < n_valid ? sel[slot] : -1;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
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
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = (tid >> 5) + i * kColStep;
      if (c < kChunksRow)
        *reinterpret_cast<u32x4*>(&tile[(c * kKeysPerTile + my_key) * 16]) = pre[i];
    }
  };

  if (n_tiles > 0) gather(0);
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();  // previous tile fully consumed
    store();
    __syncthreads();
    if (t + 1 < n_tiles) gather(t + 1);
    if (!wave_has_heads) continue;

    // S^T = K . Q^T for the 32 keys of the tile (two 16-key row blocks).
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &tile[((4 * ks + g) * kKeysPerTile + mb * 16 + r16) * 16]);
        s[mb] = mfma16x16x32_bf16(a, qf[ks], s[mb]);
      }
    }
    // Online softmax in the log2 domain; lane column = head, rows = keys 16mb + 4g + i.
    const int slot0 = t * kKeysPerTile;
    float x[2][4];
    float mt = -__builtin_inff();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = slot0 + mb * 16 + g * 4 + i < n_valid;
        x[mb][i] = ok ? s[mb][i] * scale_log2 : -__builtin_inff();
        mt = __builtin_fmaxf(mt, x[mb][i]);
      }
    mt = __builtin_fmaxf(mt, shfl_xor(mt, 16));
    mt = __builtin_fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = __builtin_fmaxf(m_run, mt);  // finite: every tile has a valid slot
    const float alpha = __builtin_exp2f(m_run - m_new);
    m_run = m_new;
    // Each probability goes to the MFMA as a bf16 pair hi + lo (lo = the bf16 rounding of
    // p - hi), so the P.V product sees p to about 16 significant bits instead of 8.
    i16x8 hbits, lbits;
    float psum = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_exp2f(x[mb][i] - m_new);
        psum += p;
        const uint16_t hb = float_to_bf16_bits(p);
        hbits[mb * 4 + i] = static_cast<short>(hb);
        lbits[mb * 4 + i] = static_cast<short>(float_to_bf16_bits(p - bf16_bits_to_float(hb)));
      }
    const bf16x8 pf_hi = bf16x8_from_bits(hbits);
    const bf16x8 pf_lo = bf16x8_from_bits(lbits);
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) oacc[nb] *= alpha;

    // O^T += V^T . P^T.  Contraction slots 0..3 <-> keys 4g+e, 4..7 <-> keys 16+4g+e,
    // matching where the S^T accumulator left the probabilities.
    const int tr_key = 4 * g + (r16 >> 2);
    const int tr_col = 4 * (r16 & 3);  // dims within a 16-dim block
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int dim = nb * 16 + tr_col;
      const int c = kVBase + (dim >> 3);
      const int byte = (dim & 7) * 2;
      const i16x4 lo = lds_read_tr16(&tile[(c * kKeysPerTile + tr_key) * 16 + byte]);
      const i16x4 hi = lds_read_tr16(&tile[(c * kKeysPerTile + 16 + tr_key) * 16 + byte]);
      const bf16x8 vt = join_tr(lo, hi);
      oacc[nb] = mfma16x16x32_bf16(vt, pf_hi, oacc[nb]);
      oacc[nb] = mfma16x16x32_bf16(vt, pf_lo, oacc[nb]);
    }
  }

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
    lse[row * h + head] = n_valid > 0 ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
}

template <int DQK, int DV, bool SEP, bool F32>
hipError_t launch_fwd_variant(const void* q, const void* kv, int64_t ld_kv, const void* v,
                              int64_t ld_v, const int32_t* idx, int k, void* o, float* lse,
                              int64_t nq, int64_t n_pools, int h, float scale,
                              hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, SEP, F32>), dim3(static_cast<unsigned>(nq)),
                     dim3(kFwdThreads), 0, stream, static_cast<const uint16_t*>(q),
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
