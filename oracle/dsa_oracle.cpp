// CPU oracle for the DeepSeek Sparse Attention (DSA) layer.
//
// TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg of the bench
// load this library; the product library never does, and the two share no code, header,
// table or constant.  It is built with g++ alone.
//
// What it computes (page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens"):
//  * section "Model and bottleneck": an indexer scores every pooled key entry ("one pool per
//    4 tokens") for every query, and sparse attention then reads only about 2048 selected
//    entries per query;
//  * section "Four optimizations", item 1 (DSA truly sparse): the indexer is computed in
//    chunks of queries, the selected pool indices are int32, and the sparse kernel runs on
//    DeepSeek-V3.2-shaped tensors (latent KV rows of 576 with a 512-wide value part).
// The pages print no formula.  Where they are silent this file takes the plainest reading:
//  * indexer score I[t,s] = sum_j w[t,j] * max(0, q[t,j,:] . k[s,:]) over the H_I indexer
//    heads, one pooled key row shared by all heads (the lightning indexer as published with
//    DeepSeek-V3.2; any global scale folds into w);
//  * pool s is visible to query t iff 4s+3 <= t, so row t sees the prefix [0, V(t)) with
//    V(t) = min(P, floor((t+1)/4));
//  * top-k keeps the first min(k, V(t)) entries of the visible pools sorted by score
//    descending, lower pool index first on equal scores, and fills the rest with -1;
//  * sparse attention is softmax(scale * q . K[idx]) applied to V[idx] per query head, all
//    heads sharing one latent KV row; V is the first d_v columns of that row unless a
//    separate V table is given; a row with no valid slot gives O = 0 and LSE = -inf;
//  * the backward pass is the exact gradient of that attention in the valid slots;
//  * a pooled key is the average of its 4 tokens' rows weighted by the softmax of their gate
//    scores (the pages name "k-pool gate scores" but print no formula).
//
// Arithmetic: plain loops in double precision, one rounding at the output where the output
// has a storage type (indexer scores are rounded once to fp32).  Every entry point takes an
// explicit list of query rows so that large configurations can be checked on a sample.
//
// Error behaviour: functions return 0 on success and a negative code on bad arguments
// (-1 null pointer / bad size, -2 index out of range).  Nothing is thrown across the ABI.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <thread>
#include <vector>

namespace {

// bfloat16 is the upper half of an IEEE binary32.
double decode_bf16(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits, subnormals when the
// exponent field is 0, no infinities, S.1111.111 is NaN.
double decode_e4m3(uint8_t bits) {
  const int sign = bits >> 7;
  const int expo = (bits >> 3) & 0xF;
  const int mant = bits & 0x7;
  if (expo == 0xF && mant == 0x7) return std::numeric_limits<double>::quiet_NaN();
  double mag;
  if (expo == 0)
    mag = std::ldexp(static_cast<double>(mant), -9);  // mant/8 * 2^(1-7)
  else
    mag = std::ldexp(static_cast<double>(8 + mant), expo - 10);  // (1 + mant/8) * 2^(expo-7)
  return sign ? -mag : mag;
}

int64_t visible_pools(int64_t t, int64_t n_pools) {
  if (t < 0) return 0;
  return std::min<int64_t>(n_pools, (t + 1) / 4);
}

int resolve_threads(int nthreads, int64_t work_items) {
  int n = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  if (n < 1) n = 1;
  if (work_items < n) n = static_cast<int>(std::max<int64_t>(1, work_items));
  return n;
}

// Runs body(i) for i in [0, n) on a pool of threads that take rows one at a time.
template <class F>
void parallel_rows(int64_t n, int nthreads, F body) {
  const int nt = resolve_threads(nthreads, n);
  if (nt == 1) {
    for (int64_t i = 0; i < n; ++i) body(i, 0);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  for (int w = 0; w < nt; ++w)
    pool.emplace_back([&, w] {
      for (int64_t i = next++; i < n; i = next++) body(i, w);
    });
  for (auto& th : pool) th.join();
}

// Runs body(i, w) for i in [0, n) with worker w taking the fixed contiguous block
// [w * n / nt, (w + 1) * n / nt): the work each worker sees, and so any per-worker
// floating-point accumulation, does not depend on thread timing.
template <class F>
void parallel_rows_static(int64_t n, int nt, F body) {
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) body(i, 0);
    return;
  }
  std::vector<std::thread> pool;
  for (int w = 0; w < nt; ++w)
    pool.emplace_back([&, w] {
      const int64_t lo = n * w / nt, hi = n * (w + 1) / nt;
      for (int64_t i = lo; i < hi; ++i) body(i, w);
    });
  for (auto& th : pool) th.join();
}

// Decodes a table of `rows` rows of `cols` values with row stride `stride` (elements).
std::vector<double> decode_table(const void* src, int dtype, int64_t rows, int64_t cols,
                                 int64_t stride) {
  std::vector<double> out(static_cast<size_t>(rows * cols));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const int64_t at = r * stride + c;
      out[r * cols + c] = dtype == 1 ? decode_e4m3(static_cast<const uint8_t*>(src)[at])
                                     : decode_bf16(static_cast<const uint16_t*>(src)[at]);
    }
  return out;
}

}  // namespace

extern "C" {

int dsa_oracle_abi_version(void) { return 1; }

int64_t dsa_oracle_visible(int64_t t, int64_t n_pools) { return visible_pools(t, n_pools); }

void dsa_oracle_decode_bf16(const uint16_t* src, double* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = decode_bf16(src[i]);
}

void dsa_oracle_decode_e4m3(const uint8_t* src, double* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = decode_e4m3(src[i]);
}

// Indexer scores for the listed query rows.
//   q      [nrows, h_i, d_i] (row stride q_row_stride elements), bf16 (dtype 0) or e4m3 (1)
//   k      [n_pools, d_i] (row stride k_row_stride elements), same dtype
//   w      fp32; row r's head weights start at w + r * w_row_stride (0 = one shared vector)
//   rows   absolute query positions t of the listed rows
//   out    [nrows, ld_out] fp32: out[r, s] = I[t, s] for s < V(t), -inf for s >= V(t)
int dsa_oracle_index_scores(const void* q, int64_t q_row_stride, const void* k,
                            int64_t k_row_stride, const float* w, int64_t w_row_stride,
                            int dtype, const int64_t* rows, int64_t nrows, int64_t n_pools,
                            int h_i, int d_i, float* out, int64_t ld_out, int nthreads) {
  if (!q || !k || !w || !rows || !out || nrows < 0 || n_pools < 0 || h_i <= 0 || d_i <= 0 ||
      ld_out < n_pools || q_row_stride < int64_t(h_i) * d_i || k_row_stride < d_i ||
      (dtype != 0 && dtype != 1))
    return -1;
  const std::vector<double> keys = decode_table(k, dtype, n_pools, d_i, k_row_stride);
  parallel_rows(nrows, nthreads, [&](int64_t r, int) {
    const int64_t t = rows[r];
    const int64_t vis = visible_pools(t, n_pools);
    const char* qbase = static_cast<const char*>(q) +
                        r * q_row_stride * (dtype == 1 ? 1 : 2);
    const std::vector<double> qr = decode_table(qbase, dtype, h_i, d_i, d_i);
    const float* wr = w + r * w_row_stride;
    float* orow = out + r * ld_out;
    for (int64_t s = 0; s < vis; ++s) {
      const double* ks = &keys[s * d_i];
      double score = 0.0;
      for (int j = 0; j < h_i; ++j) {
        double dot = 0.0;
        for (int d = 0; d < d_i; ++d) dot += qr[j * d_i + d] * ks[d];
        const double relu = dot > 0.0 ? dot : 0.0;
        score += static_cast<double>(wr[j]) * relu;
      }
      float f = static_cast<float>(score);  // one round-to-nearest-even to fp32
      if (f == 0.0f) f = 0.0f;              // -0 and +0 are the same score
      orow[s] = f;
    }
    for (int64_t s = vis; s < n_pools; ++s) orow[s] = -std::numeric_limits<float>::infinity();
  });
  return 0;
}

// Top-k selection for the listed rows: the visible pools [0, V(t)) of row r of `scores`
// (row stride ld), sorted by score descending with the lower pool index first among equal
// scores; the first min(k, V(t)) pool indices go to idx[r, :], the rest of the row is -1.
int dsa_oracle_topk(const float* scores, int64_t ld, const int64_t* rows, int64_t nrows,
                    int64_t n_pools, int k, int32_t* idx, int nthreads) {
  if (!scores || !rows || !idx || nrows < 0 || n_pools < 0 || ld < n_pools || k <= 0) return -1;
  parallel_rows(nrows, nthreads, [&](int64_t r, int) {
    const int64_t vis = visible_pools(rows[r], n_pools);
    const float* srow = scores + r * ld;
    std::vector<int64_t> order(static_cast<size_t>(vis));
    std::iota(order.begin(), order.end(), int64_t{0});
    // A stable sort keeps ascending pool index among equal scores (+0 == -0 compare equal).
    std::stable_sort(order.begin(), order.end(),
                     [srow](int64_t a, int64_t b) { return srow[a] > srow[b]; });
    const int64_t take = std::min<int64_t>(k, vis);
    int32_t* irow = idx + r * k;
    for (int64_t i = 0; i < take; ++i) irow[i] = static_cast<int32_t>(order[i]);
    for (int64_t i = take; i < k; ++i) irow[i] = -1;
  });
  return 0;
}

namespace {

// Attention operands, all already decoded to double.
struct AttnArgs {
  const double* q;  // [nrows, h, d_qk], dense
  const double* kv;  // [n_pools, ld_kv]
  int64_t ld_kv;
  const double* v;  // nullptr: V is kv[:, :d_v]
  int64_t ld_v;
  const int32_t* idx;  // [nrows, k]
  int k;
  int64_t nrows, n_pools;
  int h, d_qk, d_v;
  double scale;
};

int check_attn(const AttnArgs& a) {
  if (!a.q || !a.kv || !a.idx || a.k <= 0 || a.nrows < 0 || a.n_pools < 0 || a.h <= 0 ||
      a.d_qk <= 0 || a.d_v <= 0 || a.ld_kv < a.d_qk || (a.v && a.ld_v < a.d_v) ||
      (!a.v && a.d_v > a.ld_kv))
    return -1;
  for (int64_t i = 0; i < a.nrows * a.k; ++i)
    if (a.idx[i] < -1 || a.idx[i] >= a.n_pools) return -2;
  return 0;
}

double key_at(const AttnArgs& a, int64_t row, int d) { return a.kv[row * a.ld_kv + d]; }
double val_at(const AttnArgs& a, int64_t row, int e) {
  return a.v ? a.v[row * a.ld_v + e] : a.kv[row * a.ld_kv + e];
}

// Logits of one (row, head) over its valid slots (idx != -1, in slot order); returns the
// log-sum-exp (natural log), -inf when the row has no valid slot.
double head_logits(const AttnArgs& a, int64_t r, int hh, std::vector<int32_t>& sel,
                   std::vector<double>& logit) {
  sel.clear();
  logit.clear();
  const int32_t* irow = a.idx + r * a.k;
  for (int j = 0; j < a.k; ++j)
    if (irow[j] >= 0) sel.push_back(irow[j]);
  if (sel.empty()) return -std::numeric_limits<double>::infinity();
  const double* qh = a.q + (r * a.h + hh) * a.d_qk;
  double mx = -std::numeric_limits<double>::infinity();
  for (int32_t s : sel) {
    double dot = 0.0;
    for (int d = 0; d < a.d_qk; ++d) dot += qh[d] * key_at(a, s, d);
    logit.push_back(a.scale * dot);
    mx = std::max(mx, logit.back());
  }
  double sum = 0.0;
  for (double x : logit) sum += std::exp(x - mx);
  return mx + std::log(sum);
}

int attn_fwd(const AttnArgs& a, double* o, double* lse, int nthreads) {
  if (!o || !lse) return -1;
  if (int rc = check_attn(a)) return rc;
  parallel_rows(a.nrows * a.h, nthreads, [&](int64_t item, int) {
    const int64_t r = item / a.h;
    const int hh = static_cast<int>(item % a.h);
    std::vector<int32_t> sel;
    std::vector<double> logit;
    const double l = head_logits(a, r, hh, sel, logit);
    double* oh = o + (r * a.h + hh) * a.d_v;
    std::fill(oh, oh + a.d_v, 0.0);
    lse[r * a.h + hh] = l;
    for (size_t j = 0; j < sel.size(); ++j) {
      const double p = std::exp(logit[j] - l);
      for (int e = 0; e < a.d_v; ++e) oh[e] += p * val_at(a, sel[j], e);
    }
  });
  return 0;
}

int attn_bwd(const AttnArgs& a, const double* d_o, double* dq, double* dk, double* dv,
             int nthreads) {
  if (!d_o || !dq || !dk) return -1;
  if (int rc = check_attn(a)) return rc;
  const int64_t n_pools = a.n_pools;
  const int nt = resolve_threads(nthreads, a.nrows * a.h);
  // One private accumulator per worker (fixed row blocks), summed in worker order at the end.
  std::vector<std::vector<double>> part_k(nt), part_v(nt);
  for (int w = 0; w < nt; ++w) {
    part_k[w].assign(static_cast<size_t>(n_pools * a.d_qk), 0.0);
    if (dv) part_v[w].assign(static_cast<size_t>(n_pools * a.d_v), 0.0);
  }
  parallel_rows_static(a.nrows * a.h, nt, [&](int64_t item, int w) {
    const int64_t r = item / a.h;
    const int hh = static_cast<int>(item % a.h);
    std::vector<int32_t> sel;
    std::vector<double> logit;
    const double l = head_logits(a, r, hh, sel, logit);
    double* dqh = dq + (r * a.h + hh) * a.d_qk;
    std::fill(dqh, dqh + a.d_qk, 0.0);
    if (sel.empty()) return;
    const double* qh = a.q + (r * a.h + hh) * a.d_qk;
    const double* doh = d_o + (r * a.h + hh) * a.d_v;
    const size_t n = sel.size();
    std::vector<double> p(n), dp(n);
    double delta = 0.0;  // sum_j p_j dP_j, which equals dO . O
    for (size_t j = 0; j < n; ++j) {
      p[j] = std::exp(logit[j] - l);
      double acc = 0.0;
      for (int e = 0; e < a.d_v; ++e) acc += doh[e] * val_at(a, sel[j], e);
      dp[j] = acc;
      delta += p[j] * acc;
    }
    for (size_t j = 0; j < n; ++j) {
      const double ds = p[j] * (dp[j] - delta);  // gradient w.r.t. the logit of slot j
      const int64_t s = sel[j];
      for (int d = 0; d < a.d_qk; ++d) dqh[d] += a.scale * ds * key_at(a, s, d);
      double* gk = &part_k[w][s * a.d_qk];
      for (int d = 0; d < a.d_qk; ++d) gk[d] += a.scale * ds * qh[d];
      if (dv) {
        double* gv = &part_v[w][s * a.d_v];
        for (int e = 0; e < a.d_v; ++e) gv[e] += p[j] * doh[e];
      } else {
        for (int e = 0; e < a.d_v; ++e) gk[e] += p[j] * doh[e];
      }
    }
  });
  std::fill(dk, dk + n_pools * a.d_qk, 0.0);
  if (dv) std::fill(dv, dv + n_pools * a.d_v, 0.0);
  for (int w = 0; w < nt; ++w) {
    for (int64_t i = 0; i < n_pools * a.d_qk; ++i) dk[i] += part_k[w][i];
    if (dv)
      for (int64_t i = 0; i < n_pools * a.d_v; ++i) dv[i] += part_v[w][i];
  }
  return 0;
}

std::vector<double> decode_bf16_span(const uint16_t* src, int64_t n) {
  std::vector<double> out(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) out[i] = decode_bf16(src[i]);
  return out;
}

}  // namespace

// Sparse MQA attention forward for the listed rows (row r of q and idx is the r-th listed
// query), double-precision operands.  q [nrows, h, d_qk]; kv [n_pools, ld_kv] (keys are
// the first d_qk columns; V is the first d_v columns unless v [n_pools, ld_v] is given);
// idx [nrows, k] pool indices, -1 = empty slot.  o [nrows, h, d_v] and lse [nrows, h].
int dsa_oracle_sparse_attn_fwd_f64(const double* q, const double* kv, int64_t ld_kv,
                                   const double* v, int64_t ld_v, const int32_t* idx, int k,
                                   int64_t nrows, int64_t n_pools, int h, int d_qk, int d_v,
                                   double scale, double* o, double* lse, int nthreads) {
  const AttnArgs a{q, kv, ld_kv, v, ld_v, idx, k, nrows, n_pools, h, d_qk, d_v, scale};
  return attn_fwd(a, o, lse, nthreads);
}

// Same, with bf16 operands (bit patterns); q is dense [nrows, h, d_qk].
int dsa_oracle_sparse_attn_fwd(const uint16_t* q, const uint16_t* kv, int64_t ld_kv,
                               const uint16_t* v, int64_t ld_v, const int32_t* idx, int k,
                               int64_t nrows, int64_t n_pools, int h, int d_qk, int d_v,
                               double scale, double* o, double* lse, int nthreads) {
  if (!q || !kv || nrows < 0 || n_pools < 0 || h <= 0 || d_qk <= 0 || ld_kv < 0 || ld_v < 0)
    return -1;
  const std::vector<double> qd = decode_bf16_span(q, nrows * h * d_qk);
  const std::vector<double> kvd = decode_bf16_span(kv, n_pools * ld_kv);
  const std::vector<double> vd = v ? decode_bf16_span(v, n_pools * ld_v) : std::vector<double>();
  const AttnArgs a{qd.data(), kvd.data(), ld_kv, v ? vd.data() : nullptr, ld_v, idx, k,
                   nrows, n_pools, h, d_qk, d_v, scale};
  return attn_fwd(a, o, lse, nthreads);
}

// Backward of the sparse attention above for the listed rows, given dO [nrows, h, d_v].
// Outputs, all double and all overwritten:
//   dq [nrows, h, d_qk];
//   dk [n_pools, d_qk]: gradient through the key part of the KV rows;
//   dv [n_pools, d_v]: gradient through V; when dv is null it is added into dk[:, :d_v],
//      which is the gradient of a latent KV row whose first d_v columns are also V.
// Only the listed rows contribute to dk / dv.
int dsa_oracle_sparse_attn_bwd_f64(const double* q, const double* kv, int64_t ld_kv,
                                   const double* v, int64_t ld_v, const int32_t* idx, int k,
                                   const double* d_o, int64_t nrows, int64_t n_pools, int h,
                                   int d_qk, int d_v, double scale, double* dq, double* dk,
                                   double* dv, int nthreads) {
  const AttnArgs a{q, kv, ld_kv, v, ld_v, idx, k, nrows, n_pools, h, d_qk, d_v, scale};
  return attn_bwd(a, d_o, dq, dk, dv, nthreads);
}

// Same, with bf16 operands (bit patterns) including dO.
int dsa_oracle_sparse_attn_bwd(const uint16_t* q, const uint16_t* kv, int64_t ld_kv,
                               const uint16_t* v, int64_t ld_v, const int32_t* idx, int k,
                               const uint16_t* d_o, int64_t nrows, int64_t n_pools, int h,
                               int d_qk, int d_v, double scale, double* dq, double* dk,
                               double* dv, int nthreads) {
  if (!q || !kv || !d_o || nrows < 0 || n_pools < 0 || h <= 0 || d_qk <= 0 || d_v <= 0 ||
      ld_kv < 0 || ld_v < 0)
    return -1;
  const std::vector<double> qd = decode_bf16_span(q, nrows * h * d_qk);
  const std::vector<double> kvd = decode_bf16_span(kv, n_pools * ld_kv);
  const std::vector<double> vd = v ? decode_bf16_span(v, n_pools * ld_v) : std::vector<double>();
  const std::vector<double> dod = decode_bf16_span(d_o, nrows * h * d_v);
  const AttnArgs a{qd.data(), kvd.data(), ld_kv, v ? vd.data() : nullptr, ld_v, idx, k,
                   nrows, n_pools, h, d_qk, d_v, scale};
  return attn_bwd(a, dod.data(), dq, dk, dv, nthreads);
}

// ---------------------------------------------------------------------------------------
// Pooled keys ("one pool per 4 tokens", page "SkyRL extends GLM-5.3-Flash training context to
// 1 million tokens", section "Model and bottleneck"; pooling by "k-pool gate scores", section
// "Four optimizations", item 3).  The pages print no formula; the reading taken: pool s is
// the average of the rows of tokens 4s .. 4s+3 weighted by the softmax of their gate scores,
//     w_i = exp(g[4s+i]) / sum_j exp(g[4s+j]),   pooled[s, :] = sum_i w_i x[4s+i, :],
// for s < floor(n_tokens / 4) (a trailing partial pool is never visible, so never formed),
// rounded once to bf16 (round to nearest, ties to even).

namespace {

// The bf16 value nearest to v (ties to an even last mantissa bit), as its 16-bit pattern,
// rounded from the double directly (no intermediate float rounding).  Finite v of bf16
// range only.
uint16_t round_to_bf16(double v) {
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
  const bool neg = v < 0.0;
  const double a = neg ? -v : v;
  int e;
  (void)std::frexp(a, &e);  // a = m * 2^e with m in [0.5, 1)
  // bf16 keeps 8 significant bits for normal numbers (exponent e >= -125, i.e. a >= 2^-126);
  // below that the spacing stays 2^-133 (subnormals).
  const int shift = e >= -125 ? 8 - e : 133;
  const double r = std::nearbyint(std::ldexp(a, shift));  // default mode: ties to even
  const float f = static_cast<float>(std::ldexp(r, -shift));  // exact: 8 bits at most
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return static_cast<uint16_t>((u >> 16) | (neg ? 0x8000u : 0u));
}

}  // namespace

void dsa_oracle_round_bf16(const double* src, uint16_t* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = round_to_bf16(src[i]);
}

// x: [n_tokens, ld_x] bf16 bits (the first d columns are pooled); gate: [n_tokens] fp32.
// out_f64 (optional): [n_pools, d] the pooled values before rounding; out_bits: [n_pools, d]
// bf16 bits.  n_pools = floor(n_tokens / 4).
int dsa_oracle_pool_keys(const uint16_t* x, int64_t ld_x, const float* gate, int64_t n_tokens,
                         int d, double* out_f64, uint16_t* out_bits, int nthreads) {
  if (!x || !gate || !out_bits || n_tokens < 0 || d <= 0 || ld_x < d) return -1;
  const int64_t n_pools = n_tokens / 4;
  parallel_rows(n_pools, nthreads, [&](int64_t s, int) {
    double g[4], m = -std::numeric_limits<double>::infinity();
    for (int i = 0; i < 4; ++i) {
      g[i] = static_cast<double>(gate[4 * s + i]);
      m = std::max(m, g[i]);
    }
    double wsum = 0.0, w[4];
    for (int i = 0; i < 4; ++i) {
      w[i] = std::exp(g[i] - m);
      wsum += w[i];
    }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int i = 0; i < 4; ++i) acc += (w[i] / wsum) * decode_bf16(x[(4 * s + i) * ld_x + c]);
      if (out_f64) out_f64[s * d + c] = acc;
      out_bits[s * d + c] = round_to_bf16(acc);
    }
  });
  return 0;
}

}  // extern "C"
