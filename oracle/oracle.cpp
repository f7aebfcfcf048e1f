// CPU oracle for single-query GQA decode attention — TEST INFRASTRUCTURE ONLY.
// Plain fp64 definitions; see oracle.h for the sources and the contract.
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

const double kNegInf = -std::numeric_limits<double>::infinity();

double bf16_to_double(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// Value of element d of the q row of query head qh in sequence b.
double q_at(const oracle_problem *p, int32_t b, int32_t qh, int32_t d) {
  size_t i = (static_cast<size_t>(b) * p->KH * p->G + qh) * p->D + d;
  if (p->q_type == ORACLE_F32) return static_cast<const float *>(p->q)[i];
  if (p->q_type == ORACLE_I8)
    return static_cast<const int8_t *>(p->q)[i] *
           static_cast<double>(p->q_scale[static_cast<size_t>(b) * p->KH * p->G + qh]);
  return bf16_to_double(static_cast<const uint16_t *>(p->q)[i]);
}

// Element d of K or V row (b, kh, t); INT8 codes are multiplied by their scale.
double kv_at(const oracle_problem *p, const void *base, bool is_k, int32_t b, int32_t kh, int32_t t,
             int32_t d) {
  int64_t off = p->seq_offset[b] + static_cast<int64_t>(kh) * p->stride_h +
                static_cast<int64_t>(t) * p->stride_t + d;
  switch (p->kv_type) {
    case ORACLE_F32:
      return static_cast<const float *>(base)[off];
    case ORACLE_BF16:
      return bf16_to_double(static_cast<const uint16_t *>(base)[off]);
    default: {
      double code = static_cast<const int8_t *>(base)[off];
      if (is_k) {
        const float s = p->k_scale[static_cast<int64_t>(b * p->KH + kh) * p->k_scale_stride + t / p->k_part];
        return code * static_cast<double>(s);
      }
      return code * static_cast<double>(p->v_scale);
    }
  }
}

// The tokens (b, kh) attends to, in position order.
std::vector<int32_t> token_list(const oracle_problem *p, int32_t b, int32_t kh) {
  std::vector<int32_t> toks;
  if (p->tok_idx) {
    int32_t n = p->n_idx[b * p->KH + kh];
    const int32_t *src = p->tok_idx + static_cast<int64_t>(b * p->KH + kh) * p->idx_stride;
    toks.assign(src, src + n);
  } else {
    toks.resize(std::max(0, p->lens[b]));
    for (int32_t t = 0; t < static_cast<int32_t>(toks.size()); ++t) toks[t] = t;
  }
  return toks;
}

bool problem_ok(const oracle_problem *p) {
  if (!p || p->B < 0 || p->KH < 1 || p->G < 1 || p->D < 1) return false;
  if (!p->lens || !p->seq_offset || !p->q || !p->k || !p->v) return false;
  if (p->kv_type == ORACLE_I8 && (!p->k_scale || p->k_part < 1 || p->k_scale_stride < 1)) return false;
  if (p->tok_idx && (!p->n_idx || p->idx_stride < 0)) return false;
  if (p->q_type == ORACLE_I8 && !p->q_scale) return false;
  return true;
}

// Scaled dot products s_t = softmax_scale * q . k_t for the listed tokens.
std::vector<double> scores_of(const oracle_problem *p, int32_t b, int32_t qh,
                              const std::vector<int32_t> &toks, size_t i0, size_t i1) {
  const int32_t kh = qh / p->G;
  std::vector<double> q(p->D);
  for (int32_t d = 0; d < p->D; ++d) q[d] = q_at(p, b, qh, d);
  std::vector<double> s(i1 - i0);
  for (size_t i = i0; i < i1; ++i) {
    double acc = 0.0;
    for (int32_t d = 0; d < p->D; ++d) acc += q[d] * kv_at(p, p->k, true, b, kh, toks[i], d);
    s[i - i0] = p->softmax_scale * acc;
  }
  return s;
}

// Plain two-pass softmax attention of one row over toks[i0, i1):
// M = max s, l = sum exp(s - M), out = sum exp(s - M) v / l.
void attend(const oracle_problem *p, int32_t b, int32_t qh, const std::vector<int32_t> &toks,
            size_t i0, size_t i1, double *m_out, double *l_out, double *o) {
  const int32_t kh = qh / p->G;
  for (int32_t d = 0; d < p->D; ++d) o[d] = 0.0;
  if (i1 <= i0) {
    *m_out = kNegInf;
    *l_out = 0.0;
    return;
  }
  std::vector<double> s = scores_of(p, b, qh, toks, i0, i1);
  double M = kNegInf;
  for (double x : s) M = std::max(M, x);
  double l = 0.0;
  for (size_t i = i0; i < i1; ++i) {
    double w = std::exp(s[i - i0] - M);
    l += w;
    for (int32_t d = 0; d < p->D; ++d) o[d] += w * kv_at(p, p->v, false, b, kh, toks[i], d);
  }
  for (int32_t d = 0; d < p->D; ++d) o[d] /= l;
  *m_out = M;
  *l_out = l;
}

}  // namespace

extern "C" {

int oracle_attention_rows(const oracle_problem *p, int32_t nrows, const int32_t *row_b,
                          const int32_t *row_qh, double *out, double *lse, int32_t nthreads) {
  if (!problem_ok(p) || nrows < 0 || !row_b || !row_qh || !out || !lse) return 1;
  for (int32_t r = 0; r < nrows; ++r)
    if (row_b[r] < 0 || row_b[r] >= p->B || row_qh[r] < 0 || row_qh[r] >= p->KH * p->G) return 1;
  nthreads = std::max(1, nthreads);
  auto work = [&](int32_t tid) {
    for (int32_t r = tid; r < nrows; r += nthreads) {
      const int32_t b = row_b[r], qh = row_qh[r];
      std::vector<int32_t> toks = token_list(p, b, qh / p->G);
      double m, l;
      attend(p, b, qh, toks, 0, toks.size(), &m, &l, out + static_cast<size_t>(r) * p->D);
      lse[r] = (l > 0.0) ? m + std::log(l) : kNegInf;
    }
  };
  if (nthreads == 1) {
    work(0);
  } else {
    std::vector<std::thread> pool;
    for (int32_t i = 0; i < nthreads; ++i) pool.emplace_back(work, i);
    for (auto &th : pool) th.join();
  }
  return 0;
}

// Block-online recurrence: for each block of keys/values, the running max m,
// denominator l and unnormalised output O are updated as
//   m' = max(m, max S_j), P = exp(S_j - m'), l' = exp(m - m') l + sum P,
//   O' = exp(m - m') O + P V_j,
// and the result is O / l.
int oracle_attention_rows_online(const oracle_problem *p, int32_t nrows, const int32_t *row_b,
                                 const int32_t *row_qh, int32_t block, double *out, double *lse) {
  if (!problem_ok(p) || nrows < 0 || block < 1 || !row_b || !row_qh || !out || !lse) return 1;
  for (int32_t r = 0; r < nrows; ++r) {
    const int32_t b = row_b[r], qh = row_qh[r];
    if (b < 0 || b >= p->B || qh < 0 || qh >= p->KH * p->G) return 1;
    const int32_t kh = qh / p->G;
    std::vector<int32_t> toks = token_list(p, b, kh);
    double m = kNegInf, l = 0.0;
    std::vector<double> O(p->D, 0.0);
    for (size_t j = 0; j < toks.size(); j += block) {
      size_t j1 = std::min(toks.size(), j + static_cast<size_t>(block));
      std::vector<double> S = scores_of(p, b, qh, toks, j, j1);
      double m_new = m;
      for (double x : S) m_new = std::max(m_new, x);
      const double alpha = std::exp(m - m_new);
      double psum = 0.0;
      std::vector<double> PV(p->D, 0.0);
      for (size_t i = j; i < j1; ++i) {
        const double pij = std::exp(S[i - j] - m_new);
        psum += pij;
        for (int32_t d = 0; d < p->D; ++d) PV[d] += pij * kv_at(p, p->v, false, b, kh, toks[i], d);
      }
      l = alpha * l + psum;
      for (int32_t d = 0; d < p->D; ++d) O[d] = alpha * O[d] + PV[d];
      m = m_new;
    }
    double *o = out + static_cast<size_t>(r) * p->D;
    for (int32_t d = 0; d < p->D; ++d) o[d] = (l > 0.0) ? O[d] / l : 0.0;
    lse[r] = (l > 0.0) ? m + std::log(l) : kNegInf;
  }
  return 0;
}

int oracle_partial(const oracle_problem *p, int32_t b, int32_t qh, int32_t t0, int32_t t1,
                   double *m, double *l, double *o) {
  if (!problem_ok(p) || !m || !l || !o) return 1;
  if (b < 0 || b >= p->B || qh < 0 || qh >= p->KH * p->G) return 1;
  std::vector<int32_t> toks = token_list(p, b, qh / p->G);
  const int32_t n = static_cast<int32_t>(toks.size());
  t0 = std::max(0, std::min(t0, n));
  t1 = std::max(t0, std::min(t1, n));
  attend(p, b, qh, toks, t0, t1, m, l, o);
  return 0;
}

// Partials (m_c, l_c, o_c) with o_c normalised: M = max m_c,
// l = sum exp(m_c - M) l_c, out = sum exp(m_c - M) l_c o_c / l, lse = M + ln l.
// Empty partials (l_c = 0) contribute nothing.
int oracle_merge(int32_t n, int32_t D, const double *m, const double *l, const double *o,
                 double *out, double *lse) {
  if (n < 0 || D < 1 || (n > 0 && (!m || !l || !o)) || !out || !lse) return 1;
  double M = kNegInf;
  for (int32_t c = 0; c < n; ++c)
    if (l[c] > 0.0) M = std::max(M, m[c]);
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (M == kNegInf) {
    *lse = kNegInf;
    return 0;
  }
  double L = 0.0;
  for (int32_t c = 0; c < n; ++c) {
    if (!(l[c] > 0.0)) continue;
    const double w = std::exp(m[c] - M) * l[c];
    L += w;
    for (int32_t d = 0; d < D; ++d) out[d] += w * o[static_cast<size_t>(c) * D + d];
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= L;
  *lse = M + std::log(L);
  return 0;
}

}  // extern "C"

namespace {

float bf16_to_float(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// q_val = round(val / scale) with scale = max|x| / 127, all in IEEE fp32 and
// round-half-to-even; codes are clamped to the symmetric range [-127, 127].
int8_t quantise(float x, float scale) {
  if (scale == 0.0f) return 0;
  const float qf = x / scale;
  float r = std::nearbyint(qf);
  r = std::min(127.0f, std::max(-127.0f, r));
  return static_cast<int8_t>(r);
}

}  // namespace

extern "C" {

int oracle_quant_partitions(int32_t B, int32_t KH, int32_t D, const int32_t *lens,
                            const int64_t *seq_offset, int64_t stride_h, int64_t stride_t,
                            const uint16_t *x_bf16, int32_t part, int8_t *codes, float *scales,
                            int32_t scale_stride) {
  if (B < 0 || KH < 1 || D < 1 || part < 1 || scale_stride < 1 || !lens || !seq_offset || !x_bf16 ||
      !codes || !scales)
    return 1;
  for (int32_t b = 0; b < B; ++b) {
    if (static_cast<int64_t>(lens[b] + part - 1) / part > scale_stride) return 1;
    for (int32_t kh = 0; kh < KH; ++kh) {
      const int64_t base = seq_offset[b] + kh * stride_h;
      for (int32_t t0 = 0; t0 < lens[b]; t0 += part) {
        const int32_t t1 = std::min(lens[b], t0 + part);
        float amax = 0.0f;
        for (int32_t t = t0; t < t1; ++t)
          for (int32_t d = 0; d < D; ++d)
            amax = std::max(amax, std::fabs(bf16_to_float(x_bf16[base + t * stride_t + d])));
        const float scale = amax / 127.0f;
        scales[static_cast<int64_t>(b * KH + kh) * scale_stride + t0 / part] = scale;
        for (int32_t t = t0; t < t1; ++t)
          for (int32_t d = 0; d < D; ++d) {
            const int64_t off = base + t * stride_t + d;
            codes[off] = quantise(bf16_to_float(x_bf16[off]), scale);
          }
      }
    }
  }
  return 0;
}

int oracle_quant_tensor(int32_t B, int32_t KH, int32_t D, const int32_t *lens,
                        const int64_t *seq_offset, int64_t stride_h, int64_t stride_t,
                        const uint16_t *x_bf16, int8_t *codes, float *scale) {
  if (B < 0 || KH < 1 || D < 1 || !lens || !seq_offset || !x_bf16 || !codes || !scale) return 1;
  float amax = 0.0f;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t kh = 0; kh < KH; ++kh)
      for (int32_t t = 0; t < lens[b]; ++t)
        for (int32_t d = 0; d < D; ++d)
          amax = std::max(amax,
                          std::fabs(bf16_to_float(x_bf16[seq_offset[b] + kh * stride_h + t * stride_t + d])));
  const float s = amax / 127.0f;
  *scale = s;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t kh = 0; kh < KH; ++kh)
      for (int32_t t = 0; t < lens[b]; ++t)
        for (int32_t d = 0; d < D; ++d) {
          const int64_t off = seq_offset[b] + kh * stride_h + t * stride_t + d;
          codes[off] = quantise(bf16_to_float(x_bf16[off]), s);
        }
  return 0;
}

int oracle_quant_rows(int32_t rows, int32_t D, const uint16_t *x_bf16, int8_t *codes, float *scales) {
  if (rows < 0 || D < 1 || !x_bf16 || !codes || !scales) return 1;
  for (int32_t r = 0; r < rows; ++r) {
    const uint16_t *x = x_bf16 + static_cast<int64_t>(r) * D;
    float amax = 0.0f;
    for (int32_t d = 0; d < D; ++d) amax = std::max(amax, std::fabs(bf16_to_float(x[d])));
    const float scale = amax / 127.0f;
    scales[r] = scale;
    for (int32_t d = 0; d < D; ++d) codes[static_cast<int64_t>(r) * D + d] = quantise(bf16_to_float(x[d]), scale);
  }
  return 0;
}

int oracle_quant_static(int64_t n, const uint16_t *x_bf16, float scale, int8_t *codes) {
  if (n < 0 || !x_bf16 || !codes || !(scale >= 0.0f)) return 1;
  for (int64_t i = 0; i < n; ++i) codes[i] = quantise(bf16_to_float(x_bf16[i]), scale);
  return 0;
}

int oracle_value_lognorm(const oracle_problem *p, int32_t b, int32_t kh, double eps, double *out) {
  if (!problem_ok(p) || !out || b < 0 || b >= p->B || kh < 0 || kh >= p->KH) return 1;
  for (int32_t t = 0; t < p->lens[b]; ++t) {
    double ss = 0.0;
    for (int32_t d = 0; d < p->D; ++d) {
      const double x = kv_at(p, p->v, false, b, kh, t, d);
      ss += x * x;
    }
    out[t] = std::log(std::sqrt(ss) + eps);
  }
  return 0;
}

// Output-aware score: routing logit q.k/sqrt(d) averaged over the G query
// heads sharing the KV head, plus beta times the log value magnitude.
int oracle_oam_scores(const oracle_problem *p, int32_t b, int32_t kh, double beta, double eps,
                      double *scores) {
  if (!problem_ok(p) || !scores || b < 0 || b >= p->B || kh < 0 || kh >= p->KH) return 1;
  const int32_t L = p->lens[b];
  std::vector<double> vlog(std::max(0, L));
  if (L > 0 && oracle_value_lognorm(p, b, kh, eps, vlog.data())) return 1;
  std::vector<double> qs(static_cast<size_t>(p->G) * p->D);
  for (int32_t g = 0; g < p->G; ++g)
    for (int32_t d = 0; d < p->D; ++d) qs[static_cast<size_t>(g) * p->D + d] = q_at(p, b, kh * p->G + g, d);
  for (int32_t t = 0; t < L; ++t) {
    double route = 0.0;
    for (int32_t g = 0; g < p->G; ++g) {
      double dot = 0.0;
      for (int32_t d = 0; d < p->D; ++d) dot += qs[static_cast<size_t>(g) * p->D + d] * kv_at(p, p->k, true, b, kh, t, d);
      route += dot * p->softmax_scale;
    }
    scores[t] = route / p->G + beta * vlog[t];
  }
  return 0;
}

int32_t oracle_topk_sort(const double *scores, int32_t L, int32_t k, int32_t *idx_out) {
  if (L < 0 || k < 0 || (L > 0 && !scores) || !idx_out) return -1;
  std::vector<int32_t> order(L);
  for (int32_t i = 0; i < L; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (scores[a] != scores[b]) return scores[a] > scores[b];
    return a < b;
  });
  const int32_t n = std::min(k, L);
  order.resize(n);
  std::sort(order.begin(), order.end());
  std::copy(order.begin(), order.end(), idx_out);
  return n;
}

int32_t oracle_block_select(const oracle_problem *p, int32_t b, int32_t kh, int32_t block_tokens, int32_t n_blocks,
                            double beta, double eps, int32_t *idx_out, double *block_scores) {
  if (!problem_ok(p) || !idx_out || block_tokens < 1 || n_blocks < 0 || b < 0 || b >= p->B || kh < 0 ||
      kh >= p->KH)
    return -1;
  const int32_t L = std::max(0, p->lens[b]);
  std::vector<double> tok(L);
  if (L > 0 && oracle_oam_scores(p, b, kh, beta, eps, tok.data())) return -1;
  const int32_t nb = (L + block_tokens - 1) / block_tokens;
  std::vector<double> bs(nb);
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t t0 = j * block_tokens, t1 = std::min(L, t0 + block_tokens);
    double sum = 0.0;
    for (int32_t t = t0; t < t1; ++t) sum += tok[t];
    bs[j] = sum / (t1 - t0);
  }
  if (block_scores) std::copy(bs.begin(), bs.end(), block_scores);
  std::vector<int32_t> kept(nb);
  const int32_t nk = oracle_topk_sort(bs.data(), nb, n_blocks, kept.data());
  int32_t n = 0;
  for (int32_t i = 0; i < nk; ++i)
    for (int32_t t = kept[i] * block_tokens; t < std::min(L, (kept[i] + 1) * block_tokens); ++t) idx_out[n++] = t;
  return n;
}

int32_t oracle_topk_select(const double *scores, int32_t L, int32_t k, int32_t *idx_out) {
  if (L < 0 || k < 0 || (L > 0 && !scores) || !idx_out) return -1;
  std::vector<int32_t> order(L);
  for (int32_t i = 0; i < L; ++i) order[i] = i;
  const int32_t n = std::min(k, L);
  auto before = [&](int32_t a, int32_t b) {
    if (scores[a] != scores[b]) return scores[a] > scores[b];
    return a < b;
  };
  if (n > 0 && n < L) std::nth_element(order.begin(), order.begin() + (n - 1), order.end(), before);
  order.resize(n);
  std::sort(order.begin(), order.end());
  std::copy(order.begin(), order.end(), idx_out);
  return n;
}

}  // extern "C"
