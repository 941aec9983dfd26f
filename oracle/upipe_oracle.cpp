// upipe_oracle.cpp -- fp64 CPU oracle for one GPU's share of a causal GQA
// self-attention layer (forward and backward), unchunked.
//
// TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
// benchmark's CPU-baseline leg load this library.  It shares no source,
// header, table or helper with the GPU library, and the GPU library never
// calls it.
//
// What it follows (pages on "Untied Ulysses: Memory-Efficient Context
// Parallelism via Headwise Chunking"):
//  * paper.rainbus.top summary, section 前置知识 / DeepSpeed Ulysses: after the
//    sequence-to-head exchange a device holds every position for a subset of
//    heads and computes full attention for those heads on its own.
//  * same page, section 前置知识 / 分组查询注意力 (GQA): H query heads, G key/value
//    heads, each block of H/G consecutive query heads shares one KV head.
//  * same page, sections 核心方法 and 方法步骤详情: headwise chunking only splits
//    the H heads into H/U stages; each stage projects its heads' Q, K, V from X
//    and runs attention over the full sequence.  Stages partition independent
//    per-head work, so the chunked layer reaches exactly the unchunked result:
//    this oracle is that unchunked definition and U does not appear in it.
//  * fugumt.com abstract: chunking happens "at the attention head level".
//
// Readings where the pages are silent (each one listed in the design notes):
//  softmax scale tau = 1/sqrt(d_head); causal mask j <= i (diagonal kept);
//  no bias or dropout; batch 1; query head h uses KV
//  head floor(h / (H/G)); LSE is the natural log of sum_j exp(tau q_i.k_j);
//  the backward is that of L = sum(O * dO) (dO given), with gradients for
//  X, Wq, Wk, Wv.
//
// Rotary position embedding (optional, rope_theta > 0; not on the pages, it
// belongs to the Llama and Qwen model families that run this layer): the
// rotate-half form.  For frequency c < d/2, w_c = theta^(-2c/d), and at token
// position i the pair (c, c + d/2) of every query and key row is rotated by
// the angle i*w_c:
//   y[c]       = x[c] cos(i w_c) - x[c + d/2] sin(i w_c)
//   y[c + d/2] = x[c + d/2] cos(i w_c) + x[c] sin(i w_c)
// Values are not rotated.  The backward applies the transposed rotation to
// the gradients of the rotated rows.
//
// QK-norm (optional, the *_qkn entry points; not on the pages, it belongs to
// the Qwen3 family the pages train): every projected query and key row x of a
// head (d values) is RMS-normalised and scaled by a weight shared by all
// heads, gamma_q for queries and gamma_k for keys, before the rotary
// embedding:
//   r = 1 / sqrt(sum_c x_c^2 / d + eps),  xhat = x r,  y_c = gamma_c xhat_c.
// Its backward, for the gradient gy of y:
//   gx_c = r (gamma_c gy_c - xhat_c (sum_e gamma_e gy_e xhat_e) / d),
//   dgamma_c = sum over heads and rows of gy_c xhat_c.
//
// Output projection (optional, oracle_out_proj; not on the pages' step list,
// it is the linear map that follows attention in the Llama and Qwen blocks):
// Y = O Wo^T with Wo [d_model][H*d]; for L = sum(Y * dY) the attention output
// receives dO = dY Wo and the weight dWo = dY^T O.
//
// Arithmetic: every input element is decoded exactly into an fp64 value
// (bf16 bits, fp32 or fp64 storage) and everything after that is fp64, in
// plain loops: a row's softmax is two passes (max, then exp/sum), there is
// no tiling and no online rescaling.  Work is spread over threads by output
// row only; each output element is produced by exactly one thread with a
// fixed loop order, so results do not depend on the thread count.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>
#include <functional>

namespace {

// ---------------------------------------------------------------- decoding
// enc: 0 = bf16 bit patterns (uint16), 1 = fp32, 2 = fp64.
double decode_one(const void* p, int enc, int64_t i) {
  if (enc == 0) {
    uint16_t h = static_cast<const uint16_t*>(p)[i];
    uint32_t u = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return static_cast<double>(f);
  }
  if (enc == 1) return static_cast<double>(static_cast<const float*>(p)[i]);
  return static_cast<const double*>(p)[i];
}

std::vector<double> decode(const void* p, int enc, int64_t n) {
  std::vector<double> out(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) out[i] = decode_one(p, enc, i);
  return out;
}

// ---------------------------------------------------------------- threads
void parallel_for(int64_t n, int nthreads, const std::function<void(int64_t)>& body) {
  if (nthreads < 1) nthreads = 1;
  if (n <= 0) return;
  int64_t t = std::min<int64_t>(nthreads, n);
  if (t == 1) {
    for (int64_t i = 0; i < n; ++i) body(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int64_t w = 0; w < t; ++w) {
    pool.emplace_back([&, w]() {
      // interleaved assignment balances the triangular causal work
      for (int64_t i = w; i < n; i += t) body(i);
    });
  }
  for (auto& th : pool) th.join();
}

double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t k = 0; k < n; ++k) s += a[k] * b[k];
  return s;
}

struct Shape {
  int64_t S, D;
  int H, G, d, causal;
  double rope_theta;  // 0: no rotary embedding
  int r() const { return H / G; }
  int kv(int h) const { return h / r(); }
  double tau() const { return 1.0 / std::sqrt(static_cast<double>(d)); }
  // keys visible to query row i: [0, last(i)]
  int64_t last(int64_t i) const { return causal ? i : S - 1; }
};

bool shape_ok(const Shape& s) {
  return s.S >= 1 && s.D >= 1 && s.H >= 1 && s.G >= 1 && s.d >= 1 && (s.H % s.G) == 0 &&
         s.rope_theta >= 0.0 && (s.rope_theta == 0.0 || s.d % 2 == 0);
}

// Rotary embedding of rows [0, nrows) of a [nrows][d] block whose row t sits at
// token position pos[t] (pos = null: position t).  sign = +1 rotates by +angle
// (forward), -1 by -angle (the transpose, for gradients).
void rotate_rows(double* x, int64_t nrows, const int64_t* pos, const Shape& s, int sign) {
  if (s.rope_theta == 0.0) return;
  const int half = s.d / 2;
  for (int64_t t = 0; t < nrows; ++t) {
    const double i = static_cast<double>(pos ? pos[t] : t);
    double* row = x + t * s.d;
    for (int c = 0; c < half; ++c) {
      const double w = std::pow(s.rope_theta, -2.0 * c / s.d);
      const double cs = std::cos(i * w), sn = sign * std::sin(i * w);
      const double a = row[c], b = row[c + half];
      row[c] = a * cs - b * sn;
      row[c + half] = b * cs + a * sn;
    }
  }
}

// QK-norm weights (decoded), off when empty.
struct QkNorm {
  double eps = 0.0;
  std::vector<double> gq, gk;  // [d] each
  bool on() const { return !gq.empty(); }
};

// RMS-normalise rows [0, nrows) of a [nrows][d] block in place and scale by
// gamma; xhat (the normalised rows) and rinv (1/rms per row) are kept when
// given, for the backward.
void normalize_rows(double* x, int64_t nrows, int d, const std::vector<double>& gamma, double eps,
                    double* xhat, double* rinv) {
  for (int64_t t = 0; t < nrows; ++t) {
    double* row = x + t * d;
    double ss = 0.0;
    for (int c = 0; c < d; ++c) ss += row[c] * row[c];
    const double r = 1.0 / std::sqrt(ss / d + eps);
    if (rinv) rinv[t] = r;
    for (int c = 0; c < d; ++c) {
      const double xh = row[c] * r;
      if (xhat) xhat[t * d + c] = xh;
      row[c] = gamma[c] * xh;
    }
  }
}

// Backward of normalize_rows: g holds the gradient of the scaled rows on
// entry and that of the unnormalised rows on exit; dgamma accumulates
// sum_t g_t * xhat_t (rows ascending).
void normalize_rows_bwd(double* g, int64_t nrows, int d, const std::vector<double>& gamma,
                        const double* xhat, const double* rinv, double* dgamma) {
  for (int64_t t = 0; t < nrows; ++t) {
    double* row = g + t * d;
    const double* xh = xhat + t * d;
    double dot_gx = 0.0;
    for (int c = 0; c < d; ++c) {
      dot_gx += gamma[c] * row[c] * xh[c];
      dgamma[c] += row[c] * xh[c];
    }
    for (int c = 0; c < d; ++c) row[c] = rinv[t] * (gamma[c] * row[c] - xh[c] * dot_gx / d);
  }
}

// Project rows [0, nrows) of X ([S][D]) through the rows of W that belong to
// head `head` (W is [nh*d][D], head h = rows h*d .. h*d+d-1):
// out[i][c] = sum_k X[i][k] * W[head*d + c][k]   (out is [nrows][d]).
// Each output is one sum over k ascending, as dot() forms it; eight outputs
// of a row are formed side by side (independent sums, so the same values).
void project_head(const std::vector<double>& X, const std::vector<double>& W, const Shape& s,
                  int head, int64_t nrows, const int64_t* rows, double* out, int nthreads) {
  constexpr int CB = 8;
  parallel_for(nrows, nthreads, [&](int64_t t) {
    int64_t i = rows ? rows[t] : t;
    const double* x = &X[static_cast<size_t>(i * s.D)];
    int c = 0;
    for (; c + CB <= s.d; c += CB) {
      const double* w[CB];
      double acc[CB];
      for (int b = 0; b < CB; ++b) {
        w[b] = &W[static_cast<size_t>((static_cast<int64_t>(head) * s.d + c + b) * s.D)];
        acc[b] = 0.0;
      }
      for (int64_t k = 0; k < s.D; ++k)
        for (int b = 0; b < CB; ++b) acc[b] += x[k] * w[b][k];
      for (int b = 0; b < CB; ++b) out[t * s.d + c + b] = acc[b];
    }
    for (; c < s.d; ++c) {
      const double* w = &W[static_cast<size_t>((static_cast<int64_t>(head) * s.d + c) * s.D)];
      out[t * s.d + c] = dot(x, w, s.D);
    }
  });
}

// dW[row][k] = sum_i grad[i][row] * X[i][k] for the nheads*d rows of a
// gradient held as [nheads][S][d], each element summed over i ascending.
// A block of rows is accumulated while X streams by once (the same sums in
// the same order as one element at a time).
void weight_grad(const std::vector<double>& grad, const std::vector<double>& X, int64_t S,
                 int64_t D, int d, int nheads, double* dW, int nthreads) {
  constexpr int RB = 32;
  const int64_t nrow = static_cast<int64_t>(nheads) * d;
  const int64_t nblk = (nrow + RB - 1) / RB;
  parallel_for(nblk, nthreads, [&](int64_t b) {
    const int64_t r0 = b * RB, r1 = std::min(nrow, r0 + RB);
    std::vector<double> acc(static_cast<size_t>((r1 - r0) * D), 0.0);
    for (int64_t i = 0; i < S; ++i) {
      const double* x = &X[static_cast<size_t>(i * D)];
      for (int64_t row = r0; row < r1; ++row) {
        const int64_t h = row / d, c = row % d;
        const double g = grad[static_cast<size_t>((h * S + i) * d + c)];
        double* a = &acc[static_cast<size_t>((row - r0) * D)];
        for (int64_t k = 0; k < D; ++k) a[k] += g * x[k];
      }
    }
    std::copy(acc.begin(), acc.end(), dW + r0 * D);
  });
}

// dX[i][k] = sum_h sum_c dQ_h[i][c] Wq[h*d+c][k]
//          + sum_g sum_c (dK_g[i][c] Wk[g*d+c][k] + dV_g[i][c] Wv[g*d+c][k]),
// the terms added in that order (query heads, then per KV head and column the
// key and value terms as one pair).  Row i of dX is accumulated while the
// weight rows stream by (the same sums, in the same order, per element).
// dQ is [H][n][d] and dK, dV are [G][n][d]; rows t of those give dX row t.
void input_grad(const std::vector<double>& dQ, const std::vector<double>& dK,
                const std::vector<double>& dV, const std::vector<double>& Wq,
                const std::vector<double>& Wk, const std::vector<double>& Wv, int64_t n,
                int64_t D, int H, int G, int d, double* dX, int nthreads) {
  parallel_for(n, nthreads, [&](int64_t t) {
    double* acc = dX + t * D;
    for (int64_t k = 0; k < D; ++k) acc[k] = 0.0;
    for (int h = 0; h < H; ++h)
      for (int c = 0; c < d; ++c) {
        const double g = dQ[static_cast<size_t>((h * n + t) * d + c)];
        const double* w = &Wq[static_cast<size_t>((static_cast<int64_t>(h) * d + c) * D)];
        for (int64_t k = 0; k < D; ++k) acc[k] += g * w[k];
      }
    for (int g = 0; g < G; ++g)
      for (int c = 0; c < d; ++c) {
        const double gk = dK[static_cast<size_t>((g * n + t) * d + c)];
        const double gv = dV[static_cast<size_t>((g * n + t) * d + c)];
        const double* wk = &Wk[static_cast<size_t>((static_cast<int64_t>(g) * d + c) * D)];
        const double* wv = &Wv[static_cast<size_t>((static_cast<int64_t>(g) * d + c) * D)];
        for (int64_t k = 0; k < D; ++k) acc[k] += gk * wk[k] + gv * wv[k];
      }
  });
}

// Row i of one head's attention, given q_i, all K and V of the KV head.
// Writes o (d values) and returns LSE.  Two passes over the visible keys.
double attend_row(const double* q, const double* K, const double* V, const Shape& s, int64_t i,
                  double* o, std::vector<double>& scores) {
  int64_t n = s.last(i) + 1;
  scores.resize(static_cast<size_t>(n));
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    scores[j] = s.tau() * dot(q, K + j * s.d, s.d);
    m = std::max(m, scores[j]);
  }
  double sum = 0.0;
  for (int64_t j = 0; j < n; ++j) sum += std::exp(scores[j] - m);
  double lse = m + std::log(sum);
  for (int c = 0; c < s.d; ++c) o[c] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double p = std::exp(scores[j] - lse);
    for (int c = 0; c < s.d; ++c) o[c] += p * V[j * s.d + c];
  }
  return lse;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

QkNorm decode_norm(const void* gqp, const void* gkp, int enc, int d, double eps) {
  QkNorm n;
  if (gqp && gkp) {
    n.eps = eps;
    n.gq = decode(gqp, enc, d);
    n.gk = decode(gkp, enc, d);
  }
  return n;
}

int forward_impl(const Shape& s, const QkNorm& nrm, int enc, const void* Xp, const void* Wqp,
                 const void* Wkp, const void* Wvp, double* O, double* LSE, int nthreads) {
  const int64_t S = s.S, D = s.D;
  const int H = s.H, G = s.G, d = s.d;
  std::vector<double> X = decode(Xp, enc, S * D);
  std::vector<double> Wq = decode(Wqp, enc, static_cast<int64_t>(H) * d * D);
  std::vector<double> Wk = decode(Wkp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> Wv = decode(Wvp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> K(static_cast<size_t>(S * d)), V(static_cast<size_t>(S * d)),
      Q(static_cast<size_t>(S * d));
  for (int g = 0; g < G; ++g) {
    project_head(X, Wk, s, g, S, nullptr, K.data(), nthreads);
    project_head(X, Wv, s, g, S, nullptr, V.data(), nthreads);
    if (nrm.on()) normalize_rows(K.data(), S, d, nrm.gk, nrm.eps, nullptr, nullptr);
    rotate_rows(K.data(), S, nullptr, s, +1);
    for (int h = g * s.r(); h < (g + 1) * s.r(); ++h) {
      project_head(X, Wq, s, h, S, nullptr, Q.data(), nthreads);
      if (nrm.on()) normalize_rows(Q.data(), S, d, nrm.gq, nrm.eps, nullptr, nullptr);
      rotate_rows(Q.data(), S, nullptr, s, +1);
      parallel_for(S, nthreads, [&](int64_t i) {
        std::vector<double> scores;
        std::vector<double> o(static_cast<size_t>(d));
        LSE[static_cast<int64_t>(h) * S + i] =
            attend_row(&Q[i * d], K.data(), V.data(), s, i, o.data(), scores);
        for (int c = 0; c < d; ++c) O[i * (static_cast<int64_t>(H) * d) + h * d + c] = o[c];
      });
    }
  }
  return 0;
}

}  // namespace

extern "C" {

// Forward.  X [S][D], Wq [H*d][D], Wk/Wv [G*d][D] in encoding `enc`.
// Outputs (fp64, caller-owned): O [S][H*d] (column h*d+c), LSE [H][S].
// Returns 0, or 1 on an invalid shape.
int oracle_forward(int64_t S, int64_t D, int H, int G, int d, int causal, double rope_theta,
                   int enc, const void* Xp, const void* Wqp, const void* Wkp, const void* Wvp,
                   double* O, double* LSE, int nthreads) {
  Shape s{S, D, H, G, d, causal, rope_theta};
  if (!shape_ok(s)) return 1;
  return forward_impl(s, QkNorm(), enc, Xp, Wqp, Wkp, Wvp, O, LSE, nthreads);
}

// Forward with QK-norm: gamma_q, gamma_k [d] in encoding `enc`, eps >= 0.
int oracle_forward_qkn(int64_t S, int64_t D, int H, int G, int d, int causal, double rope_theta,
                       double eps, int enc, const void* Xp, const void* Wqp, const void* Wkp,
                       const void* Wvp, const void* gqp, const void* gkp, double* O, double* LSE,
                       int nthreads) {
  Shape s{S, D, H, G, d, causal, rope_theta};
  if (!shape_ok(s) || !gqp || !gkp || !(eps >= 0.0)) return 1;
  return forward_impl(s, decode_norm(gqp, gkp, enc, d, eps), enc, Xp, Wqp, Wkp, Wvp, O, LSE,
                      nthreads);
}

// Forward on a subset of query rows and of query heads [h0, h1).  rows[0..nrows)
// are token indices; keys/values are projected only for the KV heads of those
// query heads and the positions those rows see.  Outputs: Orows [nrows][H*d],
// LSErows [H][nrows] (fp64); entries of other heads are left untouched.
}  // extern "C"

namespace {

int forward_rows_impl(const Shape& s, const QkNorm& nrm, int enc, const void* Xp, const void* Wqp,
                      const void* Wkp, const void* Wvp, const int64_t* rows, int64_t nrows, int h0,
                      int h1, double* Orows, double* LSErows, int nthreads) {
  const int64_t S = s.S, D = s.D;
  const int H = s.H, G = s.G, d = s.d;
  if (nrows < 0 || h0 < 0 || h1 > H || h0 >= h1) return 1;
  int64_t need = 0;  // keys needed: [0, need)
  for (int64_t t = 0; t < nrows; ++t) {
    if (rows[t] < 0 || rows[t] >= S) return 1;
    need = std::max(need, s.last(rows[t]) + 1);
  }
  // Decode only the X rows that are used.
  std::vector<double> X(static_cast<size_t>(need * D));
  for (int64_t i = 0; i < need * D; ++i) X[i] = decode_one(Xp, enc, i);
  std::vector<double> Xq(static_cast<size_t>(nrows * D));
  for (int64_t t = 0; t < nrows; ++t)
    for (int64_t k = 0; k < D; ++k) Xq[t * D + k] = decode_one(Xp, enc, rows[t] * D + k);
  std::vector<double> Wq = decode(Wqp, enc, static_cast<int64_t>(H) * d * D);
  std::vector<double> Wk = decode(Wkp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> Wv = decode(Wvp, enc, static_cast<int64_t>(G) * d * D);
  Shape sk = s;
  sk.S = need;
  std::vector<double> K(static_cast<size_t>(need * d)), V(static_cast<size_t>(need * d)),
      Q(static_cast<size_t>(nrows * d));
  Shape sq = s;
  sq.S = nrows;
  for (int g = s.kv(h0); g <= s.kv(h1 - 1); ++g) {
    project_head(X, Wk, sk, g, need, nullptr, K.data(), nthreads);
    project_head(X, Wv, sk, g, need, nullptr, V.data(), nthreads);
    if (nrm.on()) normalize_rows(K.data(), need, d, nrm.gk, nrm.eps, nullptr, nullptr);
    rotate_rows(K.data(), need, nullptr, s, +1);
    for (int h = std::max(h0, g * s.r()); h < std::min(h1, (g + 1) * s.r()); ++h) {
      project_head(Xq, Wq, sq, h, nrows, nullptr, Q.data(), nthreads);
      if (nrm.on()) normalize_rows(Q.data(), nrows, d, nrm.gq, nrm.eps, nullptr, nullptr);
      rotate_rows(Q.data(), nrows, rows, s, +1);
      parallel_for(nrows, nthreads, [&](int64_t t) {
        std::vector<double> scores;
        std::vector<double> o(static_cast<size_t>(d));
        LSErows[static_cast<int64_t>(h) * nrows + t] =
            attend_row(&Q[t * d], K.data(), V.data(), s, rows[t], o.data(), scores);
        for (int c = 0; c < d; ++c) Orows[t * (static_cast<int64_t>(H) * d) + h * d + c] = o[c];
      });
    }
  }
  return 0;
}

}  // namespace

extern "C" {

int oracle_forward_rows(int64_t S, int64_t D, int H, int G, int d, int causal,
                        double rope_theta, int enc, const void* Xp, const void* Wqp,
                        const void* Wkp, const void* Wvp, const int64_t* rows, int64_t nrows,
                        int h0, int h1, double* Orows, double* LSErows, int nthreads) {
  Shape s{S, D, H, G, d, causal, rope_theta};
  if (!shape_ok(s)) return 1;
  return forward_rows_impl(s, QkNorm(), enc, Xp, Wqp, Wkp, Wvp, rows, nrows, h0, h1, Orows,
                           LSErows, nthreads);
}

// Sampled rows with QK-norm (gamma_q, gamma_k [d] in encoding `enc`, eps >= 0).
int oracle_forward_rows_qkn(int64_t S, int64_t D, int H, int G, int d, int causal,
                            double rope_theta, double eps, int enc, const void* Xp,
                            const void* Wqp, const void* Wkp, const void* Wvp, const void* gqp,
                            const void* gkp, const int64_t* rows, int64_t nrows, int h0, int h1,
                            double* Orows, double* LSErows, int nthreads) {
  Shape s{S, D, H, G, d, causal, rope_theta};
  if (!shape_ok(s) || !gqp || !gkp || !(eps >= 0.0)) return 1;
  return forward_rows_impl(s, decode_norm(gqp, gkp, enc, d, eps), enc, Xp, Wqp, Wkp, Wvp, rows,
                           nrows, h0, h1, Orows, LSErows, nthreads);
}

// Forward + backward of L = sum(O * dO).
// Inputs in encoding `enc`: X, Wq, Wk, Wv, dO [S][H*d].
// Outputs (fp64): O, LSE as in oracle_forward; dX [S][D]; dWq [H*d][D];
// dWk, dWv [G*d][D].
//
// With P = softmax(tau Q K^T) (masked) and D_i = <dO_i, O_i>:
//   dP_ij = <dO_i, V_j>,  dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = tau sum_j dS_ij K_j,   dK_j = tau sum_{h in group} sum_i dS_ij Q_i,
//   dV_j = sum_{h in group} sum_i P_ij dO_i
//   dW* = d*^T X,   dX = sum_h dQ_h Wq_h + sum_g (dK_g Wk_g + dV_g Wv_g)
// Row quantities (dQ) are computed by a pass over query rows, column
// quantities (dK, dV) by a pass over key rows; each recomputes P and dP from
// Q, K, V, LSE and dO, so no two threads ever write the same element.
}  // extern "C"

namespace {

int backward_impl(const Shape& s, const QkNorm& nrm, int enc, const void* Xp, const void* Wqp,
                  const void* Wkp, const void* Wvp, const void* dOp, double* O, double* LSE,
                  double* dX, double* dWq, double* dWk, double* dWv, double* dgq, double* dgk,
                  int nthreads) {
  const int64_t S = s.S, D = s.D;
  const int H = s.H, G = s.G, d = s.d, causal = s.causal;
  const int64_t Hd = static_cast<int64_t>(H) * d;
  const int r = s.r();
  std::vector<double> X = decode(Xp, enc, S * D);
  std::vector<double> Wq = decode(Wqp, enc, Hd * D);
  std::vector<double> Wk = decode(Wkp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> Wv = decode(Wvp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> dO = decode(dOp, enc, S * Hd);

  // Projections for every head (the oracle is not memory-frugal).
  std::vector<double> Q(static_cast<size_t>(H * S * d)), K(static_cast<size_t>(G * S * d)),
      V(static_cast<size_t>(G * S * d));
  // Q and K are kept normalised (QK-norm) and rotated (when rope_theta > 0):
  // the attention sees them so.
  std::vector<double> xq, rq, xk, rk;  // QK-norm: normalised rows and 1/rms, for the backward
  if (nrm.on()) {
    xq.resize(static_cast<size_t>(H * S * d));
    rq.resize(static_cast<size_t>(H * S));
    xk.resize(static_cast<size_t>(G * S * d));
    rk.resize(static_cast<size_t>(G * S));
  }
  for (int h = 0; h < H; ++h) {
    project_head(X, Wq, s, h, S, nullptr, &Q[h * S * d], nthreads);
    if (nrm.on()) normalize_rows(&Q[h * S * d], S, d, nrm.gq, nrm.eps, &xq[h * S * d], &rq[h * S]);
    rotate_rows(&Q[h * S * d], S, nullptr, s, +1);
  }
  for (int g = 0; g < G; ++g) {
    project_head(X, Wk, s, g, S, nullptr, &K[g * S * d], nthreads);
    project_head(X, Wv, s, g, S, nullptr, &V[g * S * d], nthreads);
    if (nrm.on()) normalize_rows(&K[g * S * d], S, d, nrm.gk, nrm.eps, &xk[g * S * d], &rk[g * S]);
    rotate_rows(&K[g * S * d], S, nullptr, s, +1);
  }

  // Forward (O, LSE) and D.
  std::vector<double> Dv(static_cast<size_t>(H * S));
  for (int h = 0; h < H; ++h) {
    const int g = s.kv(h);
    parallel_for(S, nthreads, [&](int64_t i) {
      std::vector<double> scores;
      std::vector<double> o(static_cast<size_t>(d));
      LSE[h * S + i] = attend_row(&Q[(h * S + i) * d], &K[g * S * d], &V[g * S * d], s, i,
                                  o.data(), scores);
      double dd = 0.0;
      for (int c = 0; c < d; ++c) {
        O[i * Hd + h * d + c] = o[c];
        dd += dO[i * Hd + h * d + c] * o[c];
      }
      Dv[h * S + i] = dd;
    });
  }

  auto prob = [&](int h, int64_t i, int64_t j) {  // P_ij for head h
    const int g = s.kv(h);
    double sc = s.tau() * dot(&Q[(h * S + i) * d], &K[(g * S + j) * d], d);
    return std::exp(sc - LSE[h * S + i]);
  };
  auto dprob = [&](int h, int64_t i, int64_t j) {  // dP_ij for head h
    const int g = s.kv(h);
    return dot(&dO[i * Hd + h * d], &V[(g * S + j) * d], d);
  };

  // dQ: pass over query rows.
  std::vector<double> dQ(static_cast<size_t>(H * S * d), 0.0);
  for (int h = 0; h < H; ++h) {
    const int g = s.kv(h);
    parallel_for(S, nthreads, [&](int64_t i) {
      double* dq = &dQ[(h * S + i) * d];
      for (int64_t j = 0; j <= s.last(i); ++j) {
        double dsij = prob(h, i, j) * (dprob(h, i, j) - Dv[h * S + i]);
        for (int c = 0; c < d; ++c) dq[c] += s.tau() * dsij * K[(g * S + j) * d + c];
      }
    });
  }

  // dK, dV: pass over key rows; query heads of the group in ascending order.
  std::vector<double> dK(static_cast<size_t>(G * S * d), 0.0), dV(static_cast<size_t>(G * S * d), 0.0);
  for (int g = 0; g < G; ++g) {
    parallel_for(S, nthreads, [&](int64_t j) {
      double* dk = &dK[(g * S + j) * d];
      double* dv = &dV[(g * S + j) * d];
      for (int h = g * r; h < (g + 1) * r; ++h) {
        // query rows that see key j
        int64_t i0 = causal ? j : 0;
        for (int64_t i = i0; i < S; ++i) {
          double p = prob(h, i, j);
          double dsij = p * (dprob(h, i, j) - Dv[h * S + i]);
          for (int c = 0; c < d; ++c) {
            dk[c] += s.tau() * dsij * Q[(h * S + i) * d + c];
            dv[c] += p * dO[i * Hd + h * d + c];
          }
        }
      }
    });
  }

  // dQ and dK so far are gradients of the rotated rows; the projections see
  // them through the transposed rotation.
  for (int h = 0; h < H; ++h) rotate_rows(&dQ[h * S * d], S, nullptr, s, -1);
  for (int g = 0; g < G; ++g) rotate_rows(&dK[g * S * d], S, nullptr, s, -1);
  // QK-norm: then back through the normalisation (heads ascending, rows
  // ascending in the weight gradients).
  if (nrm.on()) {
    for (int c = 0; c < d; ++c) dgq[c] = dgk[c] = 0.0;
    for (int h = 0; h < H; ++h)
      normalize_rows_bwd(&dQ[h * S * d], S, d, nrm.gq, &xq[h * S * d], &rq[h * S], dgq);
    for (int g = 0; g < G; ++g)
      normalize_rows_bwd(&dK[g * S * d], S, d, nrm.gk, &xk[g * S * d], &rk[g * S], dgk);
  }

  // Weight gradients: dW[row][k] = sum_i grad[i][row] * X[i][k].
  weight_grad(dQ, X, S, D, d, H, dWq, nthreads);
  weight_grad(dK, X, S, D, d, G, dWk, nthreads);
  weight_grad(dV, X, S, D, d, G, dWv, nthreads);

  // Input gradient: dX[i][k] = sum over projected rows of grad * W.
  input_grad(dQ, dK, dV, Wq, Wk, Wv, S, D, H, G, d, dX, nthreads);
  return 0;
}

}  // namespace

extern "C" {

int oracle_backward(int64_t S, int64_t D, int H, int G, int d, int causal, double rope_theta,
                    int enc, const void* Xp, const void* Wqp, const void* Wkp, const void* Wvp,
                    const void* dOp, double* O, double* LSE, double* dX, double* dWq,
                    double* dWk, double* dWv, int nthreads) {
  Shape s{S, D, H, G, d, causal, rope_theta};
  if (!shape_ok(s)) return 1;
  return backward_impl(s, QkNorm(), enc, Xp, Wqp, Wkp, Wvp, dOp, O, LSE, dX, dWq, dWk, dWv,
                       nullptr, nullptr, nthreads);
}

// Backward with QK-norm (gamma_q, gamma_k [d] in encoding `enc`, eps >= 0);
// also writes dgamma_q, dgamma_k [d] (fp64).
int oracle_backward_qkn(int64_t S, int64_t D, int H, int G, int d, int causal, double rope_theta,
                        double eps, int enc, const void* Xp, const void* Wqp, const void* Wkp,
                        const void* Wvp, const void* gqp, const void* gkp, const void* dOp,
                        double* O, double* LSE, double* dX, double* dWq, double* dWk, double* dWv,
                        double* dgq, double* dgk, int nthreads) {
  Shape s{S, D, H, G, d, causal, rope_theta};
  if (!shape_ok(s) || !gqp || !gkp || !dgq || !dgk || !(eps >= 0.0)) return 1;
  return backward_impl(s, decode_norm(gqp, gkp, enc, d, eps), enc, Xp, Wqp, Wkp, Wvp, dOp, O,
                       LSE, dX, dWq, dWk, dWv, dgq, dgk, nthreads);
}

// Input gradient at the last rows [t0, S) of a causal layer, from the same
// definition as oracle_backward but without the O(S^2) passes: row t of dX
// needs dQ_h[t] (query row t against keys <= t), and dK_g[t], dV_g[t], which
// gather over query rows i >= t only, so every attention row involved lies in
// [t0, S).  K and V are projected for all positions; Q, O, LSE and D only for
// rows [t0, S).  Output dXt [(S - t0)][D] (fp64).  Returns 0, or 1 on an
// invalid shape, t0 outside [0, S) or a non-causal layer.
int oracle_dx_tail(int64_t S, int64_t D, int H, int G, int d, double rope_theta, int enc,
                   const void* Xp, const void* Wqp, const void* Wkp, const void* Wvp,
                   const void* dOp, int64_t t0, double* dXt, int nthreads) {
  Shape s{S, D, H, G, d, 1, rope_theta};
  if (!shape_ok(s) || t0 < 0 || t0 >= S) return 1;
  const int64_t Hd = static_cast<int64_t>(H) * d, n = S - t0;
  const int r = s.r();
  std::vector<double> X = decode(Xp, enc, S * D);
  std::vector<double> Wq = decode(Wqp, enc, Hd * D);
  std::vector<double> Wk = decode(Wkp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> Wv = decode(Wvp, enc, static_cast<int64_t>(G) * d * D);
  std::vector<double> dO = decode(dOp, enc, S * Hd);
  std::vector<int64_t> rows(static_cast<size_t>(n));
  for (int64_t t = 0; t < n; ++t) rows[t] = t0 + t;

  std::vector<double> K(static_cast<size_t>(G * S * d)), V(static_cast<size_t>(G * S * d));
  for (int g = 0; g < G; ++g) {
    project_head(X, Wk, s, g, S, nullptr, &K[g * S * d], nthreads);
    project_head(X, Wv, s, g, S, nullptr, &V[g * S * d], nthreads);
    rotate_rows(&K[g * S * d], S, nullptr, s, +1);
  }
  // Q, LSE and D of query rows [t0, S) (index t = i - t0).
  std::vector<double> Q(static_cast<size_t>(H * n * d)), LSE(static_cast<size_t>(H * n)),
      Dv(static_cast<size_t>(H * n));
  for (int h = 0; h < H; ++h) {
    project_head(X, Wq, s, h, n, rows.data(), &Q[h * n * d], nthreads);
    rotate_rows(&Q[h * n * d], n, rows.data(), s, +1);
    const int g = s.kv(h);
    parallel_for(n, nthreads, [&](int64_t t) {
      std::vector<double> scores;
      std::vector<double> o(static_cast<size_t>(d));
      const int64_t i = t0 + t;
      LSE[h * n + t] = attend_row(&Q[(h * n + t) * d], &K[g * S * d], &V[g * S * d], s, i,
                                  o.data(), scores);
      Dv[h * n + t] = dot(&dO[i * Hd + h * d], o.data(), d);
    });
  }
  auto prob = [&](int h, int64_t t, int64_t j) {  // P of query row t0 + t, key j
    const int g = s.kv(h);
    return std::exp(s.tau() * dot(&Q[(h * n + t) * d], &K[(g * S + j) * d], d) - LSE[h * n + t]);
  };
  auto dprob = [&](int h, int64_t t, int64_t j) {
    const int g = s.kv(h);
    return dot(&dO[(t0 + t) * Hd + h * d], &V[(g * S + j) * d], d);
  };
  // dQ of rows [t0, S): keys 0 .. i.
  std::vector<double> dQ(static_cast<size_t>(H * n * d), 0.0);
  for (int h = 0; h < H; ++h) {
    const int g = s.kv(h);
    parallel_for(n, nthreads, [&](int64_t t) {
      double* dq = &dQ[(h * n + t) * d];
      for (int64_t j = 0; j <= t0 + t; ++j) {
        const double ds = prob(h, t, j) * (dprob(h, t, j) - Dv[h * n + t]);
        for (int c = 0; c < d; ++c) dq[c] += s.tau() * ds * K[(g * S + j) * d + c];
      }
    });
  }
  // dK, dV of key rows [t0, S): query rows i >= key, heads of the group ascending.
  std::vector<double> dK(static_cast<size_t>(G * n * d), 0.0), dV(static_cast<size_t>(G * n * d), 0.0);
  for (int g = 0; g < G; ++g) {
    parallel_for(n, nthreads, [&](int64_t tj) {
      const int64_t j = t0 + tj;
      double* dk = &dK[(g * n + tj) * d];
      double* dv = &dV[(g * n + tj) * d];
      for (int h = g * r; h < (g + 1) * r; ++h) {
        for (int64_t t = tj; t < n; ++t) {
          const double p = prob(h, t, j);
          const double ds = p * (dprob(h, t, j) - Dv[h * n + t]);
          for (int c = 0; c < d; ++c) {
            dk[c] += s.tau() * ds * Q[(h * n + t) * d + c];
            dv[c] += p * dO[(t0 + t) * Hd + h * d + c];
          }
        }
      }
    });
  }
  for (int h = 0; h < H; ++h) rotate_rows(&dQ[h * n * d], n, rows.data(), s, -1);
  for (int g = 0; g < G; ++g) rotate_rows(&dK[g * n * d], n, rows.data(), s, -1);
  input_grad(dQ, dK, dV, Wq, Wk, Wv, n, D, H, G, d, dXt, nthreads);
  return 0;
}

// Output projection and its backward, by definition.  O [S][Hd] fp64 (the
// attention output), Wo [D][Hd] and dY [S][D] in encoding `enc` (dY may be
// null: forward only).  Outputs (fp64, caller-owned, any may be null):
//   Y[i][k]   = sum_c O[i][c] Wo[k][c]
//   dO[i][c]  = sum_k dY[i][k] Wo[k][c]
//   dWo[k][c] = sum_i dY[i][k] O[i][c]
// Returns 0, or 1 on an invalid shape.
int oracle_out_proj(int64_t S, int64_t D, int64_t Hd, int enc, const double* O, const void* Wop,
                    const void* dYp, double* Y, double* dO, double* dWo, int nthreads) {
  if (S < 0 || D < 1 || Hd < 1) return 1;
  std::vector<double> Wo = decode(Wop, enc, D * Hd);
  if (Y)
    parallel_for(S, nthreads, [&](int64_t i) {
      for (int64_t k = 0; k < D; ++k) Y[i * D + k] = dot(&O[i * Hd], &Wo[k * Hd], Hd);
    });
  if (!dYp) return 0;
  std::vector<double> dY = decode(dYp, enc, S * D);
  if (dO)
    parallel_for(S, nthreads, [&](int64_t i) {
      for (int64_t c = 0; c < Hd; ++c) {
        double acc = 0.0;
        for (int64_t k = 0; k < D; ++k) acc += dY[i * D + k] * Wo[k * Hd + c];
        dO[i * Hd + c] = acc;
      }
    });
  if (dWo)
    parallel_for(D, nthreads, [&](int64_t k) {
      for (int64_t c = 0; c < Hd; ++c) {
        double acc = 0.0;
        for (int64_t i = 0; i < S; ++i) acc += dY[i * D + k] * O[i * Hd + c];
        dWo[k * Hd + c] = acc;
      }
    });
  return 0;
}

}  // extern "C"
