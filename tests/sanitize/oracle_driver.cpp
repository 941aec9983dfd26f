// Runs every entry point of the fp64 oracle on small inputs under
// AddressSanitizer and UndefinedBehaviorSanitizer (built with g++ together
// with oracle/upipe_oracle.cpp): all three input encodings, causal and full,
// GQA and MHA, with the rotary embedding, QK-norm and the output projection,
// sampled rows, the dX tail, and shapes the oracle must reject.  Checks that
// outputs are finite and that the forward-only entry points give the same
// bits as the backward's forward.  Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int oracle_forward(int64_t, int64_t, int, int, int, int, double, int, const void*, const void*,
                   const void*, const void*, double*, double*, int);
int oracle_forward_qkn(int64_t, int64_t, int, int, int, int, double, double, int, const void*,
                       const void*, const void*, const void*, const void*, const void*, double*,
                       double*, int);
int oracle_forward_rows(int64_t, int64_t, int, int, int, int, double, int, const void*, const void*,
                        const void*, const void*, const int64_t*, int64_t, int, int, double*,
                        double*, int);
int oracle_backward(int64_t, int64_t, int, int, int, int, double, int, const void*, const void*,
                    const void*, const void*, const void*, double*, double*, double*, double*,
                    double*, double*, int);
int oracle_backward_qkn(int64_t, int64_t, int, int, int, int, double, double, int, const void*,
                        const void*, const void*, const void*, const void*, const void*,
                        const void*, double*, double*, double*, double*, double*, double*, double*,
                        double*, int);
int oracle_dx_tail(int64_t, int64_t, int, int, int, double, int, const void*, const void*,
                   const void*, const void*, const void*, int64_t, double*, int);
int oracle_out_proj(int64_t, int64_t, int64_t, int, const double*, const void*, const void*,
                    double*, double*, double*, int);
}

namespace {
int g_fail = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);       \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

bool finite(const std::vector<double>& v) {
  for (double x : v)
    if (!std::isfinite(x)) return false;
  return true;
}

// n values ~ N(0, sd^2) in encoding enc (0 bf16 bits, 1 fp32, 2 fp64).
std::vector<unsigned char> draw(size_t n, double sd, int enc, std::mt19937& rng) {
  std::normal_distribution<double> nd(0.0, sd);
  const size_t w = enc == 0 ? 2 : enc == 1 ? 4 : 8;
  std::vector<unsigned char> out(n * w);
  for (size_t i = 0; i < n; ++i) {
    const double v = nd(rng);
    if (enc == 2) {
      std::memcpy(&out[i * 8], &v, 8);
    } else {
      const float f = static_cast<float>(v);
      if (enc == 1) {
        std::memcpy(&out[i * 4], &f, 4);
      } else {
        uint32_t u;
        std::memcpy(&u, &f, 4);
        const uint16_t h = static_cast<uint16_t>(u >> 16);  // truncation is fine for test data
        std::memcpy(&out[i * 2], &h, 2);
      }
    }
  }
  return out;
}

void run(int64_t S, int64_t D, int H, int G, int d, int causal, double theta, int enc, bool qkn) {
  std::mt19937 rng(static_cast<unsigned>(S * 131 + H * 7 + enc));
  const int64_t Hd = static_cast<int64_t>(H) * d;
  auto X = draw(S * D, 1.0, enc, rng), Wq = draw(Hd * D, 0.2, enc, rng),
       Wk = draw(static_cast<int64_t>(G) * d * D, 0.2, enc, rng),
       Wv = draw(static_cast<int64_t>(G) * d * D, 0.2, enc, rng), dO = draw(S * Hd, 1.0, enc, rng),
       gq = draw(d, 0.3, enc, rng), gk = draw(d, 0.3, enc, rng);
  std::vector<double> O(S * Hd), L(H * S), O2(S * Hd), L2(H * S), dX(S * D), dWq(Hd * D),
      dWk(G * d * D), dWv(G * d * D), dgq(d), dgk(d);
  if (qkn) {
    CHECK(oracle_forward_qkn(S, D, H, G, d, causal, theta, 1e-6, enc, X.data(), Wq.data(), Wk.data(),
                             Wv.data(), gq.data(), gk.data(), O.data(), L.data(), 2) == 0);
    CHECK(oracle_backward_qkn(S, D, H, G, d, causal, theta, 1e-6, enc, X.data(), Wq.data(),
                              Wk.data(), Wv.data(), gq.data(), gk.data(), dO.data(), O2.data(),
                              L2.data(), dX.data(), dWq.data(), dWk.data(), dWv.data(), dgq.data(),
                              dgk.data(), 3) == 0);
    CHECK(finite(dgq) && finite(dgk));
  } else {
    CHECK(oracle_forward(S, D, H, G, d, causal, theta, enc, X.data(), Wq.data(), Wk.data(), Wv.data(),
                         O.data(), L.data(), 2) == 0);
    CHECK(oracle_backward(S, D, H, G, d, causal, theta, enc, X.data(), Wq.data(), Wk.data(),
                          Wv.data(), dO.data(), O2.data(), L2.data(), dX.data(), dWq.data(),
                          dWk.data(), dWv.data(), 3) == 0);
  }
  CHECK(O == O2 && L == L2);
  CHECK(finite(O) && finite(L) && finite(dX) && finite(dWq) && finite(dWk) && finite(dWv));
  if (!qkn) {
    const int64_t rows[3] = {0, S / 2, S - 1};
    std::vector<double> Or(3 * Hd, NAN), Lr(H * 3, NAN);
    CHECK(oracle_forward_rows(S, D, H, G, d, causal, theta, enc, X.data(), Wq.data(), Wk.data(),
                              Wv.data(), rows, 3, 0, H, Or.data(), Lr.data(), 2) == 0);
    for (int t = 0; t < 3; ++t)
      for (int64_t c = 0; c < Hd; ++c) CHECK(std::fabs(Or[t * Hd + c] - O[rows[t] * Hd + c]) < 1e-9);
    if (causal) {
      const int64_t t0 = S - 2;
      std::vector<double> tail(2 * D);
      CHECK(oracle_dx_tail(S, D, H, G, d, theta, enc, X.data(), Wq.data(), Wk.data(), Wv.data(),
                           dO.data(), t0, tail.data(), 2) == 0);
      for (int64_t i = 0; i < 2 * D; ++i) CHECK(std::fabs(tail[i] - dX[t0 * D + i]) < 1e-9);
      CHECK(oracle_dx_tail(S, D, H, G, d, theta, enc, X.data(), Wq.data(), Wk.data(), Wv.data(),
                           dO.data(), S, tail.data(), 2) == 1);
    }
    auto Wo = draw(static_cast<size_t>(D * Hd), 0.2, enc, rng), dY = draw(S * D, 1.0, enc, rng);
    std::vector<double> Y(S * D), dOo(S * Hd), dWo(D * Hd);
    CHECK(oracle_out_proj(S, D, Hd, enc, O.data(), Wo.data(), dY.data(), Y.data(), dOo.data(),
                          dWo.data(), 2) == 0);
    CHECK(finite(Y) && finite(dOo) && finite(dWo));
    CHECK(oracle_out_proj(S, D, Hd, enc, O.data(), Wo.data(), nullptr, Y.data(), nullptr, nullptr,
                          1) == 0);
  }
}
}  // namespace

int main() {
  for (int enc = 0; enc < 3; ++enc) {
    run(37, 24, 4, 2, 8, 1, 0.0, enc, false);
    run(29, 16, 3, 3, 8, 0, 100.0, enc, false);
    run(21, 12, 4, 1, 8, 1, 1e4, enc, true);
    run(17, 20, 2, 2, 6, 0, 0.0, enc, true);
  }
  // rejected shapes and arguments
  std::vector<double> buf(4096, 0.0), out(4096);
  CHECK(oracle_forward(8, 4, 3, 2, 4, 1, 0.0, 2, buf.data(), buf.data(), buf.data(), buf.data(),
                       out.data(), out.data(), 1) == 1);  // G does not divide H
  CHECK(oracle_forward(8, 4, 2, 1, 3, 1, 10.0, 2, buf.data(), buf.data(), buf.data(), buf.data(),
                       out.data(), out.data(), 1) == 1);  // rope with odd d
  CHECK(oracle_forward_qkn(8, 4, 2, 1, 4, 1, 0.0, -1.0, 2, buf.data(), buf.data(), buf.data(),
                           buf.data(), buf.data(), buf.data(), out.data(), out.data(), 1) == 1);
  const int64_t bad_row = 8;
  CHECK(oracle_forward_rows(8, 4, 2, 1, 4, 1, 0.0, 2, buf.data(), buf.data(), buf.data(), buf.data(),
                            &bad_row, 1, 0, 2, out.data(), out.data(), 1) == 1);
  std::printf("%s: %d failures\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
