// Exercises the C ABI's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ against hip_stubs.cpp; no GPU):
//  * plans over a grid of shapes, U, flags, dtypes (valid and invalid): the
//    head schedule covers every head once in ascending order, loads and
//    finishes every KV head once, and the workspace regions are 256-byte
//    aligned, inside the phase's size and pairwise disjoint;
//  * every entry point with bad arguments returns an error before anything
//    reaches a kernel launcher or the HIP runtime;
//  * the empty sequence zero-fills the weight gradients only;
//  * with the stand-in launchers succeeding, whole forward and backward calls
//    (plain, pipelined, output projection, QK-norm, more than 64 chunks per
//    launch) run their stage loops.
// Exit status 0 when every check holds; failures are printed.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <utility>
#include <vector>

#include "../../headwise_chunked_context_stage_amd/csrc/upipe_internal.h"

extern int g_launches, g_fills, g_hip_calls;
extern bool g_ok;

namespace {

int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);          \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

struct Region {
  size_t off, bytes;
};

// Regions of a plan's workspace (offset, bytes) in the backward's layout.
void check_layout(const upipe::Plan& p) {
  const upipe::WsLayout& w = p.ws;
  const size_t e = p.elem(), Sd = static_cast<size_t>(p.S) * p.d, nkv = p.kv_per_stage;
  const size_t nb = (static_cast<size_t>(p.S) + upipe::kNormBlock - 1) / upipe::kNormBlock;
  const int copies = p.pipeline ? 2 : 1;
  std::vector<Region> fwd, bwd;
  for (int c = 0; c < copies; ++c) {
    fwd.push_back({w.q[c], p.U * Sd * e});
    fwd.push_back({w.k[c], nkv * Sd * e});
    fwd.push_back({w.v[c], nkv * Sd * e});
    bwd.push_back({w.dq[c], p.U * Sd * e});
    bwd.push_back({w.dd[c], static_cast<size_t>(p.U) * p.S * 4});
    bwd.push_back({w.lse2[c], static_cast<size_t>(p.U) * p.S * 4});
    bwd.push_back({w.dk[c], nkv * Sd * e});
    bwd.push_back({w.dv[c], nkv * Sd * e});
    if (p.qk_norm) {
      bwd.push_back({w.xq[c], p.U * Sd * 4});
      bwd.push_back({w.rq[c], static_cast<size_t>(p.U) * p.S * 4});
      bwd.push_back({w.xk[c], nkv * Sd * 4});
      bwd.push_back({w.rk[c], nkv * p.S * 4});
      if (p.dtype == UPIPE_BF16) {
        bwd.push_back({w.gq32[c], p.U * Sd * 4});
        bwd.push_back({w.gk32[c], nkv * Sd * 4});
      }
    }
  }
  if (w.dk_acc) {
    bwd.push_back({w.dk_acc, Sd * 4});
    bwd.push_back({w.dv_acc, Sd * 4});
  }
  if (p.dtype == UPIPE_BF16 && upipe::dkv_split(p.S) == 2) bwd.push_back({w.kvp, 4 * Sd * 4});
  if (p.dtype == UPIPE_BF16) {  // the weight gradients' part sums, for the most chunks of one call
    int nmax = 0;
    for (const upipe::Stage& st : p.stages) nmax = std::max(nmax, st.nq + (st.done ? 2 * st.nkv : 0));
    if (p.out_proj) nmax = std::max(nmax, p.H);
    nmax = std::min(nmax, upipe::kMaxChunks);
    bwd.push_back({w.dws, upipe::dw_scratch_bytes(p.S, p.D, nmax)});
  }
  if (p.out_proj) bwd.push_back({w.dob, p.U * Sd * e});
  if (p.qk_norm) {
    bwd.push_back({w.pq, static_cast<size_t>(p.U) * nb * p.d * 4});
    bwd.push_back({w.pk, nkv * nb * p.d * 4});
  }
  for (const Region& r : fwd) {
    CHECK(r.off % upipe::kAlign == 0);
    CHECK(r.off + r.bytes <= w.fwd_bytes);
  }
  std::vector<Region> all = fwd;
  all.insert(all.end(), bwd.begin(), bwd.end());
  for (const Region& r : all) {
    CHECK(r.off % upipe::kAlign == 0);
    CHECK(r.off + r.bytes <= w.bwd_bytes);
  }
  for (size_t i = 0; i < all.size(); ++i)
    for (size_t j = i + 1; j < all.size(); ++j) {
      if (all[i].bytes == 0 || all[j].bytes == 0) continue;
      if (all[i].off == all[j].off && all[i].bytes == all[j].bytes && !p.pipeline) continue;
      const bool disjoint = all[i].off + all[i].bytes <= all[j].off || all[j].off + all[j].bytes <= all[i].off;
      CHECK(disjoint);
    }
}

void check_schedule(const upipe_plan* h) {
  const upipe::Plan& p = h->p;
  const int n = upipe_num_stages(h);
  CHECK(n == p.H / p.U);
  std::vector<int> loads(p.G, 0), dones(p.G, 0);
  int next = 0;
  for (int s = 0; s < n; ++s) {
    int q0, nq, k0, nk, ld, dn;
    CHECK(upipe_stage_info(h, s, &q0, &nq, &k0, &nk, &ld, &dn) == UPIPE_OK);
    CHECK(q0 == next && nq == p.U);
    next += nq;
    for (int g = k0; g < k0 + nk; ++g) {
      CHECK(g >= 0 && g < p.G);
      if (g < 0 || g >= p.G) continue;
      loads[g] += ld;
      dones[g] += dn;
    }
  }
  CHECK(next == p.H);
  for (int g = 0; g < p.G; ++g) CHECK(loads[g] == 1 && dones[g] == 1);
  CHECK(upipe_stage_info(h, n, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == UPIPE_ERR_ARG);
  CHECK(upipe_stage_info(h, -1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == UPIPE_ERR_ARG);
}

// Every bad call must fail before a launcher or the runtime is reached.
void check_rejections(const upipe_plan* h) {
  const upipe::Plan& p = h->p;
  g_ok = false;
  const int l0 = g_launches, c0 = g_hip_calls;
  void* a = fake(0x10000);  // aligned stand-ins, never dereferenced
  void* mis = fake(0x10008);
  float* fa = static_cast<float*>(a);
  const size_t ws_need = std::max(p.ws.fwd_bytes, p.ws.bwd_bytes);
  if (p.S > 0 && !p.qk_norm) {
    CHECK(upipe_fwd(h, nullptr, a, a, a, a, fa, a, ws_need, nullptr) == UPIPE_ERR_ARG);
    CHECK(upipe_fwd(h, mis, a, a, a, a, fa, a, ws_need, nullptr) == UPIPE_ERR_ARG);
    CHECK(upipe_fwd(h, a, a, a, a, a, fa, a, p.ws.fwd_bytes - 1, nullptr) == UPIPE_ERR_WORKSPACE);
    CHECK(upipe_fwd(h, a, a, a, a, a, fa, fake(0x10010), ws_need, nullptr) == UPIPE_ERR_WORKSPACE);
    CHECK(upipe_bwd(h, a, a, a, a, a, a, fa, fa, fa, fa, nullptr, a, ws_need, nullptr) == UPIPE_ERR_ARG);
    CHECK(upipe_bwd(h, a, a, a, a, a, a, fa, fa, fa, fa, fa, a, p.ws.bwd_bytes - 1, nullptr) ==
          UPIPE_ERR_WORKSPACE);
  }
  if (p.qk_norm) {
    CHECK(upipe_fwd(h, a, a, a, a, a, fa, a, ws_need, nullptr) == UPIPE_ERR_ARG);
    CHECK(upipe_bwd(h, a, a, a, a, a, a, fa, fa, fa, fa, fa, a, ws_need, nullptr) == UPIPE_ERR_ARG);
  }
  if (!p.out_proj) {
    CHECK(upipe_fwd_out(h, a, a, a, a, a, a, fa, fa, a, ws_need, nullptr) == UPIPE_ERR_ARG);
    CHECK(upipe_bwd_out(h, a, a, a, a, a, a, a, fa, fa, fa, fa, fa, fa, a, ws_need, nullptr) ==
          UPIPE_ERR_ARG);
  }
  // io-struct entry points: a missing required tensor, an unused one given
  upipe_fwd_io f;
  std::memset(&f, 0, sizeof(f));
  f.X = f.Wq = f.Wk = f.Wv = a;
  f.O = a;
  f.LSE = fa;
  if (p.qk_norm) f.q_norm = f.k_norm = a;
  if (p.out_proj) {
    f.Wo = a;
    f.Y = fa;
  }
  upipe_fwd_io g = f;
  g.q_norm = p.qk_norm ? nullptr : a;
  CHECK(upipe_fwd_ex(h, &g, a, ws_need, nullptr) == UPIPE_ERR_ARG);
  g = f;
  g.Wo = p.out_proj ? nullptr : a;
  CHECK(upipe_fwd_ex(h, &g, a, ws_need, nullptr) == UPIPE_ERR_ARG);
  CHECK(upipe_fwd_ex(h, nullptr, a, ws_need, nullptr) == UPIPE_ERR_ARG);
  if (p.S > 0) {
    g = f;
    g.X = mis;
    CHECK(upipe_fwd_ex(h, &g, a, ws_need, nullptr) == UPIPE_ERR_ARG);
    CHECK(upipe_fwd_ex(h, &f, a, p.ws.fwd_bytes - 1, nullptr) == UPIPE_ERR_WORKSPACE);
  }
  upipe_bwd_io b;
  std::memset(&b, 0, sizeof(b));
  b.X = b.Wq = b.Wk = b.Wv = b.O = a;
  b.LSE = fa;
  b.dX = b.dWq = b.dWk = b.dWv = fa;
  if (p.out_proj) {
    b.dY = b.Wo = a;
    b.dWo = fa;
  } else {
    b.dO = a;
  }
  if (p.qk_norm) {
    b.q_norm = b.k_norm = a;
    b.dq_norm = b.dk_norm = fa;
  }
  upipe_bwd_io c = b;
  c.dk_norm = p.qk_norm ? nullptr : fa;
  CHECK(upipe_bwd_ex(h, &c, a, ws_need, nullptr) == UPIPE_ERR_ARG);
  c = b;
  c.dO = p.out_proj ? a : nullptr;
  CHECK(upipe_bwd_ex(h, &c, a, ws_need, nullptr) == UPIPE_ERR_ARG);
  if (p.S > 0) CHECK(upipe_bwd_ex(h, &b, a, p.ws.bwd_bytes - 1, nullptr) == UPIPE_ERR_WORKSPACE);
  CHECK(g_launches == l0);
  CHECK(g_hip_calls == c0);
}

// With the stand-in launchers succeeding: whole calls through the stage loops.
void run_calls(const upipe_plan* h) {
  const upipe::Plan& p = h->p;
  g_ok = true;
  void* a = fake(0x10000);
  float* fa = static_cast<float*>(a);
  const size_t ws = std::max(p.ws.fwd_bytes, p.ws.bwd_bytes);
  const int l0 = g_launches;
  upipe_fwd_io f;
  std::memset(&f, 0, sizeof(f));
  f.X = f.Wq = f.Wk = f.Wv = f.O = a;
  f.LSE = fa;
  if (p.qk_norm) f.q_norm = f.k_norm = a;
  if (p.out_proj) {
    f.Wo = a;
    f.Y = fa;
  }
  CHECK(upipe_fwd_ex(h, &f, a, ws, nullptr) == UPIPE_OK);
  upipe_bwd_io b;
  std::memset(&b, 0, sizeof(b));
  b.X = b.Wq = b.Wk = b.Wv = b.O = a;
  b.LSE = fa;
  b.dX = b.dWq = b.dWk = b.dWv = fa;
  if (p.out_proj) {
    b.dY = b.Wo = a;
    b.dWo = fa;
  } else {
    b.dO = a;
  }
  if (p.qk_norm) {
    b.q_norm = b.k_norm = a;
    b.dq_norm = b.dk_norm = fa;
  }
  CHECK(upipe_bwd_ex(h, &b, a, ws, nullptr) == UPIPE_OK);
  if (p.S > 0) CHECK(g_launches > l0);
  g_ok = false;
}

struct Case {
  int64_t S, D;
  int H, G, d, U, causal, dtype, flags;
  double rope, eps;
  int expect;
};

}  // namespace

int main() {
  std::vector<Case> cases;
  const int flagsets[] = {0, UPIPE_PIPELINE, UPIPE_OUT_PROJ, UPIPE_QK_NORM,
                          UPIPE_PIPELINE | UPIPE_OUT_PROJ | UPIPE_QK_NORM};
  for (int fl : flagsets) {
    for (int U : {1, 2, 4, 8}) cases.push_back({1000, 512, 8, 2, 128, U, 1, UPIPE_BF16, fl, 1e4, 1e-6, UPIPE_OK});
    for (int U : {1, 2, 4}) cases.push_back({320, 256, 4, 2, 64, U, 0, UPIPE_F32, fl, 0.0, 0.0, UPIPE_OK});
    cases.push_back({0, 256, 4, 2, 128, 2, 1, UPIPE_BF16, fl, 0.0, 1e-6, UPIPE_OK});
    cases.push_back({1, 256, 4, 4, 128, 4, 1, UPIPE_BF16, fl, 0.0, 1e-6, UPIPE_OK});
    // 128 heads in one stage: more than 64 chunks per launch
    cases.push_back({256, 256, 128, 2, 128, 128, 1, UPIPE_BF16, fl, 0.0, 1e-6, UPIPE_OK});
  }
  // invalid plans
  cases.push_back({128, 256, 4, 3, 64, 1, 1, UPIPE_F32, 0, 0.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({128, 256, 24, 4, 128, 4, 1, UPIPE_BF16, 0, 0.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({128, 256, 4, 2, 96, 1, 1, UPIPE_F32, 0, 0.0, 0.0, UPIPE_ERR_UNSUPPORTED});
  cases.push_back({128, 256, 4, 2, 64, 1, 1, UPIPE_BF16, 0, 0.0, 0.0, UPIPE_ERR_UNSUPPORTED});
  cases.push_back({128, 256, 4, 2, 128, 1, 1, UPIPE_BF16, 8, 0.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({128, 256, 4, 2, 128, 1, 1, UPIPE_BF16, UPIPE_QK_NORM, 0.0, -1.0, UPIPE_ERR_ARG});
  cases.push_back({128, 256, 4, 2, 128, 1, 1, UPIPE_BF16, UPIPE_QK_NORM, 0.0, NAN, UPIPE_ERR_ARG});
  cases.push_back({128, 256, 4, 2, 128, 1, 1, UPIPE_BF16, 0, -2.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({128, 256, 4, 2, 128, 1, 2, UPIPE_BF16, 0, 0.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({-5, 256, 4, 2, 128, 1, 1, UPIPE_BF16, 0, 0.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({128, 0, 4, 2, 128, 1, 1, UPIPE_BF16, 0, 0.0, 0.0, UPIPE_ERR_ARG});
  cases.push_back({128, 200, 4, 2, 128, 1, 1, UPIPE_BF16, 0, 0.0, 0.0, UPIPE_ERR_UNSUPPORTED});

  for (const Case& c : cases) {
    upipe_plan* h = reinterpret_cast<upipe_plan*>(0x1);
    const upipe_options o{c.flags, c.rope, c.eps};
    const int rc = upipe_create_opt(&h, c.S, c.D, c.H, c.G, c.d, c.U, c.causal, c.dtype, &o);
    CHECK(rc == c.expect);
    if (rc != UPIPE_OK) {
      CHECK(h == nullptr);
      continue;
    }
    check_layout(h->p);
    check_schedule(h);
    check_rejections(h);
    if (c.S == 0) {
      // the empty sequence: weight gradients (and dgamma) zero-filled, nothing launched
      const int f0 = g_fills, l0 = g_launches;
      upipe_bwd_io b;
      std::memset(&b, 0, sizeof(b));
      float* fa = static_cast<float*>(fake(0x10000));
      b.dWq = b.dWk = b.dWv = fa;
      if (c.flags & UPIPE_OUT_PROJ) b.dWo = fa, b.Wo = b.dY = fake(0x10000);
      else b.dO = fake(0x10000);
      if (c.flags & UPIPE_QK_NORM) b.q_norm = b.k_norm = fake(0x10000), b.dq_norm = b.dk_norm = fa;
      CHECK(upipe_bwd_ex(h, &b, nullptr, 0, nullptr) == UPIPE_OK);
      CHECK(g_fills - f0 == 3 + ((c.flags & UPIPE_OUT_PROJ) ? 1 : 0) + ((c.flags & UPIPE_QK_NORM) ? 2 : 0));
      CHECK(g_launches == l0);
    }
    run_calls(h);
    upipe_destroy(h);
  }
  upipe_destroy(nullptr);

  int U = -1;
  CHECK(upipe_auto_u(131072, 4096, 32, 8, 128, 1, UPIPE_BF16, size_t(1) << 29, &U) == UPIPE_OK && U == 4);
  CHECK(upipe_auto_u(131072, 4096, 32, 8, 128, 1, UPIPE_BF16, 1000, &U) == UPIPE_ERR_WORKSPACE && U == 0);
  CHECK(upipe_auto_u(128, 256, 4, 3, 64, 1, UPIPE_F32, size_t(1) << 30, &U) == UPIPE_ERR_ARG);
  CHECK(upipe_auto_u(128, 256, 4, 2, 64, 1, UPIPE_F32, size_t(1) << 30, nullptr) == UPIPE_ERR_ARG);
  CHECK(std::strcmp(upipe_strerror(0), "ok") == 0);
  CHECK(std::strcmp(upipe_strerror(-7), "unknown error") == 0);
  CHECK(std::strcmp(upipe_kernel_name(UPIPE_K_COUNT), "unknown") == 0);
  CHECK(std::strcmp(upipe_kernel_name(UPIPE_K_NORM), "norm") == 0);
  CHECK(upipe_create_opt(nullptr, 1, 128, 1, 1, 128, 1, 1, UPIPE_BF16, nullptr) == UPIPE_ERR_ARG);

  // timing: records made while enabled are read back and released
  g_ok = true;
  CHECK(upipe_timing_enable(1) == UPIPE_OK);
  upipe_plan* h = nullptr;
  CHECK(upipe_create(&h, 512, 256, 4, 2, 128, 2, 1, UPIPE_BF16) == UPIPE_OK);
  run_calls(h);
  g_ok = true;
  double ms[UPIPE_K_COUNT] = {0};
  int64_t n[UPIPE_K_COUNT] = {0};
  CHECK(upipe_timing_read(ms, n, UPIPE_K_COUNT) == UPIPE_OK);
  CHECK(n[UPIPE_K_ATTN_FWD] == 2 && n[UPIPE_K_ATTN_DQ] == 2);
  CHECK(upipe_timing_enable(0) == UPIPE_OK);
  upipe_destroy(h);
  g_ok = false;

  std::printf("%s: %zu plans, %d launches stood in for, %d failures\n", g_fail ? "FAILED" : "ok",
              cases.size(), g_launches, g_fail);
  return g_fail ? 1 : 0;
}
