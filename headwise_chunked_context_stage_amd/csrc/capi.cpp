// capi.cpp -- the C ABI: validation, the stage loop of the forward and the
// backward, and optional per-launch timing.
//
// Stage loop (paper.rainbus.top summary of "Untied Ulysses", section
// 方法步骤详情, steps (1) and (3); the all-to-all steps (2) and (4) move data
// between devices and have no counterpart on one GPU):
//   forward,  stage s:  project Q of its U heads (and K, V when it opens a
//                       KV group) into the stage buffers, then attention over
//                       the full sequence into the stage's columns of O.
//   backward, stage s:  recompute the same projections, D = rowsum(dO*O),
//                       dK/dV (carried in fp32 across the stages of a group),
//                       dQ, the weight gradients of the stage's heads, and
//                       dX += (gradients) x (weights) with dX itself as the
//                       running fp32 sum.
// All work is enqueued on the caller's stream; nothing here synchronises.
// A pipelined plan also uses one helper stream per device: the projections
// of the next stage and the gradient GEMMs of the current one run there,
// ordered against the attention kernels on the caller's stream by events.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "upipe_internal.h"

using namespace upipe;

namespace {

// ------------------------------------------------------------------ timing
struct TimingRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_tmu;
// read without the lock on every launch, written under it by upipe_timing_enable
std::atomic<bool> g_timing{false};
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
TimingRec g_open{-1, nullptr, nullptr};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool ptr_ok(const void* p) { return p != nullptr && aligned(p, 16); }

// A pointer the plan uses must be valid, one it does not use must be null.
bool need(const void* p, bool used) { return used ? ptr_ok(p) : p == nullptr; }

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }
const char* at(const void* base, size_t off) { return static_cast<const char*>(base) + off; }

#define UPIPE_TRY(expr)                  \
  do {                                   \
    hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return UPIPE_ERR_HIP; \
  } while (0)

// Launch wrappers: time the launch when timing is on.
template <typename F>
hipError_t timed(int kind, hipStream_t st, F&& f) {
  timing_begin(kind, st);
  hipError_t e = f();
  timing_end(kind, st);
  return e;
}

struct Kernels {
  decltype(&bf16::proj) proj;
  decltype(&bf16::attn_fwd) attn_fwd;
  decltype(&bf16::bwd_pre) bwd_pre;
  decltype(&bf16::attn_dkv) attn_dkv;
  decltype(&bf16::attn_dq) attn_dq;
  decltype(&bf16::dw) dw;
  decltype(&bf16::dx) dx;
  decltype(&bf16::oproj) oproj;
  decltype(&bf16::dout) dout;
  decltype(&bf16::dwo) dwo;
};

// fp32 variant: the rotary embedding runs as in-place passes right after the
// producing kernel (the bf16 kernels apply it in their epilogues, before
// rounding).  fp32 storage is exact, so both orders give the same values.
hipError_t f32_proj(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t,
                    const Rope& rope, const NormArgs& nrm, hipStream_t st) {
  hipError_t e = f32::proj(X, S, D, d, t, st);
  for (int i = 0; i < t.n && e == hipSuccess; ++i) {
    const int k = t.nkind[i];
    if (k) {  // QK-norm, then the rotary embedding, as the bf16 epilogue does
      const int64_t idx = t.nidx[i];
      e = norm::fwd_f32(static_cast<float*>(t.a[i]), 1, S, d,
                        static_cast<const float*>(nrm.gamma[k - 1]), nrm.eps,
                        nrm.store ? nrm.xh[k - 1] + idx * S * d : nullptr,
                        nrm.store ? nrm.ri[k - 1] + idx * S : nullptr, st);
    }
    if (e == hipSuccess && ((t.rot >> i) & 1))
      e = f32::rope(static_cast<float*>(t.a[i]), 1, S, d, rope, +1, st);
  }
  return e;
}

hipError_t f32_attn_dq(const AttnArgs& a, hipStream_t st) {
  hipError_t e = f32::attn_dq(a, st);
  if (e == hipSuccess && a.rope.on)
    e = f32::rope(static_cast<float*>(a.dq), a.nq, a.S, a.d, a.rope, -1, st);
  return e;
}

hipError_t f32_attn_dkv(const AttnArgs& a, hipStream_t st) {
  hipError_t e = f32::attn_dkv(a, st);
  const int nkv = a.nq >= a.r ? a.nq / a.r : 1;
  if (e == hipSuccess && a.rope.on && a.last_of_group)
    e = f32::rope(static_cast<float*>(a.dk), nkv, a.S, a.d, a.rope, -1, st);
  return e;
}

Kernels kernels_for(int dtype) {
  if (dtype == UPIPE_BF16)
    return {bf16::proj, bf16::attn_fwd, bf16::bwd_pre, bf16::attn_dkv, bf16::attn_dq, bf16::dw,
            bf16::dx, bf16::oproj, bf16::dout, bf16::dwo};
  return {f32_proj, f32::attn_fwd, f32::bwd_pre, f32_attn_dkv, f32_attn_dq, f32::dw, f32::dx,
          f32::oproj, f32::dout, f32::dwo};
}

// Project the stage's query heads (and its KV heads when it opens their group)
// into the stage buffers.  Chunks: one per head, d rows of the weight each.
// QK-norm weights and their gradients for one call (null when the plan has
// no QK-norm; the gradients only in the backward).
struct NormIn {
  const void* gq;
  const void* gk;
  float* dgq;
  float* dgk;
};

// Project the stage's query heads (and its KV heads when it opens their group)
// into the stage buffers.  Chunks: one per head, d rows of the weight each.
// With QK-norm, queries and keys are normalised (and with `store` their
// normalised rows and 1/rms kept in the workspace for the backward).
hipError_t stage_projection(const Plan& p, const Stage& st, const Kernels& K, const void* X,
                            const void* Wq, const void* Wk, const void* Wv, void* ws,
                            hipStream_t s, const NormIn& nin, bool store) {
  const size_t e = p.elem();
  const size_t wrows = static_cast<size_t>(p.d) * p.D * e;  // bytes of one head's weight rows
  const size_t hbuf = static_cast<size_t>(p.S) * p.d * e;   // bytes of one head's [S][d] buffer
  struct Job {
    const void* w;
    void* a;
    bool rotate;  // queries and keys take the rotary embedding, values do not
    int kind, idx;  // QK-norm: 1 = query head idx, 2 = key head idx, 0 = none
  };
  const bool rope = p.rope.on != 0;
  const int qn = p.qk_norm ? 1 : 0, kn = p.qk_norm ? 2 : 0;
  std::vector<Job> jobs;
  for (int h = 0; h < st.nq; ++h)
    jobs.push_back({at(Wq, (st.q0 + h) * wrows), at(ws, p.ws.q[st.slot] + h * hbuf), rope, qn, h});
  if (st.load) {
    for (int g = 0; g < st.nkv; ++g) {
      jobs.push_back({at(Wk, (st.kv0 + g) * wrows), at(ws, p.ws.k[st.kvslot] + g * hbuf), rope, kn, g});
      jobs.push_back({at(Wv, (st.kv0 + g) * wrows), at(ws, p.ws.v[st.kvslot] + g * hbuf), false, 0, 0});
    }
  }
  NormArgs nrm;
  std::memset(&nrm, 0, sizeof(nrm));
  if (p.qk_norm) {
    nrm.gamma[0] = nin.gq;
    nrm.gamma[1] = nin.gk;
    nrm.eps = static_cast<float>(p.qk_eps);
    nrm.store = store ? 1 : 0;
    if (store) {
      nrm.xh[0] = reinterpret_cast<float*>(at(ws, p.ws.xq[st.slot]));
      nrm.ri[0] = reinterpret_cast<float*>(at(ws, p.ws.rq[st.slot]));
      nrm.xh[1] = reinterpret_cast<float*>(at(ws, p.ws.xk[st.kvslot]));
      nrm.ri[1] = reinterpret_cast<float*>(at(ws, p.ws.rk[st.kvslot]));
    }
  }
  for (size_t b = 0; b < jobs.size(); b += kMaxChunks) {
    ChunkTable t;
    std::memset(&t, 0, sizeof(t));
    t.n = static_cast<int>(std::min<size_t>(kMaxChunks, jobs.size() - b));
    for (int i = 0; i < t.n; ++i) {
      t.w[i] = jobs[b + i].w;
      t.a[i] = jobs[b + i].a;
      if (jobs[b + i].rotate) t.rot |= uint64_t(1) << i;
      t.nkind[i] = static_cast<unsigned char>(jobs[b + i].kind);
      t.nidx[i] = static_cast<unsigned char>(jobs[b + i].idx);
    }
    hipError_t err =
        timed(UPIPE_K_PROJ, s, [&] { return K.proj(X, p.S, p.D, p.d, t, p.rope, nrm, s); });
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

AttnArgs attn_args(const Plan& p, const Stage& st, void* ws) {
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.S = p.S;
  a.H = p.H;
  a.d = p.d;
  a.causal = p.causal;
  a.nq = st.nq;
  a.q_head0 = st.q0;
  a.r = p.r;
  a.kv_head0 = st.kv0;
  a.q = at(ws, p.ws.q[st.slot]);
  a.k = at(ws, p.ws.k[st.kvslot]);
  a.v = at(ws, p.ws.v[st.kvslot]);
  a.first_of_group = st.load ? 1 : 0;
  a.last_of_group = st.done ? 1 : 0;
  a.rope = p.rope;
  return a;
}

// Backward attention of one stage: D pre-pass, dK/dV, dQ.
struct BwdIn {
  const void *dO, *X, *Wq, *Wk, *Wv, *O;
  const float* LSE;
  float *dX, *dWq, *dWk, *dWv;
  void* ws;
};

AttnArgs bwd_args(const Plan& p, const Stage& st, const BwdIn& in) {
  AttnArgs a = attn_args(p, st, in.ws);
  a.dO = in.dO;  // the caller's [S][H*d]
  a.ldo = static_cast<int64_t>(p.H) * p.d;
  a.do_hs = p.d;
  a.do_h0 = 0;
  a.o_in = in.O;
  a.lse_in = in.LSE;
  a.dd = reinterpret_cast<float*>(at(in.ws, p.ws.dd[st.slot]));
  a.lse2 = reinterpret_cast<float*>(at(in.ws, p.ws.lse2[st.slot]));
  a.dq = at(in.ws, p.ws.dq[st.slot]);
  // dK/dV belong to the KV group: the fp32 variant carries them across the
  // group's stages in these buffers, so they follow the K/V copy
  a.dk = at(in.ws, p.ws.dk[st.kvslot]);
  a.dv = at(in.ws, p.ws.dv[st.kvslot]);
  if (p.ws.dk_acc) {
    a.dk_acc = reinterpret_cast<float*>(at(in.ws, p.ws.dk_acc));
    a.dv_acc = reinterpret_cast<float*>(at(in.ws, p.ws.dv_acc));
  }
  a.kv_split = 1;
  if (p.dtype == UPIPE_BF16 && dkv_split(p.S) == 2) {
    a.kv_split = 2;
    a.kvp = reinterpret_cast<float*>(at(in.ws, p.ws.kvp));
  }
  if (p.qk_norm && p.dtype == UPIPE_BF16) {  // fp32 gradients for the normalisation's backward
    a.dq32 = reinterpret_cast<float*>(at(in.ws, p.ws.gq32[st.slot]));
    a.dk32 = reinterpret_cast<float*>(at(in.ws, p.ws.gk32[st.kvslot]));
  }
  return a;
}

// QK-norm backward of a stage, after its dK/dV and dQ: the gradients of the
// normalised query rows (and, when the stage completes its KV heads, key
// rows) go back through the normalisation into the buffers the gradient
// GEMMs read, and their per-block products are added into dgamma in order.
hipError_t stage_norm_bwd(const Plan& p, const Stage& st, const BwdIn& in, const NormIn& nin,
                          bool first_q, bool first_k, hipStream_t s) {
  const bool bf = p.dtype == UPIPE_BF16;
  auto f = [&](size_t off) { return reinterpret_cast<float*>(at(in.ws, off)); };
  hipError_t e = timed(UPIPE_K_NORM, s, [&] {
    const float* g = bf ? f(p.ws.gq32[st.slot]) : f(p.ws.dq[st.slot]);
    hipError_t r = norm::bwd(g, f(p.ws.xq[st.slot]), f(p.ws.rq[st.slot]), nin.gq, bf ? 1 : 0,
                             at(in.ws, p.ws.dq[st.slot]), bf ? 1 : 0, f(p.ws.pq), st.nq, p.S, p.d,
                             s);
    if (r == hipSuccess) r = norm::gamma_sum(nin.dgq, f(p.ws.pq), st.nq, p.S, p.d, first_q, s);
    return r;
  });
  if (e != hipSuccess || !st.done) return e;
  return timed(UPIPE_K_NORM, s, [&] {
    const float* g = bf ? f(p.ws.gk32[st.kvslot]) : f(p.ws.dk[st.kvslot]);
    hipError_t r = norm::bwd(g, f(p.ws.xk[st.kvslot]), f(p.ws.rk[st.kvslot]), nin.gk, bf ? 1 : 0,
                             at(in.ws, p.ws.dk[st.kvslot]), bf ? 1 : 0, f(p.ws.pk), st.nkv, p.S,
                             p.d, s);
    if (r == hipSuccess) r = norm::gamma_sum(nin.dgk, f(p.ws.pk), st.nkv, p.S, p.d, first_k, s);
    return r;
  });
}

// Weight and input gradients of one stage, in the one global order used for
// dX: inside each KV group, its query heads ascending, then the group's dK,
// then its dV.  Every U walks this same sequence, so dX is summed in the same
// order.
hipError_t stage_gradients(const Plan& p, const Stage& st, const Kernels& K, const BwdIn& in,
                           bool first_stage, hipStream_t s) {
  const size_t e = p.elem();
  const size_t wrows = static_cast<size_t>(p.d) * p.D * e;
  const size_t dwrows = static_cast<size_t>(p.d) * p.D;  // fp32 elements of one head's dW rows
  const size_t hbuf = static_cast<size_t>(p.S) * p.d * e;
  char* dq = at(in.ws, p.ws.dq[st.slot]);
  char* dk = at(in.ws, p.ws.dk[st.kvslot]);
  char* dv = at(in.ws, p.ws.dv[st.kvslot]);
  struct Chunk {
    void* a;
    const void* w;
    float* dw;
  };
  std::vector<Chunk> chunks;
  auto add_q = [&](int hq) {
    chunks.push_back({dq + (hq - st.q0) * hbuf, at(in.Wq, hq * wrows), in.dWq + hq * dwrows});
  };
  auto add_kv = [&](int g) {
    chunks.push_back({dk + (g - st.kv0) * hbuf, at(in.Wk, g * wrows), in.dWk + g * dwrows});
    chunks.push_back({dv + (g - st.kv0) * hbuf, at(in.Wv, g * wrows), in.dWv + g * dwrows});
  };
  for (int hq = st.q0; hq < st.q0 + st.nq; ++hq) {
    add_q(hq);
    const bool group_end = ((hq + 1) % p.r) == 0;
    if (group_end && st.done) add_kv(hq / p.r);
  }
  for (size_t b = 0; b < chunks.size(); b += kMaxChunks) {
    ChunkTable t;
    std::memset(&t, 0, sizeof(t));
    t.n = static_cast<int>(std::min<size_t>(kMaxChunks, chunks.size() - b));
    for (int i = 0; i < t.n; ++i) {
      t.a[i] = chunks[b + i].a;
      t.w[i] = chunks[b + i].w;
      t.dw[i] = chunks[b + i].dw;
    }
    t.czero = first_stage && b == 0;  // the first dX launch starts the running sum
    float* dws = reinterpret_cast<float*>(at(in.ws, p.ws.dws));
    hipError_t err = timed(UPIPE_K_DW, s, [&] { return K.dw(in.X, p.S, p.D, p.d, t, dws, s); });
    if (err != hipSuccess) return err;
    err = timed(UPIPE_K_DX, s, [&] { return K.dx(in.dX, p.S, p.D, p.d, t, s); });
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// ------------------------------------------------------- output projection
// The output projection's operands for one call (null members: not used).
struct OutProj {
  const void* Wo;  // [D][H*d]
  float* Y;        // forward: [S][D] fp32 running sum
  const void* dY;  // backward: [S][D]
  const void* O;   // backward: the forward's O [S][H*d]
  float* dWo;      // backward: [D][H*d] fp32
};

// The stage's heads as chunks: a = the head's columns of A (row stride H*d),
// w = the same columns of Wo, dw = the same columns of dWo; `out` (if set)
// replaces a by the head's [S][d] slice of the stage dO buffer.
template <typename F>
hipError_t per_head_chunks(const Plan& p, const Stage& st, const void* A, const void* Wo,
                           float* dWo, char* out, F&& launch) {
  const size_t e = p.elem();
  for (int b = 0; b < st.nq; b += kMaxChunks) {
    ChunkTable t;
    std::memset(&t, 0, sizeof(t));
    t.n = std::min(kMaxChunks, st.nq - b);
    for (int i = 0; i < t.n; ++i) {
      const int u = b + i, h = st.q0 + u;
      const size_t col = static_cast<size_t>(h) * p.d;
      t.w[i] = at(Wo, col * e);
      t.a[i] = out ? static_cast<void*>(out + static_cast<size_t>(u) * p.S * p.d * e)
                   : const_cast<char*>(at(A, col * e));
      t.dw[i] = dWo ? dWo + col : nullptr;
    }
    hipError_t err = launch(t);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Every head at once (the projections below need only the finished O, or
// the inputs dY and O).
Stage all_heads(const Plan& p) {
  Stage st{};
  st.q0 = 0;
  st.nq = p.H;
  return st;
}

// Forward, after the last stage: Y = O Wo^T over all heads, ascending, with
// Y as the fp32 running sum (the first launch starts it from zero).  Summing the stages' O_s Wo_s^T
// into Y one stage at a time gives the same bits (the sum runs through Y in
// fp32 in the same head order), at 8 x the read-modify-write of Y.
hipError_t layer_oproj(const Plan& p, const Kernels& K, const void* O, const OutProj& op,
                       hipStream_t s) {
  const int64_t ld = static_cast<int64_t>(p.H) * p.d;
  bool first = true;  // the first launch starts Y's running sum (no zero fill)
  return per_head_chunks(p, all_heads(p), O, op.Wo, nullptr, nullptr, [&](const ChunkTable& t) {
    ChunkTable tt = t;
    tt.czero = first ? 1 : 0;
    first = false;
    return timed(UPIPE_K_OPROJ, s, [&] { return K.oproj(op.Y, p.S, p.D, p.d, tt, ld, s); });
  });
}

// Backward, before the stage's attention backward: dO of its heads into the
// stage buffer.
hipError_t stage_dout(const Plan& p, const Stage& st, const Kernels& K, void* ws,
                      const OutProj& op, hipStream_t s) {
  const int64_t ld = static_cast<int64_t>(p.H) * p.d;
  return per_head_chunks(p, st, nullptr, op.Wo, nullptr, at(ws, p.ws.dob), [&](const ChunkTable& t) {
    return timed(UPIPE_K_DOUT, s, [&] { return K.dout(op.dY, p.S, p.D, p.d, t, ld, s); });
  });
}

// Backward: dWo = dY^T O for every head (one launch fills the chip; a
// stage's heads alone would leave it half idle).
hipError_t layer_dwo(const Plan& p, const Kernels& K, const OutProj& op, void* ws, hipStream_t s) {
  const int64_t ld = static_cast<int64_t>(p.H) * p.d;
  float* dws = reinterpret_cast<float*>(at(ws, p.ws.dws));
  return per_head_chunks(p, all_heads(p), op.O, op.Wo, op.dWo, nullptr, [&](const ChunkTable& t) {
    return timed(UPIPE_K_DWO, s, [&] { return K.dwo(op.dY, p.S, p.D, p.d, t, ld, dws, s); });
  });
}

// The attention backward of a stage reads dO from the stage buffer.
AttnArgs with_stage_do(const Plan& p, const Stage& st, void* ws, AttnArgs a) {
  a.dO = at(ws, p.ws.dob);
  a.ldo = p.d;
  a.do_hs = static_cast<int64_t>(p.S) * p.d;
  a.do_h0 = st.q0;
  return a;
}

// ------------------------------------------------------------ pipelining
// One helper stream per device, created on first use and kept.
std::mutex g_smu;
std::map<int, hipStream_t> g_helper;

hipError_t helper_stream(hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_smu);
  auto it = g_helper.find(dev);
  if (it != g_helper.end()) {
    *out = it->second;
    return hipSuccess;
  }
  hipStream_t h = nullptr;
  e = hipStreamCreateWithFlags(&h, hipStreamNonBlocking);
  if (e != hipSuccess) return e;
  g_helper[dev] = h;
  *out = h;
  return hipSuccess;
}

// Ordering events.  A call takes a set, records and waits on them while it
// enqueues, and gives them back before it returns: a wait binds to the record
// that precedes it on the host, so a later call may record the same events
// again while earlier work is still in flight.
constexpr int kSyncEvents = 8;
std::mutex g_emu;
std::vector<hipEvent_t> g_sync_pool;

struct SyncEvents {
  hipEvent_t ev[kSyncEvents] = {};
  int n = 0;
  hipError_t take() {
    std::lock_guard<std::mutex> g(g_emu);
    while (n < kSyncEvents) {
      if (!g_sync_pool.empty()) {
        ev[n++] = g_sync_pool.back();
        g_sync_pool.pop_back();
        continue;
      }
      hipError_t e = hipEventCreateWithFlags(&ev[n], hipEventDisableTiming);
      if (e != hipSuccess) return e;
      ++n;
    }
    return hipSuccess;
  }
  ~SyncEvents() {
    std::lock_guard<std::mutex> g(g_emu);
    for (int i = 0; i < n; ++i) g_sync_pool.push_back(ev[i]);
  }
};

// `waiter` waits for the work enqueued on `signaller` so far.
hipError_t order(hipEvent_t ev, hipStream_t signaller, hipStream_t waiter) {
  hipError_t e = hipEventRecord(ev, signaller);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(waiter, ev, 0);
}

// A pipelined plan overlaps stages only where the attention grid is small
// (fewer than two rounds of 256-row query blocks over the stage's heads):
// there the last query blocks of a stage run alone and leave CUs idle.  With
// larger grids the overlap measured slower (the concurrent work disturbs the
// attention kernels' L2 sharing), and the stages run in order on the
// caller's stream as in the plain plan.
bool overlap_stages(const Plan& p) { return p.pipeline && attn_small_grid(p.S, p.U); }

// Forward, pipelined: whole stages alternate between the two streams (stage
// s on the caller's stream when s is even), so one stage's attention starts
// while the previous one's longest query blocks finish, in the CUs they
// leave idle.  Stage s's Q copy s mod 2 was last read by stage s - 2 on the
// same stream.  A stage that loads K/V into a copy first waits for the other
// stream's latest stage if that stream read the copy since its last load; a
// stage of a group loaded on the other stream waits for the load.
hipError_t fwd_pipelined(const Plan& p, const Kernels& K, const void* X, const void* Wq,
                         const void* Wk, const void* Wv, void* O, float* LSE, void* ws,
                         hipStream_t s, hipStream_t h, SyncEvents& E, const NormIn& nin) {
  hipEvent_t start = E.ev[0], kv_ready[2] = {E.ev[1], E.ev[2]}, attn_done[2] = {E.ev[3], E.ev[4]};
  const int n = static_cast<int>(p.stages.size());
  hipError_t e = order(start, s, h);  // inputs written on the caller's stream
  int load_stream[2] = {-1, -1};      // stream (0: caller's, 1: helper) of the last load into each copy
  int readers[2] = {0, 0};            // streams that read each copy since its last load (bit mask)
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    const Stage& st = p.stages[i];
    const int xi = i % 2, k = st.kvslot;
    hipStream_t x = xi == 0 ? s : h;
    if (st.load && (readers[k] & (1 << (1 - xi)))) e = hipStreamWaitEvent(x, attn_done[1 - xi], 0);
    if (e == hipSuccess) e = stage_projection(p, st, K, X, Wq, Wk, Wv, ws, x, nin, false);
    if (e == hipSuccess && st.load) {
      e = hipEventRecord(kv_ready[k], x);
      load_stream[k] = xi;
      readers[k] = 0;
    } else if (e == hipSuccess && load_stream[k] != xi) {
      e = hipStreamWaitEvent(x, kv_ready[k], 0);
    }
    readers[k] |= 1 << xi;
    if (e != hipSuccess) break;
    AttnArgs a = attn_args(p, st, ws);
    a.o = O;
    a.lse = LSE;
    e = timed(UPIPE_K_ATTN_FWD, x, [&] { return K.attn_fwd(a, x); });
    if (e == hipSuccess) e = hipEventRecord(attn_done[i % 2], x);
  }
  if (e == hipSuccess && n >= 2) e = hipStreamWaitEvent(s, attn_done[1], 0);  // join the helper stream
  return e;
}

// Backward, pipelined on small grids: whole stages alternate between the two
// streams as in the forward, so one stage's dQ (whose last query blocks run
// alone) overlaps the next stage's work.  Per stage, on its stream: the
// projection, the D pre-pass, dQ, dK/dV, the QK-norm backward and the dW and
// dX GEMMs.  Q, dQ, D and LSE*log2(e) use the stage's copy (s mod 2, last
// used by stage s - 2 on the same stream); K/V copies follow the forward's
// rule.  What stays single runs as a chain in stage order, each link waiting
// for the previous stage's: dK/dV (its fp32 sums carry across a group's
// stages), the QK-norm backward (dgamma's running sums) and the GEMMs (dX's
// running sum and the dW part sums) -- so every sum keeps its order.
hipError_t bwd_alternating(const Plan& p, const Kernels& K, const BwdIn& in, hipStream_t s,
                           hipStream_t h, SyncEvents& E, const NormIn& nin) {
  hipEvent_t start = E.ev[0], kv_ready[2] = {E.ev[1], E.ev[2]}, stage_done[2] = {E.ev[3], E.ev[4]};
  hipEvent_t dkv_done = E.ev[5], norm_done = E.ev[6], grad_done = E.ev[7];
  const int n = static_cast<int>(p.stages.size());
  hipError_t e = order(start, s, h);  // inputs written on the caller's stream
  int load_stream[2] = {-1, -1};      // stream (0: caller's, 1: helper) of the last load into each copy
  int readers[2] = {0, 0};            // streams that used each K/V copy since its last load (bit mask)
  bool k_started = false;             // dgamma_k's running sum (QK-norm)
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    const Stage& st = p.stages[i];
    const int xi = i % 2, k = st.kvslot;
    hipStream_t x = xi == 0 ? s : h;
    const bool other = i >= 1;  // the previous stage ran on the other stream
    if (st.load && (readers[k] & (1 << (1 - xi)))) e = hipStreamWaitEvent(x, stage_done[1 - xi], 0);
    if (e == hipSuccess) e = stage_projection(p, st, K, in.X, in.Wq, in.Wk, in.Wv, in.ws, x, nin, true);
    if (e == hipSuccess && st.load) {
      e = hipEventRecord(kv_ready[k], x);
      load_stream[k] = xi;
      readers[k] = 0;
    } else if (e == hipSuccess && load_stream[k] != xi) {
      e = hipStreamWaitEvent(x, kv_ready[k], 0);
    }
    readers[k] |= 1 << xi;
    if (e != hipSuccess) break;
    const AttnArgs a = bwd_args(p, st, in);
    e = timed(UPIPE_K_BWD_PRE, x, [&] { return K.bwd_pre(a, x); });
    if (e == hipSuccess) e = timed(UPIPE_K_ATTN_DQ, x, [&] { return K.attn_dq(a, x); });
    if (e == hipSuccess && other) e = hipStreamWaitEvent(x, dkv_done, 0);
    if (e == hipSuccess) e = timed(UPIPE_K_ATTN_DKV, x, [&] { return K.attn_dkv(a, x); });
    if (e == hipSuccess) e = hipEventRecord(dkv_done, x);
    if (e == hipSuccess && p.qk_norm) {
      if (other) e = hipStreamWaitEvent(x, norm_done, 0);
      if (e == hipSuccess) e = stage_norm_bwd(p, st, in, nin, i == 0, !k_started, x);
      if (e == hipSuccess) e = hipEventRecord(norm_done, x);
      k_started = k_started || st.done;
    }
    if (e == hipSuccess && other) e = hipStreamWaitEvent(x, grad_done, 0);
    if (e == hipSuccess) e = stage_gradients(p, st, K, in, i == 0, x);
    if (e == hipSuccess) e = hipEventRecord(grad_done, x);
    if (e == hipSuccess) e = hipEventRecord(stage_done[xi], x);
  }
  if (e == hipSuccess && n >= 2) e = hipStreamWaitEvent(s, stage_done[1], 0);  // join the helper stream
  return e;
}

// Backward, pipelined, with the output projection (its stage dO buffer is
// single, so stages cannot alternate).  Caller's stream: D pre-pass, dK/dV
// and dQ of each stage.  Helper stream: the projection of stage s + 1, then the dW and dX
// GEMMs of stage s, in stage order (dX keeps its one summation order).
// Copy s mod 2 of Q/K/V is free again once dQ of stage s - 1 has run; copy
// s mod 2 of dQ once dX of stage s - 2 has.  dK/dV use the K/V copy of their
// group; the group two loads back finished its dX by stage s - 2 as well.
hipError_t bwd_pipelined(const Plan& p, const Kernels& K, const BwdIn& in, hipStream_t s,
                         hipStream_t h, SyncEvents& E, const OutProj* op, const NormIn& nin) {
  hipEvent_t start = E.ev[0], proj_done[2] = {E.ev[1], E.ev[2]}, dq_done[2] = {E.ev[3], E.ev[4]},
             dx_done[2] = {E.ev[5], E.ev[6]};
  const int n = static_cast<int>(p.stages.size());
  hipError_t e = order(start, s, h);  // inputs written on the caller's stream
  if (e != hipSuccess) return e;
  e = stage_projection(p, p.stages[0], K, in.X, in.Wq, in.Wk, in.Wv, in.ws, h, nin, true);
  if (e == hipSuccess) e = hipEventRecord(proj_done[0], h);
  bool k_started = false;  // dgamma_k's running sum (QK-norm)
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    const Stage& st = p.stages[i];
    // the stage dO buffer is single: its GEMMs run on this stream, after
    // dQ of the previous stage has read it
    if (op) e = stage_dout(p, st, K, in.ws, *op, s);
    const AttnArgs a = op ? with_stage_do(p, st, in.ws, bwd_args(p, st, in)) : bwd_args(p, st, in);
    if (e == hipSuccess) e = timed(UPIPE_K_BWD_PRE, s, [&] { return K.bwd_pre(a, s); });
    if (e == hipSuccess) e = hipStreamWaitEvent(s, proj_done[i % 2], 0);
    if (e == hipSuccess && i >= 2) e = hipStreamWaitEvent(s, dx_done[i % 2], 0);
    if (e == hipSuccess) e = timed(UPIPE_K_ATTN_DKV, s, [&] { return K.attn_dkv(a, s); });
    if (e == hipSuccess) e = timed(UPIPE_K_ATTN_DQ, s, [&] { return K.attn_dq(a, s); });
    if (e == hipSuccess && p.qk_norm) {
      e = stage_norm_bwd(p, st, in, nin, i == 0, !k_started, s);
      k_started = k_started || st.done;
    }
    if (e == hipSuccess) e = hipEventRecord(dq_done[i % 2], s);
    if (e == hipSuccess && i + 1 < n) {
      if (i >= 1) e = hipStreamWaitEvent(h, dq_done[(i - 1) % 2], 0);
      if (e == hipSuccess)
        e = stage_projection(p, p.stages[i + 1], K, in.X, in.Wq, in.Wk, in.Wv, in.ws, h, nin, true);
      if (e == hipSuccess) e = hipEventRecord(proj_done[(i + 1) % 2], h);
    }
    if (e == hipSuccess) e = hipStreamWaitEvent(h, dq_done[i % 2], 0);
    if (e == hipSuccess) e = stage_gradients(p, st, K, in, i == 0, h);
    if (e == hipSuccess) e = hipEventRecord(dx_done[i % 2], h);
  }
  if (e == hipSuccess) e = hipStreamWaitEvent(s, dx_done[(n - 1) % 2], 0);  // join
  return e;
}

}  // namespace

namespace upipe {

void timing_begin(int kind, hipStream_t st) {
  if (!g_timing.load()) return;
  std::lock_guard<std::mutex> g(g_tmu);
  if (!g_timing.load()) return;
  g_open.kind = kind;
  g_open.a = take_event();
  g_open.b = take_event();
  // a failed record shows up as a failed read in upipe_timing_read
  if (g_open.a) (void)hipEventRecord(g_open.a, st);
}

void timing_end(int kind, hipStream_t st) {
  if (!g_timing.load()) return;
  std::lock_guard<std::mutex> g(g_tmu);
  if (g_open.kind != kind || !g_open.a || !g_open.b) return;
  (void)hipEventRecord(g_open.b, st);
  g_recs.push_back(g_open);
  g_open = TimingRec{-1, nullptr, nullptr};
}

}  // namespace upipe

extern "C" {

int upipe_create(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head, int U,
                 int causal, int dtype) {
  return upipe_create_ex(out, S, d_model, H, G, d_head, U, causal, dtype, 0);
}

int upipe_create_ex(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head, int U,
                    int causal, int dtype, int flags) {
  return upipe_create_rope(out, S, d_model, H, G, d_head, U, causal, dtype, flags, 0.0);
}

int upipe_create_rope(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head, int U,
                      int causal, int dtype, int flags, double rope_theta) {
  if (flags & UPIPE_QK_NORM) return UPIPE_ERR_ARG;  // needs an eps: upipe_create_opt
  const upipe_options o{flags, rope_theta, 0.0};
  return upipe_create_opt(out, S, d_model, H, G, d_head, U, causal, dtype, &o);
}

int upipe_create_opt(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head,
                     int U, int causal, int dtype, const upipe_options* opt) {
  if (!out) return UPIPE_ERR_ARG;
  *out = nullptr;
  const upipe_options o = opt ? *opt : upipe_options{0, 0.0, 0.0};
  upipe_plan* h = new (std::nothrow) upipe_plan;
  if (!h) return UPIPE_ERR_ARG;
  int rc = make_plan(h->p, S, d_model, H, G, d_head, U, causal, dtype, o.flags, o.rope_theta,
                     o.qk_norm_eps);
  if (rc != UPIPE_OK) {
    delete h;
    return rc;
  }
  *out = h;
  return UPIPE_OK;
}

void upipe_destroy(upipe_plan* p) { delete p; }

int upipe_auto_u(int64_t S, int64_t d_model, int H, int G, int d_head, int causal, int dtype,
                 size_t budget_bytes, int* U) {
  return choose_u(S, d_model, H, G, d_head, causal, dtype, budget_bytes, U);
}

size_t upipe_peak_bytes(const upipe_plan* p) {
  if (!p) return 0;
  return std::max(p->p.ws.fwd_bytes, p->p.ws.bwd_bytes);
}

size_t upipe_peak_bytes_phase(const upipe_plan* p, int phase) {
  if (!p) return 0;
  return phase == 0 ? p->p.ws.fwd_bytes : p->p.ws.bwd_bytes;
}

int upipe_num_stages(const upipe_plan* p) { return p ? static_cast<int>(p->p.stages.size()) : 0; }

int upipe_stage_info(const upipe_plan* p, int s, int* q_first, int* q_count, int* kv_first,
                     int* kv_count, int* kv_load, int* kv_done) {
  if (!p || s < 0 || s >= static_cast<int>(p->p.stages.size())) return UPIPE_ERR_ARG;
  const Stage& st = p->p.stages[s];
  if (q_first) *q_first = st.q0;
  if (q_count) *q_count = st.nq;
  if (kv_first) *kv_first = st.kv0;
  if (kv_count) *kv_count = st.nkv;
  if (kv_load) *kv_load = st.load ? 1 : 0;
  if (kv_done) *kv_done = st.done ? 1 : 0;
  return UPIPE_OK;
}

const char* upipe_strerror(int code) {
  switch (code) {
    case UPIPE_OK: return "ok";
    case UPIPE_ERR_ARG: return "invalid argument";
    case UPIPE_ERR_UNSUPPORTED: return "unsupported configuration";
    case UPIPE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case UPIPE_ERR_HIP: return "HIP call failed";
    default: return "unknown error";
  }
}

}  // extern "C"

namespace {

// Forward of every stage; `op` adds the output projection.  Arguments are
// validated by the callers.
int run_fwd(const Plan& p, const void* X, const void* Wq, const void* Wk, const void* Wv,
            void* O, float* LSE, void* ws, hipStream_t s, const OutProj* op, const NormIn& nin) {
  const Kernels K = kernels_for(p.dtype);
  if (overlap_stages(p)) {
    hipStream_t hs = nullptr;
    SyncEvents E;
    UPIPE_TRY(helper_stream(&hs));
    UPIPE_TRY(E.take());
    UPIPE_TRY(fwd_pipelined(p, K, X, Wq, Wk, Wv, O, LSE, ws, s, hs, E, nin));
  } else {
    for (const Stage& st : p.stages) {
      UPIPE_TRY(stage_projection(p, st, K, X, Wq, Wk, Wv, ws, s, nin, false));
      AttnArgs a = attn_args(p, st, ws);
      a.o = O;
      a.lse = LSE;
      UPIPE_TRY(timed(UPIPE_K_ATTN_FWD, s, [&] { return K.attn_fwd(a, s); }));
    }
  }
  if (op) UPIPE_TRY(layer_oproj(p, K, O, *op, s));  // on the caller's stream, after every stage
  return UPIPE_OK;
}

// Backward of every stage; `op` adds the output projection (dO of each stage
// from dY; in.dO unused).  Arguments are validated by the callers.
int run_bwd(const Plan& p, const BwdIn& in, hipStream_t s, const OutProj* op, const NormIn& nin) {
  const Kernels K = kernels_for(p.dtype);
  hipStream_t hs = nullptr;
  SyncEvents E;
  const bool overlap = overlap_stages(p);
  if (overlap) {  // before anything is enqueued
    UPIPE_TRY(helper_stream(&hs));
    UPIPE_TRY(E.take());
  }
  // dX needs no zero fill: the first stage's dX launch starts the running sum
  if (overlap && !op) {
    UPIPE_TRY(bwd_alternating(p, K, in, s, hs, E, nin));
  } else if (overlap) {  // the stage dO buffer is single: stages keep their order
    UPIPE_TRY(bwd_pipelined(p, K, in, s, hs, E, op, nin));
  } else {
    bool k_started = false;  // dgamma_k's running sum (QK-norm)
    for (const Stage& st : p.stages) {
      const bool first_stage = &st == &p.stages.front();
      UPIPE_TRY(stage_projection(p, st, K, in.X, in.Wq, in.Wk, in.Wv, in.ws, s, nin, true));
      if (op) UPIPE_TRY(stage_dout(p, st, K, in.ws, *op, s));
      const AttnArgs a =
          op ? with_stage_do(p, st, in.ws, bwd_args(p, st, in)) : bwd_args(p, st, in);
      UPIPE_TRY(timed(UPIPE_K_BWD_PRE, s, [&] { return K.bwd_pre(a, s); }));
      UPIPE_TRY(timed(UPIPE_K_ATTN_DKV, s, [&] { return K.attn_dkv(a, s); }));
      UPIPE_TRY(timed(UPIPE_K_ATTN_DQ, s, [&] { return K.attn_dq(a, s); }));
      if (p.qk_norm) {
        UPIPE_TRY(stage_norm_bwd(p, st, in, nin, first_stage, !k_started, s));
        k_started = k_started || st.done;
      }
      UPIPE_TRY(stage_gradients(p, st, K, in, first_stage, s));
    }
  }
  // dWo reads only the inputs dY and O; last, on the caller's stream (after
  // the pipelined path has joined its helper stream)
  if (op) UPIPE_TRY(layer_dwo(p, K, *op, in.ws, s));
  return UPIPE_OK;
}

// Empty sequence: every weight gradient is an empty sum.
int zero_weight_grads(const Plan& p, float* dWq, float* dWk, float* dWv, float* dWo,
                      hipStream_t s) {
  const size_t wq_bytes = static_cast<size_t>(p.H) * p.d * p.D * 4;
  const size_t wkv_bytes = static_cast<size_t>(p.G) * p.d * p.D * 4;
  UPIPE_TRY(timed(UPIPE_K_FILL, s, [&] { return fill_zero(dWq, wq_bytes, s); }));
  UPIPE_TRY(timed(UPIPE_K_FILL, s, [&] { return fill_zero(dWk, wkv_bytes, s); }));
  UPIPE_TRY(timed(UPIPE_K_FILL, s, [&] { return fill_zero(dWv, wkv_bytes, s); }));
  if (dWo) UPIPE_TRY(timed(UPIPE_K_FILL, s, [&] { return fill_zero(dWo, wq_bytes, s); }));
  return UPIPE_OK;
}

}  // namespace

extern "C" {

int upipe_fwd(const upipe_plan* h, const void* X, const void* Wq, const void* Wk, const void* Wv,
              void* O, float* LSE, void* ws, size_t ws_bytes, void* stream) {
  if (!h || h->p.qk_norm) return UPIPE_ERR_ARG;
  const Plan& p = h->p;
  if (p.S == 0) return UPIPE_OK;
  if (!ptr_ok(X) || !ptr_ok(Wq) || !ptr_ok(Wk) || !ptr_ok(Wv) || !ptr_ok(O) || !ptr_ok(LSE))
    return UPIPE_ERR_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < p.ws.fwd_bytes) return UPIPE_ERR_WORKSPACE;
  return run_fwd(p, X, Wq, Wk, Wv, O, LSE, ws, static_cast<hipStream_t>(stream), nullptr,
                 NormIn{});
}

int upipe_fwd_out(const upipe_plan* h, const void* X, const void* Wq, const void* Wk,
                  const void* Wv, const void* Wo, void* O, float* LSE, float* Y, void* ws,
                  size_t ws_bytes, void* stream) {
  if (!h || !h->p.out_proj || h->p.qk_norm) return UPIPE_ERR_ARG;
  const Plan& p = h->p;
  if (p.S == 0) return UPIPE_OK;
  if (!ptr_ok(X) || !ptr_ok(Wq) || !ptr_ok(Wk) || !ptr_ok(Wv) || !ptr_ok(Wo) || !ptr_ok(O) ||
      !ptr_ok(LSE) || !ptr_ok(Y))
    return UPIPE_ERR_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < p.ws.fwd_bytes) return UPIPE_ERR_WORKSPACE;
  const OutProj op{Wo, Y, nullptr, nullptr, nullptr};
  return run_fwd(p, X, Wq, Wk, Wv, O, LSE, ws, static_cast<hipStream_t>(stream), &op, NormIn{});
}

int upipe_bwd(const upipe_plan* h, const void* dO, const void* X, const void* Wq, const void* Wk,
              const void* Wv, const void* O, const float* LSE, float* dX, float* dWq, float* dWk,
              float* dWv, void* ws, size_t ws_bytes, void* stream) {
  if (!h || h->p.qk_norm) return UPIPE_ERR_ARG;
  const Plan& p = h->p;
  if (!ptr_ok(dWq) || !ptr_ok(dWk) || !ptr_ok(dWv)) return UPIPE_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.S == 0) return zero_weight_grads(p, dWq, dWk, dWv, nullptr, s);
  if (!ptr_ok(dO) || !ptr_ok(X) || !ptr_ok(Wq) || !ptr_ok(Wk) || !ptr_ok(Wv) || !ptr_ok(O) ||
      !ptr_ok(LSE) || !ptr_ok(dX))
    return UPIPE_ERR_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < p.ws.bwd_bytes) return UPIPE_ERR_WORKSPACE;
  const BwdIn in{dO, X, Wq, Wk, Wv, O, LSE, dX, dWq, dWk, dWv, ws};
  return run_bwd(p, in, s, nullptr, NormIn{});
}

int upipe_bwd_out(const upipe_plan* h, const void* dY, const void* X, const void* Wq,
                  const void* Wk, const void* Wv, const void* Wo, const void* O, const float* LSE,
                  float* dX, float* dWq, float* dWk, float* dWv, float* dWo, void* ws,
                  size_t ws_bytes, void* stream) {
  if (!h || !h->p.out_proj || h->p.qk_norm) return UPIPE_ERR_ARG;
  const Plan& p = h->p;
  if (!ptr_ok(dWq) || !ptr_ok(dWk) || !ptr_ok(dWv) || !ptr_ok(dWo)) return UPIPE_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.S == 0) return zero_weight_grads(p, dWq, dWk, dWv, dWo, s);
  if (!ptr_ok(dY) || !ptr_ok(X) || !ptr_ok(Wq) || !ptr_ok(Wk) || !ptr_ok(Wv) || !ptr_ok(Wo) ||
      !ptr_ok(O) || !ptr_ok(LSE) || !ptr_ok(dX))
    return UPIPE_ERR_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < p.ws.bwd_bytes) return UPIPE_ERR_WORKSPACE;
  const BwdIn in{nullptr, X, Wq, Wk, Wv, O, LSE, dX, dWq, dWk, dWv, ws};
  const OutProj op{Wo, nullptr, dY, O, dWo};
  return run_bwd(p, in, s, &op, NormIn{});
}

int upipe_fwd_ex(const upipe_plan* h, const upipe_fwd_io* io, void* ws, size_t ws_bytes,
                 void* stream) {
  if (!h || !io) return UPIPE_ERR_ARG;
  const Plan& p = h->p;
  // what the plan uses must be given, what it does not use must be null
  if (!need(io->q_norm, p.qk_norm) || !need(io->k_norm, p.qk_norm) || !need(io->Wo, p.out_proj) ||
      !need(io->Y, p.out_proj))
    return UPIPE_ERR_ARG;
  if (p.S == 0) return UPIPE_OK;
  if (!ptr_ok(io->X) || !ptr_ok(io->Wq) || !ptr_ok(io->Wk) || !ptr_ok(io->Wv) || !ptr_ok(io->O) ||
      !ptr_ok(io->LSE))
    return UPIPE_ERR_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < p.ws.fwd_bytes) return UPIPE_ERR_WORKSPACE;
  const OutProj op{io->Wo, io->Y, nullptr, nullptr, nullptr};
  const NormIn nin{io->q_norm, io->k_norm, nullptr, nullptr};
  return run_fwd(p, io->X, io->Wq, io->Wk, io->Wv, io->O, io->LSE, ws,
                 static_cast<hipStream_t>(stream), p.out_proj ? &op : nullptr, nin);
}

int upipe_bwd_ex(const upipe_plan* h, const upipe_bwd_io* io, void* ws, size_t ws_bytes,
                 void* stream) {
  if (!h || !io) return UPIPE_ERR_ARG;
  const Plan& p = h->p;
  if (!need(io->q_norm, p.qk_norm) || !need(io->k_norm, p.qk_norm) ||
      !need(io->dq_norm, p.qk_norm) || !need(io->dk_norm, p.qk_norm) ||
      !need(io->Wo, p.out_proj) || !need(io->dY, p.out_proj) || !need(io->dWo, p.out_proj) ||
      !need(io->dO, !p.out_proj))
    return UPIPE_ERR_ARG;
  if (!ptr_ok(io->dWq) || !ptr_ok(io->dWk) || !ptr_ok(io->dWv)) return UPIPE_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.S == 0) {
    const int rc = zero_weight_grads(p, io->dWq, io->dWk, io->dWv, io->dWo, s);
    if (rc != UPIPE_OK || !p.qk_norm) return rc;
    UPIPE_TRY(timed(UPIPE_K_FILL, s, [&] { return fill_zero(io->dq_norm, p.d * 4, s); }));
    UPIPE_TRY(timed(UPIPE_K_FILL, s, [&] { return fill_zero(io->dk_norm, p.d * 4, s); }));
    return UPIPE_OK;
  }
  if (!ptr_ok(io->X) || !ptr_ok(io->Wq) || !ptr_ok(io->Wk) || !ptr_ok(io->Wv) || !ptr_ok(io->O) ||
      !ptr_ok(io->LSE) || !ptr_ok(io->dX))
    return UPIPE_ERR_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < p.ws.bwd_bytes) return UPIPE_ERR_WORKSPACE;
  const BwdIn in{io->dO, io->X, io->Wq, io->Wk, io->Wv, io->O, io->LSE, io->dX, io->dWq, io->dWk,
                 io->dWv, ws};
  const OutProj op{io->Wo, nullptr, io->dY, io->O, io->dWo};
  const NormIn nin{io->q_norm, io->k_norm, io->dq_norm, io->dk_norm};
  return run_bwd(p, in, s, p.out_proj ? &op : nullptr, nin);
}

int upipe_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_tmu);
  g_timing.store(on != 0);
  return UPIPE_OK;
}

int upipe_timing_read(double* ms, int64_t* launches, int n) {
  std::lock_guard<std::mutex> g(g_tmu);
  int rc = UPIPE_OK;
  for (TimingRec& r : g_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      rc = UPIPE_ERR_HIP;
    if (r.kind >= 0 && r.kind < n) {
      if (ms) ms[r.kind] += t;
      if (launches) launches[r.kind] += 1;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return rc;
}

int upipe_mfma_ceiling(int waves_per_simd, int iters, double* tflops, void* stream) {
  if (!tflops || waves_per_simd < 1 || waves_per_simd > 2 || iters < 8) return UPIPE_ERR_ARG;
  return bf16::mfma_ceiling(waves_per_simd, iters, tflops, static_cast<hipStream_t>(stream)) == hipSuccess
             ? UPIPE_OK
             : UPIPE_ERR_HIP;
}

const char* upipe_kernel_name(int kind) {
  static const char* names[UPIPE_K_COUNT] = {"proj", "attn_fwd", "bwd_pre", "attn_dkv",
                                             "attn_dq", "dw", "dx", "fill",
                                             "oproj", "dout", "dwo", "norm"};
  if (kind < 0 || kind >= UPIPE_K_COUNT) return "unknown";
  return names[kind];
}

}  // extern "C"
