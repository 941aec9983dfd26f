// plan.cpp -- head schedule and stage-buffer allocator (host only).
//
// paper.rainbus.top summary of "Untied Ulysses", section 方法步骤详情: the
// layer runs in H/U stages; stage i handles heads iU .. (i+1)U-1 and the
// QKV buffers are reused by every stage, so the peak is O(U), not O(H).
// Section 技术新颖性: distinct KV heads are moved once (the GQA-aware
// schedule).  On one GPU the schedule is ascending head order: groups are
// contiguous, so a KV head is projected in the first stage of its group and
// kept until the group's last query head has been processed.
//
// Legal U on one GPU (the pages' rule "U divisible by the device count",
// section 局限与改进, concerns several devices): U divides H, and either U
// divides the group size r = H/G (a stage lies inside one group) or r divides
// U (a stage holds whole groups).  No stage ever cuts a group unevenly.
//
// Optional rotary position embedding of queries and keys (not on the pages;
// the Llama and Qwen model families that run this layer use it): rotate-half
// form with base theta.  It changes no buffer size.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "upipe_internal.h"

namespace upipe {

int make_plan(Plan& p, int64_t S, int64_t D, int H, int G, int d, int U, int causal, int dtype,
              int flags, double rope_theta, double qk_eps) {
  if ((flags & ~(UPIPE_PIPELINE | UPIPE_OUT_PROJ | UPIPE_QK_NORM)) != 0) return UPIPE_ERR_ARG;
  // rope_theta: 0 (no rotary embedding) or a finite positive base
  if (!(rope_theta >= 0.0) || !std::isfinite(rope_theta)) return UPIPE_ERR_ARG;
  // QK-norm eps: finite and >= 0 (checked only when the flag is set)
  if ((flags & UPIPE_QK_NORM) && (!(qk_eps >= 0.0) || !std::isfinite(qk_eps))) return UPIPE_ERR_ARG;
  if (S < 0 || D <= 0 || H <= 0 || G <= 0 || d <= 0 || U <= 0) return UPIPE_ERR_ARG;
  if (causal != 0 && causal != 1) return UPIPE_ERR_ARG;
  if (dtype != UPIPE_BF16 && dtype != UPIPE_F32) return UPIPE_ERR_ARG;
  if (H % G != 0) return UPIPE_ERR_ARG;
  const int r = H / G;
  if (H % U != 0) return UPIPE_ERR_ARG;
  if (!(r % U == 0 || U % r == 0)) return UPIPE_ERR_ARG;
  if (d != 64 && d != 128) return UPIPE_ERR_UNSUPPORTED;
  if (dtype == UPIPE_BF16 && d != 128) return UPIPE_ERR_UNSUPPORTED;
  if (dtype == UPIPE_BF16 && D % 128 != 0) return UPIPE_ERR_UNSUPPORTED;
  if (dtype == UPIPE_F32 && D % 64 != 0) return UPIPE_ERR_UNSUPPORTED;
  // The fp32 variant is the small exact-precision path (one thread per row).
  if (dtype == UPIPE_F32 && S > 65536) return UPIPE_ERR_UNSUPPORTED;
  // Token indices and the [S][D] / [S][H*d] offsets are 64-bit in every kernel;
  // per-row counts stay below 2^31.
  if (S > (int64_t(1) << 31) - 256) return UPIPE_ERR_UNSUPPORTED;
  if (D > (int64_t(1) << 20)) return UPIPE_ERR_UNSUPPORTED;

  p.S = S;
  p.D = D;
  p.H = H;
  p.G = G;
  p.d = d;
  p.U = U;
  p.r = r;
  p.causal = causal;
  p.dtype = dtype;
  p.kv_per_stage = std::max(1, U / r);
  p.pipeline = (flags & UPIPE_PIPELINE) ? 1 : 0;
  p.out_proj = (flags & UPIPE_OUT_PROJ) ? 1 : 0;
  p.qk_norm = (flags & UPIPE_QK_NORM) ? 1 : 0;
  p.qk_eps = p.qk_norm ? qk_eps : 0.0;
  // Rotary embedding: w_c = theta^(-2c/d) for c < d/2, kept as turns per
  // position (w_c / 2 pi) in fp64.
  p.rope_theta = rope_theta;
  std::memset(&p.rope, 0, sizeof(p.rope));
  if (rope_theta > 0.0) {
    p.rope.on = 1;
    for (int c = 0; c < d / 2; ++c)
      p.rope.fw[c] = std::pow(rope_theta, -2.0 * c / d) / (2.0 * 3.14159265358979323846);
  }

  p.stages.clear();
  int loads = 0;  // stages so far that project K and V
  for (int s = 0; s < H / U; ++s) {
    Stage st;
    st.q0 = s * U;
    st.nq = U;
    st.kv0 = st.q0 / r;
    st.nkv = p.kv_per_stage;
    if (U >= r) {
      st.load = st.done = true;
    } else {
      st.load = (st.q0 % r) == 0;
      st.done = ((st.q0 + U) % r) == 0;
    }
    if (st.load) ++loads;
    // Pipelined: consecutive stages alternate between two copies of the
    // stage buffers, and consecutive K/V loads between two copies of K/V.
    st.slot = p.pipeline ? s % 2 : 0;
    st.kvslot = p.pipeline ? (loads - 1) % 2 : 0;
    p.stages.push_back(st);
  }

  // Stage buffers: one region each, reused by every stage (two copies of
  // the per-stage regions when pipelined).
  const size_t e = p.elem();
  const size_t Sd = static_cast<size_t>(S) * d;
  const size_t nkv = p.kv_per_stage;
  WsLayout& w = p.ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const int copies = p.pipeline ? 2 : 1;
  auto take2 = [&](size_t (&at)[2], size_t bytes) {
    at[0] = take(bytes);
    at[1] = copies == 2 ? take(bytes) : at[0];
  };
  take2(w.q, U * Sd * e);
  take2(w.k, nkv * Sd * e);
  take2(w.v, nkv * Sd * e);
  w.fwd_bytes = off;
  take2(w.dd, static_cast<size_t>(U) * S * 4);
  take2(w.lse2, static_cast<size_t>(U) * S * 4);
  take2(w.dq, U * Sd * e);
  take2(w.dk, nkv * Sd * e);
  take2(w.dv, nkv * Sd * e);
  w.dk_acc = w.dv_acc = w.kvp = 0;
  if (dtype == UPIPE_BF16 && dkv_split(S) == 2) {
    w.kvp = take(4 * Sd * 4);  // two halves x (dK, dV) of one KV head, fp32
  } else if (dtype == UPIPE_BF16 && U < r) {
    w.dk_acc = take(Sd * 4);
    w.dv_acc = take(Sd * 4);
  }
  // With the output projection the backward forms each stage's dO from dY.
  w.dob = p.out_proj ? take(U * Sd * e) : 0;
  // QK-norm: the normalised rows and 1/rms of the stage's queries and keys
  // (written by the backward's projections, read by the norm's backward),
  // the fp32 gradients before that backward (bf16 only; fp32 plans keep them
  // in dQ / dK), and the per-block sums of dgamma.
  for (int c = 0; c < 2; ++c) w.xq[c] = w.rq[c] = w.xk[c] = w.rk[c] = w.gq32[c] = w.gk32[c] = 0;
  w.pq = w.pk = 0;
  if (p.qk_norm) {
    const size_t nb = (static_cast<size_t>(S) + kNormBlock - 1) / kNormBlock;
    take2(w.xq, U * Sd * 4);
    take2(w.rq, static_cast<size_t>(U) * S * 4);
    take2(w.xk, nkv * Sd * 4);
    take2(w.rk, nkv * static_cast<size_t>(S) * 4);
    if (dtype == UPIPE_BF16) {
      take2(w.gq32, U * Sd * 4);
      take2(w.gk32, nkv * Sd * 4);
    }
    w.pq = take(static_cast<size_t>(U) * nb * d * 4);
    w.pk = take(nkv * nb * d * 4);
  }
  // bf16 weight gradients: partial sums of the token parts after the first,
  // for the most chunks one call passes (a stage's heads, plus its group's K
  // and V; with the output projection, the heads of the dWo launches)
  int nmax = 0;
  for (const Stage& st : p.stages) nmax = std::max(nmax, st.nq + (st.done ? 2 * st.nkv : 0));
  if (p.out_proj) nmax = std::max(nmax, H);
  nmax = std::min(nmax, kMaxChunks);
  const size_t dws = dtype == UPIPE_BF16 ? dw_scratch_bytes(S, D, nmax) : 0;
  w.dws = dws ? take(dws) : 0;
  w.bwd_bytes = off;
  return UPIPE_OK;
}

// Chunk size from a memory budget.  The pages (paper.rainbus.top summary,
// section 独立分析的弱点) suggest choosing U from the sequence length: large U
// (few stages) for short sequences, small U (less memory) for long ones, and
// section 实验结果 reports U as a memory/throughput trade-off.  With a fixed
// budget this is the largest legal U whose workspace fits: the workspace
// grows with S * U, so a longer sequence gets a smaller U.
int choose_u(int64_t S, int64_t D, int H, int G, int d, int causal, int dtype, size_t budget,
             int* U) {
  if (!U) return UPIPE_ERR_ARG;
  *U = 0;
  if (H <= 0 || G <= 0 || H % G != 0) return UPIPE_ERR_ARG;
  const int r = H / G;
  for (int u = H; u >= 1; --u) {
    if (H % u != 0 || !(r % u == 0 || u % r == 0)) continue;
    Plan p;
    const int rc = make_plan(p, S, D, H, G, d, u, causal, dtype);
    if (rc != UPIPE_OK) return rc;  // shape errors do not depend on U
    if (std::max(p.ws.fwd_bytes, p.ws.bwd_bytes) <= budget) {
      *U = u;
      return UPIPE_OK;
    }
  }
  return UPIPE_ERR_WORKSPACE;
}

}  // namespace upipe
