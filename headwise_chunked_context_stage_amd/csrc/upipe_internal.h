// upipe_internal.h -- host-side plan, stage-buffer layout and the launch
// interface between the C ABI and the kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/upipe.h"

namespace upipe {

constexpr size_t kAlign = 256;  // every workspace region starts on a 256-byte boundary

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// One stage of the head schedule: query heads [q0, q0+nq) and the KV heads
// [kv0, kv0+nkv) they read.  `load`: the stage is the first of those KV heads'
// group, so it projects K and V; `done`: it is the last, so it finishes their
// gradients.  Stages run in ascending head order; with groups contiguous this
// projects every KV head exactly once per group.  `slot` selects the copy of
// the per-stage buffers (Q, dQ) and `kvslot` the copy of the per-group ones
// (K, V, dK, dV); both are 0 unless the plan is pipelined (two copies of each).
struct Stage {
  int q0, nq;
  int kv0, nkv;
  bool load, done;
  int slot, kvslot;
};

// Byte offsets of the stage buffers inside the caller's workspace.
// The regions indexed [2] have two copies in a pipelined plan (index = the
// stage's slot or kvslot) and one otherwise ([1] == [0]).
struct WsLayout {
  size_t q[2], k[2], v[2];     // Q [U][S][d], K [kv][S][d], V [kv][S][d]   (element type)
  size_t dd[2];                // D = rowsum(dO*O) [U][S] fp32                 (backward)
  size_t lse2[2];              // LSE * log2(e) [U][S] fp32                    (backward)
  size_t dq[2];                // dQ [U][S][d] (element type)                  (backward)
  size_t dk[2], dv[2];         // dK, dV [kv][S][d] (element type)             (backward)
  size_t dk_acc, dv_acc;       // fp32 carry of dK, dV across a group's stages (bf16, U < r, no split)
  size_t kvp;                  // bf16 with dkv_split(S) == 2: the two halves' fp32 dK, dV sums of
                               // one KV head, [half][dK, dV][S][d] (also their carry when U < r)
  size_t dob;                  // dO of the stage's heads [U][S][d] (element type), from dY through
                               // the output projection (plans with UPIPE_OUT_PROJ; else 0)
  // QK-norm (plans with UPIPE_QK_NORM; else 0), backward only:
  size_t xq[2], rq[2];         // normalised query rows [U][S][d] fp32, 1/rms [U][S] fp32
  size_t xk[2], rk[2];         // the same for the stage's keys [kv][S][d], [kv][S]
  size_t gq32[2], gk32[2];     // bf16: fp32 gradients of the normalised rows before their
                               // backward, [U][S][d] and [kv][S][d] (fp32 plans use dq/dk)
  size_t pq, pk;               // per-256-token-block sums for dgamma: [U][nb][d], [kv][nb][d]
  size_t dws;                  // bf16: partial weight gradients of the token parts after the
                               // first, dw_scratch_bytes(S, D, nmax) (none when S < 8192)
  size_t fwd_bytes, bwd_bytes;
};

// QK-norm operands of the projection epilogues: chunks with kind 1 (queries)
// or 2 (keys) are normalised with gamma[kind - 1]; with `store` set, the
// normalised rows and 1/rms of chunk i go to xh[kind - 1] + idx * S * d and
// ri[kind - 1] + idx * S (the backward's recomputation keeps them).
struct NormArgs {
  const void* gamma[2];
  float* xh[2];
  float* ri[2];
  float eps;
  int store;
};

// Rotary position embedding of queries and keys (rotate-half form): the pair
// (c, c + d/2) of a row at token position i turns by the angle i * w_c with
// w_c = theta^(-2c/d).  fw[c] = w_c / (2 pi) in fp64 (turns per position), so
// a kernel takes the fractional part of i * fw[c] in fp64 and evaluates the
// sine and cosine of that fraction of a turn in fp32.
constexpr int kMaxRopePairs = 64;  // d / 2 for d <= 128
struct Rope {
  int on;
  double fw[kMaxRopePairs];
};

struct Plan {
  int64_t S, D;
  int H, G, d, U, r, causal, dtype;
  int kv_per_stage;  // max(1, U / r)
  int pipeline;      // stage s + 1's projection overlaps stage s's attention
  int out_proj;      // the workspace holds the stage dO buffer of upipe_bwd_out
  double rope_theta; // 0: no rotary embedding
  Rope rope;         // frequencies derived from rope_theta and d
  int qk_norm;       // UPIPE_QK_NORM
  double qk_eps;
  std::vector<Stage> stages;
  WsLayout ws;
  size_t elem() const { return dtype == UPIPE_BF16 ? 2 : 4; }
};

// Validates and builds; returns a UPIPE_* code.
int make_plan(Plan& p, int64_t S, int64_t D, int H, int G, int d, int U, int causal, int dtype,
              int flags = 0, double rope_theta = 0.0, double qk_eps = 0.0);

constexpr int kNormBlock = 256;  // tokens per partial sum of dgamma
int choose_u(int64_t S, int64_t D, int H, int G, int d, int causal, int dtype, size_t budget,
             int* U);

// ------------------------------------------------------------------ launch
// A list of [S][d] operand buffers with matching weight row blocks.  Used for
// the projection (out[i] = X * W[i]^T), the weight gradient
// (dW[i] = a[i]^T X) and the input gradient (dX += sum_i a[i] W[i]).
constexpr int kMaxChunks = 64;

// bf16 weight gradients: the token range (the contraction of dW = a^T X) is
// cut into dw_parts(S) parts of equal k-step counts, a number fixed by S alone
// so that every U sums in the same order.  Each part is its own fp32 sum (its
// own workgroups, so a thin stage still fills the chip); the first goes to dW,
// the others to (P - 1) scratch tiles of [d = 128][D] fp32 per chunk, and a
// fold adds parts 1 .. P - 1 to dW in that order.  A launch takes up to
// dw_batch(P) chunks (the chunks of a launch share their reads of X), so the
// scratch holds at most 16 tiles; `nmax` is the most chunks one call passes.
inline int dw_parts(int64_t S) { return S < 8192 ? 1 : static_cast<int>(S >= 32768 ? 8 : S / 4096); }
inline int dw_batch(int parts) { return parts == 1 ? kMaxChunks : (16 / (parts - 1) > 0 ? 16 / (parts - 1) : 1); }
inline size_t dw_scratch_bytes(int64_t S, int64_t D, int nmax) {
  const int P = dw_parts(S);
  const int nb = dw_batch(P) < nmax ? dw_batch(P) : nmax;
  return P == 1 ? 0 : static_cast<size_t>(P - 1) * nb * 128 * static_cast<size_t>(D) * 4;
}
struct ChunkTable {
  int n;
  uint64_t rot;               // projection: bit i set = rotate chunk i's rows (queries, keys)
  int czero;                  // dX / Y running sums: this launch starts the sum (its C input is
                              // zero and the output is not read); same bits as reading zeros
  const void* w[kMaxChunks];  // weight rows [d][D] of this chunk
  void* a[kMaxChunks];        // [S][d] activation / gradient buffer of this chunk
  float* dw[kMaxChunks];      // [d][D] fp32 weight-gradient rows (dW launches only)
  unsigned char nkind[kMaxChunks];  // projection: 0, or QK-norm with gamma[nkind - 1]
  unsigned char nidx[kMaxChunks];   // projection: row block of the chunk in NormArgs' buffers
};

// dK/dV with fewer than 512 key tiles (S <= 65408): each key tile's query
// tiles are split into an upper and a lower half, one workgroup each, so
// that the triangular causal work does not leave the longest key tile alone
// on the critical path.  Each half is its own fp32 sum (over the group's heads
// and stages), and a combine kernel adds upper + lower.  Fixed by S alone, so
// every U sums alike.
inline int dkv_split(int64_t S) { return (S + 127) / 128 < 512 ? 2 : 1; }

// Attention grids under two rounds of 256-row query blocks (x heads): the
// forward and dQ kernels then run 128-row workgroups (the same bits), and a
// pipelined plan's forward alternates stages between its two streams.
inline bool attn_small_grid(int64_t S, int nq) { return (S + 255) / 256 * nq < 512; }

struct AttnArgs {
  int64_t S;
  int H;          // total query heads (row stride of O/dO is H*d)
  int d;
  int causal;
  int nq;         // query heads in this launch
  int q_head0;    // global index of the first query head
  int r;          // query heads per KV group
  const void* q;  // Q [nq][S][d]
  const void* k;  // K of the first KV head touched, [nkv][S][d]
  const void* v;
  int kv_head0;   // global index of the first KV head in k/v
  // forward
  void* o;        // O [S][H*d]
  float* lse;     // LSE [H][S]
  // backward
  const void* dO;       // row i of head h at dO + (h - do_h0) * do_hs + i * ldo (elements):
  int64_t ldo;          //   the caller's [S][H*d]: ldo = H*d, do_hs = d, do_h0 = 0;
  int64_t do_hs;        //   a stage buffer [U][S][d]: ldo = d, do_hs = S*d, do_h0 = the
  int do_h0;            //   stage's first query head
  const void* o_in;     // [S][H*d]
  const float* lse_in;  // [H][S]
  float* dd;            // D [nq][S]
  float* lse2;          // LSE in log2 units [nq][S], written with D
  void* dq;             // dQ [nq][S][d]
  void* dk;             // dK [nkv][S][d], element type (written when the group is done)
  void* dv;
  float* dk_acc;        // fp32 carry (bf16 only), may be null when not needed
  float* dv_acc;
  int kv_split;         // bf16: dkv_split(S); with 2, dK/dV sums go to kvp (one KV head per
  float* kvp;           //   launch, [half][dK, dV][S][d] fp32) and a combine kernel finishes them
  float* dq32;          // bf16 with QK-norm: dQ goes here in fp32 (after the rotary
  float* dk32;          //   transpose) instead of dq; the finished dK likewise
  int first_of_group;   // this launch starts the group's dK/dV accumulation
  int last_of_group;    // this launch completes it
  // rotary embedding: the bf16 kernels map the gradients of the rotated
  // queries and keys back through the transposed rotation as they write
  // dQ and the finished dK
  Rope rope;
};

// Kernel launchers (one set per element type).  Return hipSuccess or the
// launch error.  `S` is the number of tokens; X is [S][D].
namespace bf16 {
// Chunks with their bit set in t.rot are rotated (rope) before rounding.
hipError_t proj(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, const Rope& rope,
                const NormArgs& nrm, hipStream_t st);
hipError_t attn_fwd(const AttnArgs& a, hipStream_t st);
hipError_t bwd_pre(const AttnArgs& a, hipStream_t st);
hipError_t attn_dkv(const AttnArgs& a, hipStream_t st);
hipError_t attn_dq(const AttnArgs& a, hipStream_t st);
// `scratch`: dw_scratch_bytes(S, D, t.n) bytes or more (may be null when that is 0).
hipError_t dw(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, float* scratch,
              hipStream_t st);
hipError_t dx(float* dX, int64_t S, int64_t D, int d, const ChunkTable& t, hipStream_t st);
// Output projection (chunks = heads ascending; a[ch] / w[ch] point at the
// head's columns of O and Wo, row stride ld = H*d):
//   oproj: Y [S][D] fp32 += sum_ch O_ch Wo_ch^T   (Y is the running sum)
//   dout:  a[ch] ([S][d], element type) = dY Wo_ch, dY [S][D]
//   dwo:   dw[ch] (head's columns of dWo, row stride ld) = dY^T O_ch
hipError_t oproj(float* Y, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                 hipStream_t st);
hipError_t dout(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                hipStream_t st);
hipError_t dwo(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
               float* scratch, hipStream_t st);
// dense MFMA stream on every CU; TFLOP/s (synchronous)
hipError_t mfma_ceiling(int waves_per_simd, int iters, double* tflops, hipStream_t st);
}  // namespace bf16
namespace f32 {
hipError_t proj(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, hipStream_t st);
hipError_t attn_fwd(const AttnArgs& a, hipStream_t st);
hipError_t bwd_pre(const AttnArgs& a, hipStream_t st);
hipError_t attn_dkv(const AttnArgs& a, hipStream_t st);
hipError_t attn_dq(const AttnArgs& a, hipStream_t st);
// `scratch` is not used (same signature as the bf16 launcher).
hipError_t dw(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, float* scratch,
              hipStream_t st);
hipError_t dx(float* dX, int64_t S, int64_t D, int d, const ChunkTable& t, hipStream_t st);
// In-place rotation of n [S][d] fp32 buffers at `buf` (consecutive): sign +1
// rotates queries/keys, -1 applies the transposed rotation to gradients.
hipError_t rope(float* buf, int n, int64_t S, int d, const Rope& r, int sign, hipStream_t st);
hipError_t oproj(float* Y, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                 hipStream_t st);
hipError_t dout(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                hipStream_t st);
hipError_t dwo(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
               float* scratch, hipStream_t st);
}  // namespace f32
hipError_t fill_zero(void* p, size_t bytes, hipStream_t st);

// QK-norm kernels (kernels_norm.hip), d = d_head <= 128.
namespace norm {
// fp32 plans: normalise n [S][d] buffers at `x` in place (x = gamma * xhat);
// xhat / rinv (may be null) keep the normalised rows and 1/rms.
hipError_t fwd_f32(float* x, int n, int64_t S, int d, const float* gamma, float eps, float* xhat,
                   float* rinv, hipStream_t st);
// Backward of n rows blocks: g [n][S][d] fp32 gradients of the normalised
// rows -> out [n][S][d] (element type `out_bf16 ? bf16 : fp32`; may alias g
// when fp32), and part [n][nb][d] (nb = ceil(S / kNormBlock)) = per-block
// sums of g * xhat.  gamma in the element type.
hipError_t bwd(const float* g, const float* xhat, const float* rinv, const void* gamma,
               int gamma_bf16, void* out, int out_bf16, float* part, int n, int64_t S, int d,
               hipStream_t st);
// dg[c] = (first ? 0 : dg[c]) + sum over n * nb partial rows in order.
hipError_t gamma_sum(float* dg, const float* part, int n, int64_t S, int d, int first,
                     hipStream_t st);
}  // namespace norm

// Kernel timing hooks (capi.cpp).
void timing_begin(int kind, hipStream_t st);
void timing_end(int kind, hipStream_t st);

}  // namespace upipe

// The opaque handle of the public header.
struct upipe_plan {
  upipe::Plan p;
};
