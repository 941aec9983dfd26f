/* upipe.h -- C ABI of the headwise-chunked causal GQA attention layer
 * (one GPU's share), forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * The operation (pages on "Untied Ulysses: Memory-Efficient Context
 * Parallelism via Headwise Chunking"; paper.rainbus.top summary):
 *  - section 前置知识 / 分组查询注意力: H query heads, G key/value heads; every
 *    H/G consecutive query heads share one KV head (query head h reads KV head
 *    floor(h / (H/G))).
 *  - section 前置知识 / DeepSpeed Ulysses: each device computes full attention
 *    over all positions for its own subset of heads; this library is that
 *    per-device computation for one GPU's heads.
 *  - sections 核心方法 and 方法步骤详情: the layer runs in H/U stages of U heads.
 *    A stage projects X into Q, K, V of its heads, runs flash attention over
 *    the full sequence and writes its slice of the output; the same stage
 *    buffers are reused by every stage, so intermediate memory grows with U,
 *    not with H.
 *  - same page, section 技术新颖性: the GQA-aware schedule moves each distinct
 *    KV head once.  On one GPU this becomes: each KV head is projected once
 *    per group and kept while the group's query heads are processed.
 *  - the all-to-all exchanges of steps (2) and (4) are between devices and are
 *    not part of one GPU's share.
 * Readings where the pages are silent: softmax scale 1/sqrt(d_head), causal
 * mask j <= i, no bias / output projection, batch 1, natural-log LSE,
 * backward of L = sum(O * dO) with recomputation of each stage's Q, K, V.
 * A rotary position embedding of queries and keys is optional
 * (upipe_create_rope); it is off unless asked for.
 *
 * Layouts (row-major, batch 1, all tensor pointers are DEVICE pointers owned
 * by the caller; element type `dtype` unless stated):
 *   X  [S][D]            Wq [H*d][D]  (head h = rows h*d .. h*d+d-1)
 *   Wk, Wv [G*d][D]      O, dO [S][H*d]  (head h = columns h*d .. h*d+d-1)
 *   LSE [H][S] fp32      dX [S][D] fp32     dWq, dWk, dWv fp32, weight shapes
 *   ws: workspace of at least upipe_peak_bytes() bytes, 256-byte aligned.
 *
 * Results do not depend on U: every legal U gives bit-identical O, LSE, dX,
 * dWq, dWk and dWv, and repeated calls give identical bits.
 *
 * Errors: every entry point validates its arguments on the host before it
 * enqueues anything; on failure it returns a nonzero code and enqueues
 * nothing.  A failed HIP launch returns UPIPE_ERR_HIP.  Faults that happen on
 * the device surface at the caller's next synchronisation.  No entry point
 * allocates device memory or prints, and none synchronises the stream, with
 * two exceptions that exist for benchmarks: upipe_timing_read waits for the
 * timing events it reads (hipEventSynchronize), and upipe_mfma_ceiling waits
 * for its own launch.
 */
#ifndef UPIPE_H
#define UPIPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct upipe_plan upipe_plan; /* opaque, immutable after create, host memory only */

typedef enum { UPIPE_BF16 = 0, UPIPE_F32 = 1 } upipe_dtype;

enum {
  UPIPE_OK = 0,
  UPIPE_ERR_ARG = 1,         /* invalid argument: shape, U, null or misaligned pointer */
  UPIPE_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. bf16 with d_head != 128) */
  UPIPE_ERR_WORKSPACE = 3,   /* ws too small or not 256-byte aligned */
  UPIPE_ERR_HIP = 4          /* a HIP call failed */
};

/* Build a plan.  Host only: no device call, no allocation of device memory.
 *   S >= 0 tokens (S = 0 is the empty sequence), d_model = D, H query heads,
 *   G KV heads (G divides H), d_head in {64, 128} (bf16 needs 128),
 *   U query heads per stage: U divides H and (U divides H/G or H/G divides U),
 *   causal in {0, 1}, dtype a upipe_dtype.  D must be a multiple of 64 (bf16:
 *   of 128).  *out receives the plan; release it with upipe_destroy. */
int upipe_create(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head, int U,
                 int causal, int dtype);

/* Plan flags for upipe_create_ex. */
enum {
  /* Stage pipelining (the pages' suggested improvement of overlapping the
   * stages; paper.rainbus.top summary, sections 局限与改进 and 独立分析的弱点).
   * The stage buffers get two copies.  Where the attention grid is small
   * (fewer than 512 query blocks of 256 rows over a stage's U heads, e.g.
   * U = 1 at up to 64K tokens), consecutive stages overlap: the forward
   * alternates whole stages (projection and attention) between the caller's
   * stream and a second stream, so one stage's attention fills the CUs the
   * previous one's last query blocks leave idle.  The backward alternates
   * whole stages the same way (with UPIPE_OUT_PROJ, whose stage dO buffer is
   * single, it instead runs the projection of stage s + 1 and the weight-
   * and input-gradient GEMMs of stage s on the second stream while stage
   * s + 1's attention kernels run on the caller's stream).  With larger grids the stages run in order on
   * the caller's stream, as in the plain plan (overlapping them measured
   * slower there).  Every kernel, its inputs and the order of every
   * accumulation are those of the plain plan, so the results are
   * bit-identical; upipe_peak_bytes grows by one more copy of the Q, K, V
   * (and dQ, dK, dV, D and LSE) stage buffers.  The second stream (default
   * priority, one per device, created on the first pipelined call on the
   * current device, which must be the device of `stream`) and a pool of
   * events are kept until the process ends; the calls allocate no device
   * memory. */
  UPIPE_PIPELINE = 1,
  /* Output projection (upipe_fwd_out / upipe_bwd_out).  Not on the pages'
   * step list: the linear map Y = O Wo^T that follows attention in the Llama
   * and Qwen blocks, which a drop-in attention module has to include.  The
   * workspace of the backward grows by the stage's dO buffer
   * (U * S * d_head elements); upipe_fwd and upipe_bwd work as before. */
  UPIPE_OUT_PROJ = 2,
  /* QK-norm (upipe_create_opt; not on the pages: the Qwen3 attention whose
   * shape the pages train normalises each projected query and key row of a
   * head before the rotary embedding).  For a row x of d_head values:
   *   r = 1 / sqrt(sum_c x_c^2 / d_head + eps),  y_c = gamma_c * x_c * r,
   * with gamma_q [d_head] for every query head and gamma_k [d_head] for
   * every key head.  In bf16 the normalisation happens in fp32 before the
   * stage buffers' single rounding.  The backward also returns dgamma_q and
   * dgamma_k (fp32), each summed over heads ascending and 256-token blocks
   * ascending (the same bits for every U).  Such plans run only through
   * upipe_fwd_ex / upipe_bwd_ex, which take gamma; the backward's workspace
   * grows by the fp32 normalised rows of the stage's queries and keys and
   * their fp32 gradients (about 8 * S * d_head * (U + kv) bytes). */
  UPIPE_QK_NORM = 4
};

/* Options of upipe_create_opt. */
typedef struct {
  int flags;           /* a combination of UPIPE_PIPELINE, UPIPE_OUT_PROJ, UPIPE_QK_NORM */
  double rope_theta;   /* rotary embedding base, as for upipe_create_rope; 0 = none */
  double qk_norm_eps;  /* with UPIPE_QK_NORM: eps of the normalisation (finite, >= 0) */
} upipe_options;

/* upipe_create with flags (a combination of the values above; 0 gives the
 * same plan as upipe_create).  Unknown flag bits return UPIPE_ERR_ARG. */
int upipe_create_ex(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head, int U,
                    int causal, int dtype, int flags);

/* upipe_create_ex with a rotary position embedding of queries and keys.  Not
 * on the pages: the Llama and Qwen model families that run this layer rotate
 * each projected query and key row before the attention (rotate-half form).
 * For c < d_head/2 and w_c = rope_theta^(-2c/d_head), the pair (c, c+d_head/2)
 * of the row at token position i (0 .. S-1) turns by the angle i*w_c:
 *   y[c]          = x[c] cos(i w_c) - x[c + d_head/2] sin(i w_c)
 *   y[c+d_head/2] = x[c + d_head/2] cos(i w_c) + x[c] sin(i w_c)
 * Values are not rotated; the backward returns the gradients of the
 * unrotated projections (the transposed rotation).  In bf16 the rotation
 * happens in fp32 before the stage buffers' single rounding.  The angle's
 * turn fraction is taken in fp64, its sine and cosine in fp32.
 * rope_theta = 0 turns the embedding off (the plain upipe_create_ex plan);
 * a negative, NaN or infinite rope_theta returns UPIPE_ERR_ARG.  The
 * workspace does not change. */
int upipe_create_rope(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head,
                      int U, int causal, int dtype, int flags, double rope_theta);

/* upipe_create_rope with every option in one struct (opt may be NULL: no
 * options).  UPIPE_ERR_ARG for unknown flag bits, a bad rope_theta (as for
 * upipe_create_rope) or, with UPIPE_QK_NORM, a negative, NaN or infinite
 * qk_norm_eps. */
int upipe_create_opt(upipe_plan** out, int64_t S, int64_t d_model, int H, int G, int d_head,
                     int U, int causal, int dtype, const upipe_options* opt);

/* Chunk size from a memory budget (host only).  The pages (paper.rainbus.top
 * summary of "Untied Ulysses", section 独立分析的弱点) propose choosing U from
 * the sequence length, large for short sequences and small for long ones;
 * section 实验结果 describes U as a memory/throughput trade-off.  Writes to *U
 * the largest legal U (as for upipe_create) whose upipe_peak_bytes (plan
 * without flags) is at most budget_bytes, so for a fixed budget a longer S
 * gets a smaller or equal U.
 * Returns UPIPE_ERR_ARG (or UPIPE_ERR_UNSUPPORTED) for a shape upipe_create
 * rejects for every U, UPIPE_ERR_WORKSPACE when not even U = 1 fits; *U is 0
 * on failure.  U must not be NULL. */
int upipe_auto_u(int64_t S, int64_t d_model, int H, int G, int d_head, int causal, int dtype,
                 size_t budget_bytes, int* U);

/* Release a plan (NULL is ignored). */
void upipe_destroy(upipe_plan* p);

/* Workspace bytes needed by both upipe_fwd and upipe_bwd: the stage buffers
 * (Q of U heads, K and V of the KV heads a stage touches, and the backward's
 * per-stage gradient buffers).  Grows linearly with U; independent of H. */
size_t upipe_peak_bytes(const upipe_plan* p);

/* Per phase: 0 = forward only, 1 = backward. */
size_t upipe_peak_bytes_phase(const upipe_plan* p, int phase);

/* upipe_fwd, upipe_bwd, upipe_fwd_out and upipe_bwd_out return
 * UPIPE_ERR_ARG for a plan with UPIPE_QK_NORM (they have no gamma
 * arguments); upipe_fwd_ex / upipe_bwd_ex serve every plan. */

/* Forward.  Writes O [S][H*d] and LSE [H][S] (natural log of the softmax
 * denominator of the scaled scores).  Enqueued on `stream` (a hipStream_t;
 * NULL = the null stream); asynchronous. */
int upipe_fwd(const upipe_plan* p, const void* X, const void* Wq, const void* Wk, const void* Wv,
              void* O, float* LSE, void* ws, size_t ws_bytes, void* stream);

/* Backward of L = sum(O * dO), given the forward's O and LSE.  Overwrites
 * dX [S][D], dWq, dWk, dWv (fp32).  Q, K, V are recomputed stage by stage
 * from X.  Enqueued on `stream`; asynchronous. */
int upipe_bwd(const upipe_plan* p, const void* dO, const void* X, const void* Wq, const void* Wk,
              const void* Wv, const void* O, const float* LSE, float* dX, float* dWq, float* dWk,
              float* dWv, void* ws, size_t ws_bytes, void* stream);

/* The layer followed by its output projection (plan created with
 * UPIPE_OUT_PROJ, else UPIPE_ERR_ARG).  Wo is [d_model][H*d] (nn.Linear
 * "out x in", element type `dtype`).  upipe_fwd_out writes O and LSE as
 * upipe_fwd does and overwrites Y [S][d_model] (fp32) with O Wo^T, computed
 * after the last stage over all heads in ascending order with Y itself as
 * the fp32 running sum, so every U gives the same bits.  O is still the
 * caller's buffer: the backward reads it. */
int upipe_fwd_out(const upipe_plan* p, const void* X, const void* Wq, const void* Wk,
                  const void* Wv, const void* Wo, void* O, float* LSE, float* Y, void* ws,
                  size_t ws_bytes, void* stream);

/* Backward of L = sum(Y * dY), dY [S][d_model] in element type `dtype`, given
 * the forward's O and LSE.  Each stage forms its heads' dO = dY Wo (rounded
 * to the element type once, in the workspace) and runs the attention
 * backward with it; overwrites dX, dWq, dWk, dWv as upipe_bwd does and
 * dWo [d_model][H*d] (fp32) with dY^T O (one pass over all heads, since it
 * needs only the inputs dY and O). */
int upipe_bwd_out(const upipe_plan* p, const void* dY, const void* X, const void* Wq,
                  const void* Wk, const void* Wv, const void* Wo, const void* O, const float* LSE,
                  float* dX, float* dWq, float* dWk, float* dWv, float* dWo, void* ws,
                  size_t ws_bytes, void* stream);

/* The forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same results as upipe_fwd (the same
 * kernels run); the stage buffers live in a static device array of
 * upipe_noalloc_max_bytes() bytes (256 MiB) that each GPU the library runs
 * on holds from the first call on it until the process ends.  The call
 * allocates nothing.  `stream` must belong to the current device.
 * Returns UPIPE_ERR_WORKSPACE when upipe_peak_bytes_phase(p, 0) exceeds the
 * array, UPIPE_ERR_ARG for a pipelined plan (UPIPE_PIPELINE) or a stream of
 * another device, and otherwise what upipe_fwd returns.  Every call on one
 * GPU uses the same array: calls that overlap in time on one GPU (two
 * streams, two host threads) race.  Nothing in the array has to start at
 * zero; a call never reads what an earlier one left there. */
int upipe_fwd_noalloc(const upipe_plan* p, const void* X, const void* Wq, const void* Wk,
                      const void* Wv, void* O, float* LSE, void* stream);

/* Size in bytes of the static array upipe_fwd_noalloc works in. */
size_t upipe_noalloc_max_bytes(void);

/* Tensors of one forward call of upipe_fwd_ex (device pointers, caller
 * owned; layouts and element types as for upipe_fwd / upipe_fwd_out).
 * Members a plan does not use must be NULL. */
typedef struct {
  const void* X;
  const void* Wq;
  const void* Wk;
  const void* Wv;
  const void* q_norm; /* UPIPE_QK_NORM: gamma_q [d_head], element type */
  const void* k_norm; /* UPIPE_QK_NORM: gamma_k [d_head], element type */
  const void* Wo;     /* UPIPE_OUT_PROJ: [d_model][H*d] */
  void* O;            /* [S][H*d] */
  float* LSE;         /* [H][S] */
  float* Y;           /* UPIPE_OUT_PROJ: [S][d_model] fp32 */
} upipe_fwd_io;

/* Tensors of one backward call of upipe_bwd_ex.  dO is the gradient of O
 * ([S][H*d]); with UPIPE_OUT_PROJ the plan takes dY ([S][d_model]) instead
 * and dO must be NULL.  Outputs are overwritten. */
typedef struct {
  const void* dO;
  const void* dY;
  const void* X;
  const void* Wq;
  const void* Wk;
  const void* Wv;
  const void* q_norm;
  const void* k_norm;
  const void* Wo;
  const void* O;
  const float* LSE;
  float* dX;
  float* dWq;
  float* dWk;
  float* dWv;
  float* dq_norm; /* UPIPE_QK_NORM: dgamma_q [d_head] fp32 */
  float* dk_norm; /* UPIPE_QK_NORM: dgamma_k [d_head] fp32 */
  float* dWo;     /* UPIPE_OUT_PROJ: [d_model][H*d] fp32 */
} upipe_bwd_io;

/* Forward / backward of any plan (every flag combination): what upipe_fwd,
 * upipe_bwd, upipe_fwd_out and upipe_bwd_out do, plus QK-norm.  A required
 * pointer that is NULL or misaligned, or an unused one that is not NULL,
 * returns UPIPE_ERR_ARG before anything is enqueued. */
int upipe_fwd_ex(const upipe_plan* p, const upipe_fwd_io* io, void* ws, size_t ws_bytes,
                 void* stream);
int upipe_bwd_ex(const upipe_plan* p, const upipe_bwd_io* io, void* ws, size_t ws_bytes,
                 void* stream);

/* Text for an error code (static storage). */
const char* upipe_strerror(int code);

/* ---- plan introspection (host only) ---- */

/* Number of stages, H/U. */
int upipe_num_stages(const upipe_plan* p);

/* Stage s: its query heads [q_first, q_first + q_count), the KV heads it
 * touches [kv_first, kv_first + kv_count), whether it projects them (first
 * stage of their group: kv_load = 1) and whether it completes them (last
 * stage of their group: kv_done = 1).  Returns UPIPE_ERR_ARG for a bad s. */
int upipe_stage_info(const upipe_plan* p, int s, int* q_first, int* q_count, int* kv_first,
                     int* kv_count, int* kv_load, int* kv_done);

/* ---- kernel timing (for benchmarks) ----
 * When enabled, every kernel launch is bracketed by hipEvents recorded on the
 * stream it is launched on.  upipe_timing_read waits for those events, adds
 * each launch's duration (ms) and count to ms[kind] and launches[kind] for
 * kind < n, then forgets them.  Process-wide; not for concurrent callers. */
enum {
  UPIPE_K_PROJ = 0,     /* stage Q/K/V projection GEMM */
  UPIPE_K_ATTN_FWD = 1, /* attention forward */
  UPIPE_K_BWD_PRE = 2,  /* D = rowsum(dO * O) */
  UPIPE_K_ATTN_DKV = 3, /* attention backward, dK and dV */
  UPIPE_K_ATTN_DQ = 4,  /* attention backward, dQ */
  UPIPE_K_DW = 5,       /* weight-gradient GEMM */
  UPIPE_K_DX = 6,       /* input-gradient GEMM */
  UPIPE_K_FILL = 7,     /* zero fill */
  UPIPE_K_OPROJ = 8,    /* output projection Y += O Wo^T */
  UPIPE_K_DOUT = 9,     /* dO = dY Wo */
  UPIPE_K_DWO = 10,     /* dWo = dY^T O */
  UPIPE_K_NORM = 11,    /* QK-norm backward and its weight-gradient sums */
  UPIPE_K_COUNT = 12
};
int upipe_timing_enable(int on);
int upipe_timing_read(double* ms, int64_t* launches, int n);
const char* upipe_kernel_name(int kind);

/* ---- measured matrix-core ceiling (for benchmarks) ----
 * Runs a dense bf16 MFMA stream on every CU (v_mfma_f32_32x32x16_bf16, four
 * independent accumulator chains per wave, operands in registers, no memory
 * traffic) with `waves_per_simd` waves per SIMD (1..2), `iters` x 4 MFMAs per
 * wave (iters rounded down to a multiple of 4), on `stream` (a hipStream_t,
 * may be null), waits for it, and writes the achieved TFLOP/s (2*32*32*16
 * flop per MFMA) to *tflops.  The operands are pseudo-random bf16 values with
 * random mantissas: the power the matrix cores draw, and so the clock they
 * sustain, depends on the data (constant operands run about 10% faster).
 * Allocates no device memory.  UPIPE_ERR_ARG for bad arguments, UPIPE_ERR_HIP
 * on a HIP failure.  This is the practical ceiling the attention kernels are
 * compared against next to the published dense peak. */
int upipe_mfma_ceiling(int waves_per_simd, int iters, double* tflops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_H */
