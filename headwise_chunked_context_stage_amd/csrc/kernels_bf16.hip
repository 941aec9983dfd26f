// kernels_bf16.hip -- bf16 kernels of the stage loop for gfx950 (CDNA4).
//
// Every dense contraction runs on v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32
// accumulation).  Operand layout of that instruction, as used throughout:
//   A (32 x 16, M x K): lane l supplies row m = l % 32 and the 8 k-slots
//                       8*(l/32) .. 8*(l/32)+7 (one 16-byte register quad);
//   B (16 x 32, K x N): lane l supplies column n = l % 32 and the same slots;
//   C (32 x 32 fp32):   lane l holds column l % 32; register i holds row
//                       8*(i/4) + 4*(l/32) + (i%4).
// A and B pair their k-slots identically, so a contraction may visit its k
// indices in any fixed order.  This is what lets an fp32 C result feed the
// next product straight from registers: the 8 registers 8t..8t+7 of a C block
// in lane half h hold the rows 16t + {4h..4h+3, 8+4h..8+4h+3}, and an operand
// read from LDS must present the same rows in its slots 8h..8h+7 ("slot
// order").  Operands whose contraction index runs down the rows of their
// source tile are read with the transposing LDS reads (ds_read_b64_tr_b16),
// which deliver exactly that order; an operand read along rows is stored with
// its columns permuted to match (the dX GEMM's A tile).  No kernel transposes
// in registers.
//
// Attention (flash formulation; the per-stage attention of the pages,
// paper.rainbus.top summary of "Untied Ulysses", section 方法步骤详情 step (3)):
// scores s = q.k / sqrt(d), softmax in the log2 domain with the hardware exp2,
// online max/sum in fp32, LSE returned in natural log.  Backward recomputes P
// from LSE: P = exp(s - LSE), dS = P (dP - D), D = rowsum(dO * O).
//
// Rounding points (bf16, round-to-nearest-even): stage Q/K/V, O, P and dS at
// the MFMA inputs, dQ/dK/dV before the weight/input-gradient GEMMs, and (with
// the output projection) the stage's dO.  The optional rotary embedding is
// applied in fp32 before the rounding of Q/K and of dQ/dK.  All accumulation
// is fp32.  No atomics: every output element has one owner and a fixed
// summation order, so results are identical run to run and for every U.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "upipe_internal.h"
#include "bf16_common.h"
#include "rope_device.h"

namespace upipe {
namespace {

// ===================================================================== GEMMs
// 128 x 128 output tile, 64-wide k steps, 4 waves as 2 x 2 (64 x 64 each),
// LDS double-buffered with register prefetch.
constexpr int GB = 128, GK = 64, GS = GK + 8;  // tile, k step, LDS row stride (elements)
constexpr int GBUF = 2 * GB * GS;             // elements per buffer (two operand tiles)

// ---- projection: out[i][c] = sum_k X[i][k] W[c][k] for one head (d = 128).
// X streams from HBM: global loads run NRR = 4 k-steps ahead of their LDS
// store through a ring of register sets, so each has several steps of MFMA
// time to arrive (one step ahead, the loop waited on HBM latency).
// Chunks marked in t.rot (queries and keys under a rotary embedding) are
// rotated, and chunks with t.nkind set (QK-norm) RMS-normalised and scaled
// by gamma first, in fp32 before their single rounding to bf16.
__global__ __launch_bounds__(256, 2) void proj_kernel(const u16* __restrict__ X, int64_t S,
                                                      int64_t D, ChunkTable t, int nrb, Rope rope,
                                                      NormArgs nrm) {
  __shared__ __attribute__((aligned(16))) u16 lds[2 * GBUF];
  const int total = nrb * t.n;
  const int lid = xcd_remap(blockIdx.x, total);
  const int rb = lid / t.n, ch = lid % t.n;
  const u16* W = static_cast<const u16*>(t.w[ch]);
  u16* out = static_cast<u16*>(t.a[ch]);
  const int64_t i0 = static_cast<int64_t>(rb) * GB;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;

  constexpr int NRR = 4;
  const int nk = static_cast<int>(D / GK);
  u32x4 rx[NRR][4], rw[NRR][4];
  // The loads are unconditional (k-steps past the end reload the last one,
  // rows past S reload row S - 1, zeroed when stored; S >= 1 here, since the
  // entry points launch nothing for an empty sequence): a load behind a branch
  // leaves the compiler's wait counting at the join unable to trust later
  // loads, and it then waits for the whole ring, the loads just issued included.
  const bool full = i0 + GB <= S;
  auto load = [&](int set, int kb) {
    const int64_t k0 = static_cast<int64_t>(min(kb, nk - 1)) * GK;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = tid / 8 + 32 * m, chunk = tid % 8;
      const int64_t gi = min(i0 + row, S - 1);
      rx[set][m] = ld16(X + gi * D + k0 + chunk * 8);
      rw[set][m] = ld16(W + static_cast<int64_t>(row) * D + k0 + chunk * 8);
    }
  };
  auto store = [&](int set, int b) {
    u16* xs = lds + b * GBUF;
    u16* ws = xs + GB * GS;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = tid / 8 + 32 * m, chunk = tid % 8;
      const u32x4 x = full || i0 + row < S ? rx[set][m] : u32x4{0, 0, 0, 0};
      st16(xs + row * GS + chunk * 8, x);
      st16(ws + row * GS + chunk * 8, rw[set][m]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = zero16();

  // k-step kb's data sits in register set kb % NRR until its LDS store.
#pragma unroll
  for (int i = 0; i < NRR; ++i) load(i, i);
  store(0, 0);
  load(0, NRR);
  __syncthreads();
  auto body = [&](int kb, auto setc) {  // setc = (kb + 1) % NRR, a compile-time constant
    constexpr int SN = decltype(setc)::value;
    const int cur = kb & 1;
    const u16* xs = lds + cur * GBUF;
    const u16* ws = xs + GB * GS;
#pragma unroll
    for (int t4 = 0; t4 < GK / 16; ++t4) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = frag(xs + (64 * wm + 32 * mb + col) * GS + 16 * t4 + 8 * hf);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) fb[nb] = frag(ws + (64 * wn + 32 * nb + col) * GS + 16 * t4 + 8 * hf);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (kb + 1 < nk) store(SN, cur ^ 1);
    load(SN, kb + 1 + NRR);  // the set just stored takes k-step kb + 1 + NRR
    __syncthreads();
  };
  int kb = 0;
  for (; kb + NRR <= nk; kb += NRR) {
    body(kb, std::integral_constant<int, 1 % NRR>{});
    body(kb + 1, std::integral_constant<int, 2 % NRR>{});
    body(kb + 2, std::integral_constant<int, 3 % NRR>{});
    if constexpr (NRR > 3) body(kb + 3, std::integral_constant<int, 4 % NRR>{});
  }
  if (kb < nk) body(kb, std::integral_constant<int, 1 % NRR>{});
  if (kb + 1 < nk) body(kb + 1, std::integral_constant<int, 2 % NRR>{});
  if (NRR > 3 && kb + 2 < nk) body(kb + 2, std::integral_constant<int, 3 % NRR>{});
  const bool rot = (t.rot >> ch) & 1;
  const int nkd = t.nkind[ch];
  if (rot || nkd) {
    // Rotated or normalised chunk: C (fp32) -> LDS tile [128][132]; each
    // thread then reads 8 consecutive columns of a row and the 8 columns d/2
    // away, (QK-norm) scales both by gamma / rms of the row -- the 16 threads
    // of a row sum their squares with an xor butterfly, which leaves every
    // one of them the same sum --, rotates the pairs and stores 8 bf16
    // (16 bytes).  The column group is fixed per thread, so its 8
    // frequencies and gamma values are read once.
    constexpr int CF = GB + 4;
    float* cf = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 64 * wm + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
          cf[row * CF + 64 * wn + 32 * nb + col] = acc[mb][nb][i];
        }
    __syncthreads();
    const int chunk = tid % 16, c0 = 8 * chunk;
    const bool upper = chunk >= 8;  // columns d/2 .. d-1
    double fw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) fw[k] = rope.fw[(c0 % 64) + k];
    float go[8], gp[8];  // gamma at the own and the partner columns
    if (nkd) {
      const u16* gam = static_cast<const u16*>(nrm.gamma[nkd - 1]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        go[k] = __uint_as_float(static_cast<unsigned>(gam[c0 + k]) << 16);
        gp[k] = __uint_as_float(static_cast<unsigned>(gam[(c0 ^ 64) + k]) << 16);
      }
    }
    float* xh = nkd && nrm.store ? nrm.xh[nkd - 1] + static_cast<int64_t>(t.nidx[ch]) * S * DH : nullptr;
    float* ri = nkd && nrm.store ? nrm.ri[nkd - 1] + static_cast<int64_t>(t.nidx[ch]) * S : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int row = tid / 16 + 16 * m;
      const int64_t gi = i0 + row;
      // the 16 threads of a row (one 16-lane group) skip it together, so the
      // butterfly below only ever combines lanes that all take part
      if (gi >= S) continue;
      const float* own = cf + row * CF + c0;
      const float* other = cf + row * CF + (c0 ^ 64);
      float xo[8], xp[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xo[k] = own[k];
        xp[k] = other[k];
      }
      if (nkd) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += xo[k] * xo[k];
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) ss += __shfl_xor(ss, msk);
        const float r = 1.f / sqrtf(ss * (1.f / DH) + nrm.eps);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          xo[k] *= r;
          xp[k] *= r;
        }
        if (xh) {
          st16(xh + gi * DH + c0, __builtin_bit_cast(u32x4, f32x4{xo[0], xo[1], xo[2], xo[3]}));
          st16(xh + gi * DH + c0 + 4, __builtin_bit_cast(u32x4, f32x4{xo[4], xo[5], xo[6], xo[7]}));
          if (chunk == 0) ri[gi] = r;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          xo[k] *= go[k];
          xp[k] *= gp[k];
        }
      }
      float y[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (rot) {
          float cs, sn;
          rope_cs(gi, fw[k], cs, sn);
          float lo = upper ? xp[k] : xo[k], hi = upper ? xo[k] : xp[k];
          rope_fwd(lo, hi, cs, sn);
          y[k] = upper ? hi : lo;
        } else {
          y[k] = xo[k];
        }
      }
      u32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = pack2(y[2 * k], y[2 * k + 1]);
      st16(out + gi * DH + c0, v);
    }
    return;
  }
  // Epilogue: C (bf16) -> LDS tile [128][136] -> coalesced 16-byte stores.
  constexpr int CS = GB + 8;
  u16* cs = lds;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * wm + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
        const int c = 64 * wn + 32 * nb + col;
        cs[row * CS + c] = __builtin_bit_cast(u16, static_cast<__bf16>(acc[mb][nb][i]));
      }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = tid + 256 * m, row = e / 16, chunk = e % 16;
    const int64_t gi = i0 + row;
    if (gi < S) st16(out + gi * DH + chunk * 8, ld16(cs + row * CS + chunk * 8));
  }
}

// ---- weight gradient: dW[c][k] = sum_i A[i][c] X[i][k] (one chunk, K = S).
// Both operands have the contraction index i along the rows of their source
// ([S][128] activation-gradient chunk, [S][D] input), so both are copied
// row-major into LDS in the attention tile layout (64 rows of 128 columns,
// 16-byte chunks, no transposes) and read as column operands with the
// transposing LDS reads; A and B then present the same k-slot order.  A launch
// has few output tiles and a long contraction, so K is split twice, at points
// that depend on S only: into dw_parts(S) parts of the k-steps, one workgroup
// each (part 0 writes dW, part p > 0 scratch tile p - 1 of its chunk, and
// dw_fold_kernel adds the parts in order), and inside a workgroup into two
// halves, summed by two groups of four waves and added in that order through
// LDS.
namespace dwk {
constexpr int ROWS = 64;            // contraction rows per k-step
constexpr int TILE = ROWS * RS;     // one operand tile
constexpr int NRR = 3;              // k-steps of global loads in flight
}  // namespace dwk

// TR (the output projection's weight gradient): A has row stride `ld`
// (a head's columns of O [S][H*d]) and the result is stored transposed,
// dW[k][c] at t.dw[ch] + k * ld + c (dWo [d_model][H*d]).  A scratch tile
// holds a part in the output's layout with its own row stride: [128][D], or
// [D][128] for TR.
template <bool TR>
__global__ __launch_bounds__(512, 1) void dw_kernel(const u16* __restrict__ X, int64_t S, int64_t D,
                                                    ChunkTable t, int ncb, int64_t ld, int nparts,
                                                    float* __restrict__ scratch) {
  using namespace dwk;
  __shared__ __attribute__((aligned(16))) u16 lds[2][2][2 * TILE];  // [group][buffer][A tile, X tile]
  // logical id = (part, column block, chunk), chunk fastest: the chunks of a
  // column block read the same X rows; each XCD takes a contiguous range
  const int per_part = ncb * t.n;
  const int lid = xcd_remap(blockIdx.x, per_part * nparts);
  const int part = lid / per_part, rem = lid % per_part;
  const int cb = rem / t.n, ch = rem % t.n;
  const u16* A = static_cast<const u16*>(t.a[ch]);
  float* dW = part == 0 ? t.dw[ch] : scratch + (static_cast<int64_t>(part - 1) * t.n + ch) * GB * D;
  const int64_t ldw = TR ? (part == 0 ? ld : GB) : D;  // row stride of dW's layout
  const int64_t k0 = static_cast<int64_t>(cb) * GB;  // column block of D
  const int grp = threadIdx.x / 256, tid = threadIdx.x % 256;
  const int wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  // staging: thread tid moves rows tid/16 + 16 m (m < 4), 16-byte chunk tid % 16,
  // of the A tile and of the X tile
  const int srow = tid >> 4, sc = tid & 15;

  u32x4 rr[NRR][8];
  const int64_t nk_all = (S + ROWS - 1) / ROWS;
  const int p0 = static_cast<int>(nk_all * part / nparts);  // this part's k-steps [p0, p1)
  const int p1 = static_cast<int>(nk_all * (part + 1) / nparts);
  const int half = (p1 - p0 + 1) / 2;
  const int kfirst = p0 + (grp ? half : 0);       // first k-step of this group
  const int nk = grp ? p1 - p0 - half : half;     // k-steps of this group
  const int nk_max = half;                        // rounds run by both groups
  auto load = [&](int set, int kb) {
    const int64_t s0 = static_cast<int64_t>(kfirst + kb) * ROWS;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t gi = s0 + srow + 16 * m;
      const bool in = kb < nk && gi < S;
      rr[set][m] = in ? ld16(A + gi * (TR ? ld : DH) + sc * 8) : u32x4{0, 0, 0, 0};
      rr[set][4 + m] = in ? ld16(X + gi * D + k0 + sc * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int set, int b) {
    u16* at = lds[grp][b];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      st16(at + toff(srow + 16 * m, sc * 8), rr[set][m]);
      st16(at + TILE + toff(srow + 16 * m, sc * 8), rr[set][4 + m]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) acc[a2][b2] = zero16();

  // k-step kb's data sits in register set kb % NRR until its LDS store.
  // Steps beyond a group's range load zeros and are not accumulated.
  load(0, 0);
  load(1, 1);
  load(2, 2);
  store(0, 0);
  load(0, 3);
  __syncthreads();
  auto body = [&](int kb, auto setc) {  // setc = (kb + 1) % NRR, a compile-time constant
    constexpr int SN = decltype(setc)::value;
    const int cur = kb & 1;
    if (kb < nk) {
      const TileAddr ta = tile_addr(lds[grp][cur], lane);
      const TileAddr tx = tile_addr(lds[grp][cur] + TILE, lane);
#pragma unroll
      for (int t4 = 0; t4 < ROWS / 16; ++t4) {
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fa[mb] = col_frag(ta, 16 * t4, 64 * wm + 32 * mb);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) fb[nb] = col_frag(tx, 16 * t4, 64 * wn + 32 * nb);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(fa[mb], fb[nb], acc[mb][nb]);
      }
    }
    if (kb + 1 < nk_max) store(SN, cur ^ 1);
    // the set just stored takes k-step kb + 1 + NRR
    if (kb + 1 + NRR < nk_max) load(SN, kb + 1 + NRR);
    __syncthreads();
  };
  int kb = 0;
  for (; kb + NRR <= nk_max; kb += NRR) {
    body(kb, std::integral_constant<int, 1>{});
    body(kb + 1, std::integral_constant<int, 2>{});
    body(kb + 2, std::integral_constant<int, 0>{});
  }
  if (kb < nk_max) body(kb, std::integral_constant<int, 1>{});
  if (kb + 1 < nk_max) body(kb + 1, std::integral_constant<int, 2>{});

  // second half to LDS (fp32, C layout per lane), then first + second in that order
  float* red = reinterpret_cast<float*>(lds[1]);  // the second group's buffers
  if (grp == 1) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4*>(red + (((wave * 4 + mb * 2 + nb) * 4 + i4) * 64 + lane) * 4) =
              f32x4{acc[mb][nb][4 * i4], acc[mb][nb][4 * i4 + 1], acc[mb][nb][4 * i4 + 2], acc[mb][nb][4 * i4 + 3]};
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(red + (((wave * 4 + mb * 2 + nb) * 4 + i4) * 64 + lane) * 4);
          if constexpr (TR) {  // registers 4 i4 .. 4 i4 + 3 hold four consecutive c
            const int c = 64 * wm + 32 * mb + 8 * i4 + 4 * hf;
            const int64_t k = k0 + 64 * wn + 32 * nb + col;
            *reinterpret_cast<f32x4*>(dW + k * ldw + c) =
                f32x4{acc[mb][nb][4 * i4] + o[0], acc[mb][nb][4 * i4 + 1] + o[1],
                      acc[mb][nb][4 * i4 + 2] + o[2], acc[mb][nb][4 * i4 + 3] + o[3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * i4 + e;
              const int c = 64 * wm + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
              const int64_t k = k0 + 64 * wn + 32 * nb + col;
              dW[static_cast<int64_t>(c) * ldw + k] = acc[mb][nb][i] + o[e];
            }
          }
        }
  }
}

// dW of each chunk = part 0 (in dW) + part 1 + ... + part P - 1 (scratch), in
// that order.  Grid (float4 groups of a chunk's 128 x D block / 256, chunks).
template <bool TR>
__global__ __launch_bounds__(256) void dw_fold_kernel(ChunkTable t, const float* __restrict__ scratch,
                                                      int64_t D, int64_t ld, int nparts) {
  const int ch = blockIdx.y;
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;  // index in the tile
  if (e >= GB * D) return;
  // tile layout [128][D] (dW rows), or [D][128] for TR (dW at k * ld + c)
  const int64_t out = TR ? (e / GB) * ld + e % GB : e;
  f32x4 v = *reinterpret_cast<const f32x4*>(t.dw[ch] + out);
  for (int p = 1; p < nparts; ++p) {
    const f32x4 s = *reinterpret_cast<const f32x4*>(
        scratch + (static_cast<int64_t>(p - 1) * t.n + ch) * GB * D + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += s[j];
  }
  *reinterpret_cast<f32x4*>(t.dw[ch] + out) = v;
}

// ---- input gradient: dX[i][k] += sum over chunks (table order) of
// sum_c A[i][c] W[c][k].  dX itself is the fp32 running sum (the MFMA C input).
// The W tile (64 rows c x 128 columns k) is copied row-major in the attention
// tile layout and read as column operands with the transposing LDS reads,
// which present c in "slot order" (lane half h: c = 4h..4h+3, 8+4h..8+4h+3 of
// each 16); the A tile (128 rows i x 64 columns c) is stored with the middle
// 8-byte blocks of every 16-column group swapped, so that its plain row reads
// present c in the same order.  No in-register transposes.
namespace dxk {
constexpr int WT = 64 * RS;  // W tile (64 rows of 128 columns)
constexpr int AT = GB * GS;  // A tile (128 rows of 64 columns, row stride GS)
}  // namespace dxk

__global__ __launch_bounds__(256, 2) void dx_kernel(float* __restrict__ dX, int64_t S, int64_t D,
                                                    ChunkTable t, int nrb, int ncb) {
  using namespace dxk;
  __shared__ __attribute__((aligned(16))) u16 lds[2 * (AT + WT)];
  // Each XCD takes a contiguous range of tiles and walks it in panels of
  // 8 row blocks x 8 column blocks: the ~64 workgroups in flight on one XCD
  // then share 8 A row panels and 8 W column panels (about 3 MB, within its
  // L2) instead of touching every W column panel for 2 row blocks.  Rows
  // past the last whole panel keep the row-major order.
  constexpr int PR = 8, PC = 8;
  const int lid = xcd_remap(blockIdx.x, nrb * ncb);
  int rb, cb;
  if (ncb % PC == 0 && lid < (nrb / PR) * PR * ncb) {
    const int p = lid / (PR * ncb), q = lid % (PR * ncb);
    const int w = q % (PR * PC);
    rb = p * PR + w % PR;
    cb = (q / (PR * PC)) * PC + w / PR;
  } else {
    rb = lid / ncb;
    cb = lid % ncb;
  }
  const int64_t i0 = static_cast<int64_t>(rb) * GB;
  const int64_t k0 = static_cast<int64_t>(cb) * GB;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;

  // A: thread tid moves 16-column groups (row tid / 4 + 64 m, group tid % 4), m < 2;
  // W: rows tid / 16 + 16 m (m < 4), 16-byte chunk tid % 16.  Global loads run
  // NRR k-steps ahead of their LDS store through a ring of register sets (a
  // stage has few k-steps, 2 per chunk, each too short to hide a load).
  constexpr int NRR = 3;
  const int arow = tid >> 2, agrp = tid & 3;
  const int wrow = tid >> 4, wc = tid & 15;
  const int nsteps = t.n * (DH / GK);
  u32x4 ra[NRR][2][2], rw[NRR][4];
  auto load = [&](int set, int step) {
    if (step >= nsteps) return;
    const int ch = step / (DH / GK), c0 = (step % (DH / GK)) * GK;
    const u16* Ap = static_cast<const u16*>(t.a[ch]);
    const u16* Wp = static_cast<const u16*>(t.w[ch]);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int64_t gi = i0 + arow + 64 * m;
      const u16* src = Ap + gi * DH + c0 + 16 * agrp;
      ra[set][m][0] = gi < S ? ld16(src) : u32x4{0, 0, 0, 0};
      ra[set][m][1] = gi < S ? ld16(src + 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      rw[set][m] = ld16(Wp + static_cast<int64_t>(c0 + wrow + 16 * m) * D + k0 + wc * 8);
  };
  auto store = [&](int set, int b) {
    u16* as = lds + b * (AT + WT);
    u16* wt = as + AT;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      // logical columns [0-3 | 4-7] [8-11 | 12-15] -> physical [0-3 | 8-11] [4-7 | 12-15]
      const u32x4 lo = {ra[set][m][0][0], ra[set][m][0][1], ra[set][m][1][0], ra[set][m][1][1]};
      const u32x4 hi = {ra[set][m][0][2], ra[set][m][0][3], ra[set][m][1][2], ra[set][m][1][3]};
      u16* dst = as + (arow + 64 * m) * GS + 16 * agrp;
      st16(dst, lo);
      st16(dst + 8, hi);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(wt + toff(wrow + 16 * m, wc * 8), rw[set][m]);
  };

  // the first k-steps' operands, then the running dX (the C input), all in flight together.
  // C element (mb, nb, i) is row 64 wm + 32 mb + 8 (i / 4) + 4 hf + i % 4, column
  // 64 wn + 32 nb + col of the tile: a per-lane offset plus a wave-uniform row offset
  // (a scalar address) plus 32 nb.
#pragma unroll
  for (int i = 0; i < NRR; ++i) load(i, i);
  float* const ctile = dX + i0 * D;
  const int coff = (64 * wm + 4 * hf) * static_cast<int>(D) + static_cast<int>(k0) + 64 * wn + col;
  const bool cfull = i0 + GB <= S;  // no row of the tile past S
  const int crow_lim = static_cast<int>(S - i0) - (64 * wm + 4 * hf);  // row r of the lane is in when r < lim
  auto crow = [&](int mb, int i) { return 32 * mb + 8 * (i / 4) + (i % 4); };
  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* rp = ctile + static_cast<int64_t>(crow(mb, i)) * D;
        const bool in = cfull || crow(mb, i) < crow_lim;
        acc[mb][nb][i] = (in && !t.czero) ? rp[coff + 32 * nb] : 0.f;
      }

  store(0, 0);
  load(0, NRR);
  __syncthreads();
  // step sidx's data sits in register set sidx % NRR until its LDS store
  auto body = [&](int sidx, auto setc) {  // setc = (sidx + 1) % NRR, a compile-time constant
    constexpr int SN = decltype(setc)::value;
    const int cur = sidx & 1;
    const u16* as = lds + cur * (AT + WT);
    const TileAddr tw = tile_addr(lds + cur * (AT + WT) + AT, lane);
#pragma unroll
    for (int t4 = 0; t4 < GK / 16; ++t4) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = frag(as + (64 * wm + 32 * mb + col) * GS + 16 * t4 + 8 * hf);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) fb[nb] = col_frag(tw, 16 * t4, 64 * wn + 32 * nb);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (sidx + 1 < nsteps) store(SN, cur ^ 1);
    load(SN, sidx + 1 + NRR);  // the set just stored takes step sidx + 1 + NRR
    __syncthreads();
  };
  static_assert(NRR == 3 || NRR == 4, "the loop below is unrolled for 3 or 4 register sets");
  int sidx = 0;
  for (; sidx + NRR <= nsteps; sidx += NRR) {
    body(sidx, std::integral_constant<int, 1 % NRR>{});
    body(sidx + 1, std::integral_constant<int, 2 % NRR>{});
    body(sidx + 2, std::integral_constant<int, 3 % NRR>{});
    if constexpr (NRR > 3) body(sidx + 3, std::integral_constant<int, 4 % NRR>{});
  }
  if (sidx < nsteps) body(sidx, std::integral_constant<int, 1 % NRR>{});
  if (sidx + 1 < nsteps) body(sidx + 1, std::integral_constant<int, 2 % NRR>{});
  if (NRR > 3 && sidx + 2 < nsteps) body(sidx + 2, std::integral_constant<int, 3 % NRR>{});
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float* rp = ctile + static_cast<int64_t>(crow(mb, i)) * D;
        if (cfull || crow(mb, i) < crow_lim) rp[coff + 32 * nb] = acc[mb][nb][i];
      }
}

// ---- output projection: Y[i][k] += sum over chunks (heads ascending) of
// sum_c A[i][c] B[k][c], A = a head's columns of O [S][H*d], B = the same
// columns of Wo [d_model][H*d] (both with row stride ld).  Both operands run
// along the contraction in memory, so both tiles (128 rows x 64 columns) are
// staged row-major and read with plain row reads, as in the projection; Y is
// the fp32 running sum across stages (the MFMA C input), as dX is, so every
// U sums in the same order.  Tiles in panels per XCD as in dx_kernel.
__global__ __launch_bounds__(256, 2) void oproj_kernel(float* __restrict__ Y, int64_t S, int64_t D,
                                                       ChunkTable t, int nrb, int ncb, int64_t ld) {
  __shared__ __attribute__((aligned(16))) u16 lds[2 * GBUF];
  constexpr int PR = 8, PC = 8;
  const int lid = xcd_remap(blockIdx.x, nrb * ncb);
  int rb, cb;
  if (ncb % PC == 0 && lid < (nrb / PR) * PR * ncb) {
    const int p = lid / (PR * ncb), q = lid % (PR * ncb);
    const int w = q % (PR * PC);
    rb = p * PR + w % PR;
    cb = (q / (PR * PC)) * PC + w / PR;
  } else {
    rb = lid / ncb;
    cb = lid % ncb;
  }
  const int64_t i0 = static_cast<int64_t>(rb) * GB;
  const int64_t k0 = static_cast<int64_t>(cb) * GB;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  // thread tid moves 16-column groups (row tid / 4 + 64 m, group tid % 4), m < 2, of both tiles
  const int arow = tid >> 2, agrp = tid & 3;
  u32x4 ra[2][2], rb2[2][2];
  auto load = [&](int step) {
    const int ch = step / (DH / GK), c0 = (step % (DH / GK)) * GK;
    const u16* Ap = static_cast<const u16*>(t.a[ch]);
    const u16* Bp = static_cast<const u16*>(t.w[ch]);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int64_t gi = i0 + arow + 64 * m;
      const u16* src = Ap + gi * ld + c0 + 16 * agrp;
      ra[m][0] = gi < S ? ld16(src) : u32x4{0, 0, 0, 0};
      ra[m][1] = gi < S ? ld16(src + 8) : u32x4{0, 0, 0, 0};
      const u16* wsrc = Bp + (k0 + arow + 64 * m) * ld + c0 + 16 * agrp;
      rb2[m][0] = ld16(wsrc);
      rb2[m][1] = ld16(wsrc + 8);
    }
  };
  auto store = [&](int b) {
    u16* as = lds + b * GBUF;
    u16* bs = as + GB * GS;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      st16(as + (arow + 64 * m) * GS + 16 * agrp, ra[m][0]);
      st16(as + (arow + 64 * m) * GS + 16 * agrp + 8, ra[m][1]);
      st16(bs + (arow + 64 * m) * GS + 16 * agrp, rb2[m][0]);
      st16(bs + (arow + 64 * m) * GS + 16 * agrp + 8, rb2[m][1]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t gi = i0 + 64 * wm + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
        const int64_t k = k0 + 64 * wn + 32 * nb + col;
        acc[mb][nb][i] = (gi < S && !t.czero) ? Y[gi * D + k] : 0.f;
      }

  const int nsteps = t.n * (DH / GK);
  load(0);
  store(0);
  __syncthreads();
  for (int sidx = 0; sidx < nsteps; ++sidx) {
    const int cur = sidx & 1;
    if (sidx + 1 < nsteps) load(sidx + 1);
    const u16* as = lds + cur * GBUF;
    const u16* bs = as + GB * GS;
#pragma unroll
    for (int t4 = 0; t4 < GK / 16; ++t4) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = frag(as + (64 * wm + 32 * mb + col) * GS + 16 * t4 + 8 * hf);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) fb[nb] = frag(bs + (64 * wn + 32 * nb + col) * GS + 16 * t4 + 8 * hf);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (sidx + 1 < nsteps) store(cur ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t gi = i0 + 64 * wm + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
        const int64_t k = k0 + 64 * wn + 32 * nb + col;
        if (gi < S) Y[gi * D + k] = acc[mb][nb][i];
      }
}

// ---- gradient of the attention output through the output projection:
// out[i][c] = sum_k dY[i][k] B[k][c] for one head (chunk), B = the head's
// columns of Wo [d_model][H*d] (row stride ld), K = d_model.  B's
// contraction index runs down its rows, so its tile (64 rows k x 128 columns
// c) is staged row-major and read with the transposing LDS reads, and the dY
// tile is stored with the middle 8-byte blocks of every 16-column group
// swapped to present the same k-slot order, as in dx_kernel.  The result is
// rounded to bf16 once, through LDS, into the stage buffer [S][d].
__global__ __launch_bounds__(256, 2) void dout_kernel(const u16* __restrict__ dY, int64_t S,
                                                      int64_t D, ChunkTable t, int nrb, int64_t ld) {
  using namespace dxk;
  __shared__ __attribute__((aligned(16))) u16 lds[2 * (AT + WT)];
  const int total = nrb * t.n;
  const int lid = xcd_remap(blockIdx.x, total);
  const int rb = lid / t.n, ch = lid % t.n;
  const u16* Bp = static_cast<const u16*>(t.w[ch]);
  u16* out = static_cast<u16*>(t.a[ch]);
  const int64_t i0 = static_cast<int64_t>(rb) * GB;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  const int arow = tid >> 2, agrp = tid & 3;
  const int wrow = tid >> 4, wc = tid & 15;
  u32x4 ra[2][2], rw[4];
  auto load = [&](int step) {
    const int64_t kk = static_cast<int64_t>(step) * GK;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int64_t gi = i0 + arow + 64 * m;
      const u16* src = dY + gi * D + kk + 16 * agrp;
      ra[m][0] = gi < S ? ld16(src) : u32x4{0, 0, 0, 0};
      ra[m][1] = gi < S ? ld16(src + 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) rw[m] = ld16(Bp + (kk + wrow + 16 * m) * ld + wc * 8);
  };
  auto store = [&](int b) {
    u16* as = lds + b * (AT + WT);
    u16* wt = as + AT;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4 lo = {ra[m][0][0], ra[m][0][1], ra[m][1][0], ra[m][1][1]};
      const u32x4 hi = {ra[m][0][2], ra[m][0][3], ra[m][1][2], ra[m][1][3]};
      u16* dst = as + (arow + 64 * m) * GS + 16 * agrp;
      st16(dst, lo);
      st16(dst + 8, hi);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(wt + toff(wrow + 16 * m, wc * 8), rw[m]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();
  const int nsteps = static_cast<int>(D / GK);
  load(0);
  store(0);
  __syncthreads();
  for (int sidx = 0; sidx < nsteps; ++sidx) {
    const int cur = sidx & 1;
    if (sidx + 1 < nsteps) load(sidx + 1);
    const u16* as = lds + cur * (AT + WT);
    const TileAddr tw = tile_addr(lds + cur * (AT + WT) + AT, lane);
#pragma unroll
    for (int t4 = 0; t4 < GK / 16; ++t4) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = frag(as + (64 * wm + 32 * mb + col) * GS + 16 * t4 + 8 * hf);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) fb[nb] = col_frag(tw, 16 * t4, 64 * wn + 32 * nb);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (sidx + 1 < nsteps) store(cur ^ 1);
    __syncthreads();
  }
  // C (bf16) -> LDS tile [128][136] -> coalesced 16-byte stores
  constexpr int CS = GB + 8;
  u16* cs = lds;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * wm + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
        const int c = 64 * wn + 32 * nb + col;
        cs[row * CS + c] = __builtin_bit_cast(u16, static_cast<__bf16>(acc[mb][nb][i]));
      }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = tid + 256 * m, row = e / 16, chunk = e % 16;
    const int64_t gi = i0 + row;
    if (gi < S) st16(out + gi * DH + chunk * 8, ld16(cs + row * CS + chunk * 8));
  }
}

// ---- forward.  Workgroup: 256 query rows of one head (8 waves x 32 rows);
// key/value tiles of 64 rows, double-buffered, copied once for all 8 waves.
// Each wave computes S^T = K Q^T (lane = query row, registers = keys): row
// statistics are per lane plus one exchange between the lane halves, and
// O^T = V^T P^T keeps the query in the lane, so the online rescale is a
// per-lane scalar.  Waves w and w + 4 share a SIMD and run "ping-pong": each
// alternates a matrix phase and a softmax phase, one barrier phase apart, so
// one wave's MFMAs meet the other's exponentials.
//
// Small grids (fewer than two rounds of 256-row workgroups, e.g. one head of
// a 32K-token sequence) run the same code with 4 waves and 128 query rows per
// workgroup, two workgroups per CU: each wave still owns 32 query rows and
// visits the same key tiles in the same order with the same arithmetic, so
// the results are bit-identical to the 8-wave form; the waves then run matrix
// and softmax phases in turn and the other workgroup on the CU fills the gaps.
namespace fw {
constexpr int BN = 64;
constexpr int TILE = BN * 128;  // elements of one swizzled 64-row tile
constexpr float kLazy = 8.f;    // keep a stale running max while the new one exceeds it by <= 8 (log2)
}  // namespace fw

template <int NW>  // waves per workgroup: 8 (256 query rows, ping-pong) or 4 (128 rows)
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_kernel(AttnArgs a) {
  using namespace fw;
  constexpr int BM = 32 * NW;
  __shared__ __attribute__((aligned(256))) u16 kbuf[2 * TILE];
  __shared__ __attribute__((aligned(256))) u16 vbuf[2 * TILE];
  const int64_t S = a.S;
  const int nqb = static_cast<int>((S + BM - 1) / BM);
  // longest rows first; per round of 256 workgroups, each XCD takes 32
  // consecutive (query block, head) pairs, so a GQA group's heads share the
  // XCD's L2 while they stream the same K/V tiles (HBM fetch per launch
  // 9.0 -> 2.3 GB against one head per XCD pair)
  const int lid = xcd_snake(blockIdx.x, gridDim.x);
  const int qb = nqb - 1 - lid / a.nq;
  const int u = lid % a.nq;
  const int h = a.q_head0 + u;
  const int gl = h / a.r - a.kv_head0;
  const u16* Q = static_cast<const u16*>(a.q) + static_cast<int64_t>(u) * S * DH;
  const u16* K = static_cast<const u16*>(a.k) + static_cast<int64_t>(gl) * S * DH;
  const u16* V = static_cast<const u16*>(a.v) + static_cast<int64_t>(gl) * S * DH;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  // 8 waves: waves w and w + 4 share a SIMD, and the second runs one phase later
  const bool first = NW == 4 || wave < 4;
  // copy index within the group: with 8 waves the first waves copy K tiles and
  // the second V tiles; with 4 waves every wave copies both
  const int st = tid & 255;
  const int64_t qfirst = static_cast<int64_t>(qb) * BM;
  const int64_t wq0 = qfirst + 32 * wave;
  const int64_t myq = wq0 + col;
  const float c = kLog2e / sqrtf(static_cast<float>(DH));

  bf16x8 qf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    qf[t] = __builtin_bit_cast(bf16x8, myq < S ? ld16(Q + myq * DH + 16 * t + 8 * hf) : u32x4{0, 0, 0, 0});
#pragma unroll
  for (int t = 0; t < 8; ++t) settle(qf[t]);

  const int64_t kv_end = a.causal ? min(S, qfirst + BM) : S;
  const int ntiles = static_cast<int>((kv_end + BN - 1) / BN);
  auto active = [&](int j) { return !a.causal || static_cast<int64_t>(j) * BN <= wq0 + 31; };

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 s[2];   // S^T of the tile between its matrix phase and its softmax
  bf16x8 pb[4];  // P^T of the tile between its softmax and the next matrix phase

  // Matrix phase of tile j: O^T += V^T P^T of tile j - 1, then S^T = K Q^T of tile j.
  auto matrix_phase = [&](int j) {
    // raised priority: the SIMD issues this wave's MFMAs ahead of the partner
    // wave's softmax arithmetic (2% faster than equal priorities)
    __builtin_amdgcn_s_setprio(1);
    if (j >= 1 && active(j - 1)) {
      // step k4 outermost so the four accumulators alternate (each still
      // sums k4 = 0..3 in order); V operands requested 3 groups ahead.
      const SwzAddr va = swz_addr(vbuf + ((j - 1) & 1) * TILE, lane);
      bf16x8 fc[4];
      auto load_c = [&](int gi) { return swz_col_frag(va, 16 * (gi / 4), 32 * (gi % 4)); };
      fc[0] = load_c(0);
      fc[1] = load_c(1);
      fc[2] = load_c(2);
#pragma unroll
      for (int gi = 0; gi < 16; ++gi) {
        if (gi + 3 < 16) fc[(gi + 3) % 4] = load_c(gi + 3);
        __builtin_amdgcn_sched_barrier(0);
        oacc[gi % 4] = mfma(fc[gi % 4], pb[gi / 4], oacc[gi % 4]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (j < ntiles && active(j)) {
      // two accumulator chains; the K operands of step t + 2 are requested
      // before the MFMAs of step t are issued
      const SwzAddr ka = swz_addr(kbuf + (j & 1) * TILE, lane);
      s[0] = s[1] = zero16();
      bf16x8 fa[3][2];
      auto load_a = [&](int t, bf16x8 (&f)[2]) {
        f[0] = swz_row_frag(ka, 0, t);
        f[1] = swz_row_frag(ka, 1, t);
      };
      load_a(0, fa[0]);
      load_a(1, fa[1]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t + 2 < 8) load_a(t + 2, fa[(t + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        s[0] = mfma(fa[t % 3][0], qf[t], s[0]);
        s[1] = mfma(fa[t % 3][1], qf[t], s[1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Softmax phase of tile j: mask, lazy running max, P = exp2(S c - m), row sums.
  auto softmax_phase = [&](int j) {
    if (j < 0 || j >= ntiles || !active(j)) return;
    const int64_t kv0 = static_cast<int64_t>(j) * BN;
    const bool need_mask = a.causal ? (kv0 + BN - 1 > wq0) : (kv0 + BN > S);
    if (need_mask) {
      // key kv0 + n is masked when n > myq - kv0 (causal) or n >= S - kv0
      const int lim = static_cast<int>(a.causal ? min(myq - kv0, static_cast<int64_t>(BN)) :
                                                  min(S - 1 - kv0, static_cast<int64_t>(BN)));
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int n = 32 * b + 8 * (i / 4) + 4 * hf + (i % 4);
          if (n > lim) s[b][i] = -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[b][i]);
    mt = max_xor32(mt) * c;
    // Lazy running max: rescale only when the tile max exceeds it by more
    // than kLazy (p <= 2^kLazy stays exact in fp32 and in bf16's exponent).
    const float m_new = (mt > m_run + kLazy) ? mt : m_run;
    if (__ballot(m_new != m_run)) {
      const float alpha = ex2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d4][i] *= alpha;
      m_run = m_new;
    }
    float ls = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = ex2(__builtin_fmaf(s[b][i], c, -m_run));
        s[b][i] = p;
        ls += p;
      }
    l_run += ls;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) pb[k4] = pack8(s[k4 / 2], k4 % 2);
  };

  // Ping-pong: each wave alternates a matrix phase and a softmax phase, and
  // the second wave of a SIMD runs one phase behind the first, so one wave's
  // MFMAs overlap the other's exponentials.  Phases are separated by
  // workgroup barriers.  K(j) is read in phases 2j (first waves) and 2j + 1
  // (second waves); V(j) in phases 2j + 2 and 2j + 3.  Tile copies: the first
  // waves copy K tiles, the second V tiles (swizzled), 16 rows per wave, by
  // 4-row direct global-to-LDS copies, all at the start of the wave's softmax
  // phase: the matrix phase bounds each phase, and issuing a copy costs the
  // issuing wave tens of cycles.  K(j + 1) is issued in phase 2j + 1 and
  // complete at its end; V(j) is issued in phase 2j and complete at the end
  // of 2j + 1.
  const int wv = __builtin_amdgcn_readfirstlane(wave) & 3;
  // per-lane parts of the 4-row copies into the swizzled tiles: row lane / 16
  // of the four, chunk (lane % 16) ^ (4 (lane / 16) + q)
  const unsigned swx = 16u * ((lane & 15) ^ (4 * (lane >> 4))), rq = (lane >> 4) * 256u;
  // half `part` (rows 8 part .. 8 part + 7 of the wave's 16, two 4-row
  // copies); a tile that runs past S is copied whole, through registers, with part 0
  auto copy_tile = [&](const u16* src, int j, u16* dst, int part) {
    const int64_t r0 = static_cast<int64_t>(j) * BN;
    if (r0 + BN <= S) {
      const u16* g = src + (r0 + 16 * wv) * DH;
      const unsigned d = lds_byte_addr(dst) + static_cast<unsigned>(16 * wv * 256);
#pragma unroll
      for (int q = 2 * part; q < 2 * part + 2; ++q) dma_rows4(g + 4 * q * DH, d + 1024u * q, rq + (swx ^ (16u * q)));
    } else if (part == 0) {
      TileLoad<BN * 16 / 256, 256> tl;
      tl.load(src, DH, r0, S, st);
#pragma unroll
      for (int m = 0; m < BN * 16 / 256; ++m) st16(dst + swz_off((st >> 4) + 16 * m, st & 15), tl.r[m]);
    }
  };
  if (first) {
    copy_tile(K, 0, kbuf, 0);
    copy_tile(K, 0, kbuf, 1);
  }
  dma_wait();
  __syncthreads();
  if constexpr (NW == 4) {
    // no partner wave: K(j + 1) and V(j) are copied while tile j runs
    for (int j = 0; j <= ntiles; ++j) {
      if (j + 1 < ntiles) {
        copy_tile(K, j + 1, kbuf + ((j + 1) & 1) * TILE, 0);
        copy_tile(K, j + 1, kbuf + ((j + 1) & 1) * TILE, 1);
      }
      if (j < ntiles) {
        copy_tile(V, j, vbuf + (j & 1) * TILE, 0);
        copy_tile(V, j, vbuf + (j & 1) * TILE, 1);
      }
      matrix_phase(j);
      softmax_phase(j);
      dma_wait();
      __syncthreads();
    }
  } else if (first) {
    for (int j = 0; j <= ntiles; ++j) {
      matrix_phase(j);
      __syncthreads();
      if (j + 1 < ntiles) {
        copy_tile(K, j + 1, kbuf + ((j + 1) & 1) * TILE, 0);
        copy_tile(K, j + 1, kbuf + ((j + 1) & 1) * TILE, 1);
      }
      softmax_phase(j);
      dma_wait();
      __syncthreads();
    }
  } else {
    for (int j = 0; j <= ntiles; ++j) {
      if (j < ntiles) {
        copy_tile(V, j, vbuf + (j & 1) * TILE, 0);
        copy_tile(V, j, vbuf + (j & 1) * TILE, 1);
      }
      softmax_phase(j - 1);
      __syncthreads();
      matrix_phase(j);
      dma_wait();
      __syncthreads();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (myq < S) {
    u16* O = static_cast<u16*>(a.o) + myq * static_cast<int64_t>(a.H) * DH + static_cast<int64_t>(h) * DH;
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 v;
        v[0] = pack2(oacc[d4][4 * g4 + 0] * inv, oacc[d4][4 * g4 + 1] * inv);
        v[1] = pack2(oacc[d4][4 * g4 + 2] * inv, oacc[d4][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2*>(O + 32 * d4 + 8 * g4 + 4 * hf) = v;
      }
    if (hf == 0) a.lse[static_cast<int64_t>(h) * S + myq] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---- D = rowsum(dO * O) for the stage's heads (fp32), and the LSE in log2
// units for the dK/dV pass, which copies both into LDS unchanged.  16 lanes
// per row.
__global__ __launch_bounds__(256) void bwd_pre_kernel(AttnArgs a) {
  const int u = blockIdx.y;
  const int h = a.q_head0 + u;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + threadIdx.x / 16;
  const int part = threadIdx.x % 16;
  float acc = 0.f;
  if (row < a.S) {
    const int64_t off = row * static_cast<int64_t>(a.H) * DH + static_cast<int64_t>(h) * DH + part * 8;
    const int64_t goff = (h - a.do_h0) * a.do_hs + row * a.ldo + part * 8;
    const u32x4 g = ld16(static_cast<const u16*>(a.dO) + goff);
    const u32x4 o = ld16(static_cast<const u16*>(a.o_in) + off);
    const bf16x8 gb = __builtin_bit_cast(bf16x8, g), ob = __builtin_bit_cast(bf16x8, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<float>(gb[e]) * static_cast<float>(ob[e]);
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (row < a.S && part == 0) {
    a.dd[static_cast<int64_t>(u) * a.S + row] = acc;
    a.lse2[static_cast<int64_t>(u) * a.S + row] = a.lse_in[static_cast<int64_t>(h) * a.S + row] * kLog2e;
  }
}

// ---- dQ.  Workgroup: 256 query rows of one head (8 waves x 32 rows); key
// tiles of 64 rows, copied once for all 8 waves.  LDS holds two pairs of K/V
// tiles: the waves run two tiles between barriers while the next pair is
// copied in.  Orientation as in the forward (lane = query row): S^T and dP^T
// from registers Q, dO against K and V row operands, then dQ^T += K^T dS^T
// with K read as a column operand of the same tile.  The tiles are swizzled
// and filled by 4-row direct copies issued by the first wave of each SIMD:
// with two waves per SIMD the first (older) wave finishes its tiles well
// ahead of the second, so it has the time to issue them.
// Small grids run the same code with 4 waves (128 query rows, two
// workgroups per CU) and one K/V tile pair between barriers: each wave's rows,
// tiles and arithmetic are those of the 8-wave form, so the bits are too.
namespace dqk {
constexpr int BN = 64;
constexpr int TILE = BN * 128;  // swizzled 64-row tile (elements)
constexpr int BUF = 2 * TILE;   // K and V
}  // namespace dqk

template <int NW>  // waves per workgroup: 8 (256 query rows) or 4 (128 rows)
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_dq_kernel(AttnArgs a) {
  using namespace dqk;
  constexpr int BM = 32 * NW, NT = 64 * NW;
  __shared__ __attribute__((aligned(256))) u16 lds[(NW == 8 ? 4 : 2) * BUF];
  const int64_t S = a.S;
  const int nqb = static_cast<int>((S + BM - 1) / BM);
  const int lid = xcd_snake(blockIdx.x, gridDim.x);  // as in the forward (9.2 -> 2.5 GB fetched)
  const int qb = nqb - 1 - lid / a.nq;
  const int u = lid % a.nq;
  const int h = a.q_head0 + u;
  const int gl = h / a.r - a.kv_head0;
  const u16* K = static_cast<const u16*>(a.k) + static_cast<int64_t>(gl) * S * DH;
  const u16* V = static_cast<const u16*>(a.v) + static_cast<int64_t>(gl) * S * DH;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t qfirst = static_cast<int64_t>(qb) * BM;
  const int64_t wq0 = qfirst + 32 * wave;
  const int64_t myq = wq0 + col;
  const float tau = 1.f / sqrtf(static_cast<float>(DH));
  const float c = kLog2e * tau;

  bf16x8 qf[8], gf[8];
  {
    const u16* Q = static_cast<const u16*>(a.q) + static_cast<int64_t>(u) * S * DH;
    const u16* dO = static_cast<const u16*>(a.dO) + (h - a.do_h0) * a.do_hs;
    const int64_t ldo = a.ldo;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qf[t] = __builtin_bit_cast(bf16x8, myq < S ? ld16(Q + myq * DH + 16 * t + 8 * hf) : u32x4{0, 0, 0, 0});
      gf[t] = __builtin_bit_cast(bf16x8, myq < S ? ld16(dO + myq * ldo + 16 * t + 8 * hf) : u32x4{0, 0, 0, 0});
    }
  }
  float lse2 = myq < S ? a.lse_in[static_cast<int64_t>(h) * S + myq] * kLog2e : INFINITY;
  float Dq = myq < S ? a.dd[static_cast<int64_t>(u) * S + myq] : 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    settle(qf[t]);
    settle(gf[t]);
  }
  settle(lse2);
  settle(Dq);

  const int64_t kv_end = a.causal ? min(S, qfirst + BM) : S;
  const int ntiles = static_cast<int>((kv_end + BN - 1) / BN);

  // Copies: waves 0..3 each move rows 16 w .. 16 w + 15 of the K and V tiles,
  // four 4-row copies per tile.  A tile that runs past S is staged through
  // registers by every thread (rows beyond S are zero).
  unsigned voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = (lane >> 4) * 256u + 16u * ((lane & 15) ^ (4 * (lane >> 4) + q));
  auto copy_tile = [&](const u16* src, int j, u16* dst) {  // waves 0..3, whole tiles only
    const int64_t r0 = static_cast<int64_t>(j) * BN + 16 * wv;
    const unsigned d = lds_byte_addr(dst) + static_cast<unsigned>(16 * wv * 256);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma_rows4(src + (r0 + 4 * q) * DH, d + 1024u * q, voff[q]);
  };
  auto stage_regs = [&](const u16* src, int j, u16* dst) {  // every thread, synchronous
    const int64_t r0 = static_cast<int64_t>(j) * BN;
#pragma unroll
    for (int m = 0; m < BN * 16 / NT; ++m) {
      const int e = tid + NT * m, row = e >> 4, ck = e & 15;
      const u32x4 v = r0 + row < S ? ld16(src + (r0 + row) * DH + 8 * ck) : u32x4{0, 0, 0, 0};
      st16(dst + swz_off(row, ck), v);
    }
  };
  auto whole = [&](int j) { return static_cast<int64_t>(j) * BN + BN <= S; };
  // tiles j and j + 1 (when they exist) into pair slot p
  auto issue_pair = [&](int j, int p) {
    const bool w0 = j < ntiles && whole(j), w1 = j + 1 >= ntiles || whole(j + 1);
    if (w0 && w1) {
      if (wv < 4) {
        copy_tile(K, j, lds + 2 * p * BUF);
        copy_tile(V, j, lds + 2 * p * BUF + TILE);
        if (j + 1 < ntiles) {
          copy_tile(K, j + 1, lds + (2 * p + 1) * BUF);
          copy_tile(V, j + 1, lds + (2 * p + 1) * BUF + TILE);
        }
      }
    } else {
      if (j < ntiles) {
        stage_regs(K, j, lds + 2 * p * BUF);
        stage_regs(V, j, lds + 2 * p * BUF + TILE);
      }
      if (j + 1 < ntiles) {
        stage_regs(K, j + 1, lds + (2 * p + 1) * BUF);
        stage_regs(V, j + 1, lds + (2 * p + 1) * BUF + TILE);
      }
    }
  };

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = zero16();

  // 4 waves: tile j (K and V) in slot j & 1, copied one tile ahead
  auto issue_one = [&](int j, int slot) {
    if (whole(j)) {
      copy_tile(K, j, lds + slot * BUF);
      copy_tile(V, j, lds + slot * BUF + TILE);
    } else {
      stage_regs(K, j, lds + slot * BUF);
      stage_regs(V, j, lds + slot * BUF + TILE);
    }
  };
  if constexpr (NW == 4) {
    if (ntiles > 0) issue_one(0, 0);
  } else {
    issue_pair(0, 0);
  }
  dma_wait();
  __syncthreads();
  auto process = [&](int j, int cur) {
    const int64_t kv0 = static_cast<int64_t>(j) * BN;
    const bool active = !a.causal || kv0 <= wq0 + 31;
    if (active) {
      const SwzAddr ks = swz_addr(lds + cur * BUF, lane);
      const SwzAddr vs = swz_addr(lds + cur * BUF + TILE, lane);
      const bool need_mask = a.causal ? (kv0 + BN - 1 > wq0) : (kv0 + BN > S);
      // key kv0 + j is masked when j > lim
      const int lim = static_cast<int>(a.causal ? min(myq - kv0, static_cast<int64_t>(BN)) :
                                                  min(S - 1 - kv0, static_cast<int64_t>(BN)));
      // two 32-key halves, one after the other (fewer live registers); each
      // dQ^T column block still sums its four 16-key steps in order
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x16 s = zero16(), dp = zero16();
        bf16x8 fa[2][2];
        auto load_a = [&](int t, bf16x8 (&f)[2]) {
          f[0] = swz_row_frag(ks, b, t);
          f[1] = swz_row_frag(vs, b, t);
        };
        // raised priority for the S / dP products: the other wave on the
        // SIMD is then usually in its exponentials (1% faster)
        __builtin_amdgcn_s_setprio(1);
        load_a(0, fa[0]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (t + 1 < 8) load_a(t + 1, fa[(t + 1) % 2]);
          __builtin_amdgcn_sched_barrier(0);
          s = mfma(fa[t % 2][0], qf[t], s);
          dp = mfma(fa[t % 2][1], gf[t], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = ex2(__builtin_fmaf(s[i], c, -lse2));
        if (need_mask) {  // wave-uniform: only tiles that cross the diagonal or the end
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * b + 8 * (i / 4) + 4 * hf + (i % 4) > lim) s[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = s[i] * (dp[i] - Dq);
        const bf16x8 ds[2] = {pack8(dp, 0), pack8(dp, 1)};
        // step outermost: four alternating accumulators, each summing its
        // 16-key steps in order; K operands requested 2 groups ahead
        bf16x8 fc[3];
        auto load_c = [&](int gi) { return swz_col_frag(ks, 32 * b + 16 * (gi / 4), 32 * (gi % 4)); };
        fc[0] = load_c(0);
        fc[1] = load_c(1);
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
          if (gi + 2 < 8) fc[(gi + 2) % 3] = load_c(gi + 2);
          __builtin_amdgcn_sched_barrier(0);
          dq[gi % 4] = mfma(fc[gi % 3], ds[gi / 4], dq[gi % 4]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  if constexpr (NW == 4) {
    for (int j = 0; j < ntiles; ++j) {
      if (j + 1 < ntiles) issue_one(j + 1, (j + 1) & 1);
      process(j, j & 1);
      dma_wait();
      __syncthreads();
    }
  } else {
    for (int j0 = 0; j0 < ntiles; j0 += 2) {
      const int p = (j0 >> 1) & 1;  // pair slot of tiles j0, j0 + 1
      if (j0 + 2 < ntiles) issue_pair(j0 + 2, p ^ 1);
      process(j0, 2 * p);
      if (j0 + 1 < ntiles) process(j0 + 1, 2 * p + 1);
      dma_wait();
      __syncthreads();
    }
  }

  if (myq < S) {
    u16* out = static_cast<u16*>(a.dq) + (static_cast<int64_t>(u) * S + myq) * DH;
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int i = 0; i < 16; ++i) dq[d4][i] *= tau;
    if (a.rope.on) {
      // gradient of the unrotated query: the transposed rotation, applied to
      // the pairs (c, c + 64) = blocks d4 and d4 + 2 at the same register
#pragma unroll
      for (int d4 = 0; d4 < 2; ++d4)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float cs, sn;
          rope_cs(myq, a.rope.fw[32 * d4 + 8 * (i / 4) + 4 * hf + (i % 4)], cs, sn);
          float lo = dq[d4][i], hi = dq[d4 + 2][i];
          rope_bwd(lo, hi, cs, sn);
          dq[d4][i] = lo;
          dq[d4 + 2][i] = hi;
        }
    }
    if (a.dq32) {  // QK-norm: fp32, for the normalisation's backward
      float* o32 = a.dq32 + (static_cast<int64_t>(u) * S + myq) * DH;
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(o32 + 32 * d4 + 8 * g4 + 4 * hf) =
              f32x4{dq[d4][4 * g4], dq[d4][4 * g4 + 1], dq[d4][4 * g4 + 2], dq[d4][4 * g4 + 3]};
      return;
    }
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 v;
        v[0] = pack2(dq[d4][4 * g4 + 0], dq[d4][4 * g4 + 1]);
        v[1] = pack2(dq[d4][4 * g4 + 2], dq[d4][4 * g4 + 3]);
        *reinterpret_cast<u32x2*>(out + 32 * d4 + 8 * g4 + 4 * hf) = v;
      }
  }
}

// ---- dense MFMA stream: four independent accumulator chains per wave,
// operands in registers.  The operands are pseudo-random bf16 values in
// [-2, 2) with random mantissas (four sets per wave, rotated): the matrix
// core's power, and with it the clock it sustains, depends on how many bits
// toggle, and attention data are dense random values, not constants.  The
// result is stored only when iters < 0 (never), which keeps the products live
// without any memory traffic.  `rounds` x 16 MFMAs per wave.
__device__ __forceinline__ unsigned mix32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(float* sink, int rounds) {
  bf16x8 a[4], b[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    u32x4 ra, rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned h1 = mix32((blockIdx.x * 256u + threadIdx.x) * 16u + v * 4u + e), h2 = mix32(h1 ^ 0x9e3779b9u);
      ra[e] = (h1 & 0x807f807fu) | 0x3f003f00u;  // sign, mantissa random; exponent 2^-1 or 2^0
      rb[e] = (h2 & 0x807f807fu) | 0x3f003f00u;
    }
    a[v] = __builtin_bit_cast(bf16x8, ra);
    b[v] = __builtin_bit_cast(bf16x8, rb);
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  for (int it = 0; it < rounds; ++it) {  // 16 MFMAs per round
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = mfma(a[(r + i) & 3], b[(r + 2 * i) & 3], acc[i]);
  }
  if (rounds < 0) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][e];
    sink[threadIdx.x] = s;
  }
}

inline unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

namespace bf16 {

hipError_t proj(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, const Rope& rope,
                const NormArgs& nrm, hipStream_t st) {
  if (d != DH || D % GK != 0) return hipErrorInvalidValue;
  if (t.rot != 0 && !rope.on) return hipErrorInvalidValue;
  for (int i = 0; i < t.n; ++i)
    if (t.nkind[i] > 2 || (t.nkind[i] && !nrm.gamma[t.nkind[i] - 1]) ||
        (t.nkind[i] && nrm.store && (!nrm.xh[t.nkind[i] - 1] || !nrm.ri[t.nkind[i] - 1])))
      return hipErrorInvalidValue;
  const int nrb = static_cast<int>(cdiv(S, GB));
  hipLaunchKernelGGL(proj_kernel, dim3(nrb * t.n), dim3(256), 0, st, static_cast<const u16*>(X), S,
                     D, t, nrb, rope, nrm);
  return hipGetLastError();
}

// Weight gradients, dw_batch(P) chunks per launch: the parts' GEMM, then
// (P > 1) the fold of the parts into dW.
template <bool TR>
hipError_t dw_launch(const u16* B, int64_t S, int64_t D, const ChunkTable& t, int64_t ld,
                     float* scratch, hipStream_t st) {
  if (t.n <= 0) return hipSuccess;
  const int ncb = static_cast<int>(D / GB);
  const int P = dw_parts(S), nb = dw_batch(P) < t.n ? dw_batch(P) : t.n;
  if (P > 1 && !scratch) return hipErrorInvalidValue;
  for (int b = 0; b < t.n; b += nb) {
    ChunkTable u = t;
    u.n = t.n - b < nb ? t.n - b : nb;
    for (int i = 0; i < u.n; ++i) {
      u.a[i] = t.a[b + i];
      u.w[i] = t.w[b + i];
      u.dw[i] = t.dw[b + i];
    }
    hipLaunchKernelGGL(dw_kernel<TR>, dim3(ncb * u.n * P), dim3(512), 0, st, B, S, D, u, ncb, ld, P,
                       scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (P > 1) {
      hipLaunchKernelGGL(dw_fold_kernel<TR>, dim3(cdiv(GB * D / 4, 256), u.n), dim3(256), 0, st, u,
                         scratch, D, ld, P);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t dw(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, float* scratch,
              hipStream_t st) {
  if (d != DH || D % GB != 0) return hipErrorInvalidValue;
  return dw_launch<false>(static_cast<const u16*>(X), S, D, t, int64_t(DH), scratch, st);
}

hipError_t dwo(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
               float* scratch, hipStream_t st) {
  if (d != DH || D % GB != 0 || ld % 4 != 0) return hipErrorInvalidValue;
  return dw_launch<true>(static_cast<const u16*>(dY), S, D, t, ld, scratch, st);
}

hipError_t dx(float* dX, int64_t S, int64_t D, int d, const ChunkTable& t, hipStream_t st) {
  if (d != DH || D % GB != 0) return hipErrorInvalidValue;
  const int nrb = static_cast<int>(cdiv(S, GB)), ncb = static_cast<int>(D / GB);
  hipLaunchKernelGGL(dx_kernel, dim3(nrb * ncb), dim3(256), 0, st, dX, S, D, t, nrb, ncb);
  return hipGetLastError();
}

hipError_t oproj(float* Y, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                 hipStream_t st) {
  if (d != DH || D % GB != 0 || ld % 8 != 0) return hipErrorInvalidValue;
  const int nrb = static_cast<int>(cdiv(S, GB)), ncb = static_cast<int>(D / GB);
  hipLaunchKernelGGL(oproj_kernel, dim3(nrb * ncb), dim3(256), 0, st, Y, S, D, t, nrb, ncb, ld);
  return hipGetLastError();
}

hipError_t dout(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                hipStream_t st) {
  if (d != DH || D % GK != 0 || ld % 8 != 0) return hipErrorInvalidValue;
  const int nrb = static_cast<int>(cdiv(S, GB));
  hipLaunchKernelGGL(dout_kernel, dim3(nrb * t.n), dim3(256), 0, st, static_cast<const u16*>(dY), S,
                     D, t, nrb, ld);
  return hipGetLastError();
}

// Fewer than two rounds of 256-row workgroups: 128-row workgroups (the same
// bits, see the kernel).
static bool small_grid(const AttnArgs& a) { return cdiv(a.S, 256) * a.nq < 512; }

hipError_t attn_fwd(const AttnArgs& a, hipStream_t st) {
  if (a.d != DH) return hipErrorInvalidValue;
  if (small_grid(a))
    hipLaunchKernelGGL(attn_fwd_kernel<4>, dim3(cdiv(a.S, 128) * a.nq), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<8>, dim3(cdiv(a.S, 256) * a.nq), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t bwd_pre(const AttnArgs& a, hipStream_t st) {
  if (a.d != DH) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3(cdiv(a.S, 16), a.nq), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t mfma_ceiling(int waves_per_simd, int iters, double* tflops, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  hipEvent_t t0, t1;
  if ((e = hipEventCreate(&t0)) != hipSuccess) return e;
  if ((e = hipEventCreate(&t1)) != hipSuccess) {
    (void)hipEventDestroy(t0);
    return e;
  }
  const unsigned grid = static_cast<unsigned>(cus * waves_per_simd);  // 4 waves per block = 1 per SIMD
  const int rounds = iters / 4;  // iters x 4 MFMAs per wave, rounded down to whole rounds
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(256), 0, st, nullptr, rounds / 8);  // warm-up
  e = hipEventRecord(t0, st);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(256), 0, st, nullptr, rounds);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(t1, st);
  if (e == hipSuccess) e = hipEventSynchronize(t1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
  (void)hipEventDestroy(t0);
  (void)hipEventDestroy(t1);
  if (e == hipSuccess)
    *tflops = static_cast<double>(grid) * 4 * rounds * 16 * 32768.0 / (static_cast<double>(ms) * 1e-3) / 1e12;
  return e;
}

hipError_t attn_dq(const AttnArgs& a, hipStream_t st) {
  if (a.d != DH) return hipErrorInvalidValue;
  if (small_grid(a))
    hipLaunchKernelGGL(attn_dq_kernel<4>, dim3(cdiv(a.S, 128) * a.nq), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_dq_kernel<8>, dim3(cdiv(a.S, 256) * a.nq), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace bf16
}  // namespace upipe
