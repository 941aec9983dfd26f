// kernels_dkv.hip -- dK/dV pass of the attention backward for gfx950 (CDNA4).
//
// Backward of the per-stage attention (paper.rainbus.top summary of "Untied
// Ulysses", section 方法步骤详情 step (3); flash formulation): with the key in
// the lane, P = exp(S - LSE) and dS = P (dP - D) are recomputed per query
// tile, and dV += P^T dO, dK += dS^T Q accumulate in registers.
#include <hip/hip_runtime.h>

#include "upipe_internal.h"
#include "bf16_common.h"
#include "rope_device.h"

namespace upipe {
namespace {

// ---- dK, dV.  Workgroup: 128 key rows of one KV head, looping over the
// stage's query heads of that group (ascending) and over 64-row query tiles.
// Eight waves: each 32-key block has a pair of waves on one SIMD.  With the
// key in the lane (registers = query rows), the first wave of a pair computes
// S = Q K^T, P = exp(S - LSE) and dV += P^T dO; the second computes
// dP - D = dO V^T (its accumulators start from -D, the MFMA C input),
// dS = P (dP - D) with the first wave's fp32 P (exchanged through LDS lane
// for lane) and dK += dS^T Q.  P^T and dS^T are A operands
// straight from registers; dO and Q are read as column operands of the same
// row-major tiles.  Each tile takes two barrier phases: in the first, the
// second wave runs dK of the previous tile while the first wave evaluates the
// exponentials, so the SIMD's matrix unit stays busy; in the second, the
// first wave runs dV while the second forms dS.  The fp32 sums stay in
// registers, and across the stages of a group in the fp32 carry buffers.
// Below 512 key tiles (dkv_split) each key tile's query tiles are split into
// an upper and a lower half, one workgroup each with fp32 sums of its own
// (kept, and carried across stages, in the half-sum buffers), and
// dkv_combine_kernel adds upper + lower when the group is finished.
namespace kv {
constexpr int BN = 128, BM = 64;
constexpr int TILE = BM * 128;  // one swizzled 64-row tile
constexpr int NQ = 3;          // Q tiles it - 1 (dK), it (S), it + 1 (being filled)
constexpr int NG = 2;          // dO tiles it (dP, dV), it + 1 (being filled)
}  // namespace kv

__global__ __launch_bounds__(512, 1) void attn_dkv_kernel(AttnArgs a, int nkv) {
  using namespace kv;
  __shared__ __attribute__((aligned(256))) u16 qs[NQ * TILE];
  __shared__ __attribute__((aligned(256))) u16 gs[NG * TILE];
  __shared__ __attribute__((aligned(16))) float stat[2][2][BM];  // [tile & 1][LSE * log2(e), D][row]
  __shared__ __attribute__((aligned(16))) f32x4 pxch[4][8][64];  // P of each key block: [block][reg/4][lane]
  const int64_t S = a.S;
  const int lid = xcd_snake(blockIdx.x, gridDim.x);
  // logical id = (key tile, half, KV head): key tile 0 (most work) first;
  // half 1 exists only with a.kv_split == 2 (then nkv == 1)
  const int per_kt = nkv * a.kv_split;
  const int kt = lid / per_kt, half = (lid % per_kt) / nkv, gl = lid % nkv;
  const int g = a.kv_head0 + gl;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, hf = lane / 32;
  const int kb = wave & 3;      // key block of this wave (waves kb and kb + 4 share a SIMD)
  const bool pwave = wave < 4;  // S, P, dV; the others dP, dS, dK
  const int64_t wk0 = static_cast<int64_t>(kt) * BN + 32 * kb;
  const int64_t myk = wk0 + col;
  const float tau = 1.f / sqrtf(static_cast<float>(DH));
  const float c = kLog2e * tau;
  const int64_t ldo = a.ldo;

  // K rows (first wave of a pair) or V rows (second) of this key block, as B operands.
  bf16x8 kvf[8];
  {
    const u16* src = static_cast<const u16*>(pwave ? a.k : a.v) + static_cast<int64_t>(gl) * S * DH;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      kvf[t] = __builtin_bit_cast(bf16x8, myk < S ? ld16(src + myk * DH + 16 * t + 8 * hf) : u32x4{0, 0, 0, 0});
  }

  // dV (first wave) or dK (second) sums: C layout, lane = d column within
  // the 32-column block d4, registers = key rows
  f32x16 acc[4];
  // split: this half's fp32 sums of one KV head, [half][dK, dV][S][d]
  float* const part =
      a.kv_split == 2 ? a.kvp + (static_cast<int64_t>(half) * 2 + (pwave ? 1 : 0)) * S * DH : nullptr;
  {
    const float* carry = part ? part : (pwave ? a.dv_acc : a.dk_acc);
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) acc[d4] = zero16();
    if (!a.first_of_group) {
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t kr = wk0 + 8 * (i / 4) + 4 * hf + (i % 4);
          if (kr < S) acc[d4][i] = carry[(static_cast<int64_t>(gl) * S + kr) * DH + 32 * d4 + col];
        }
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) settle(kvf[t]);
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) settle(acc[d4]);

  const int h_lo = max(a.q_head0, g * a.r), h_hi = min(a.q_head0 + a.nq, (g + 1) * a.r);
  const int nqt = static_cast<int>((S + BM - 1) / BM);
  const int qt0 = a.causal ? static_cast<int>((static_cast<int64_t>(kt) * BN) / BM) : 0;
  // query tiles [qlo, qhi) of this workgroup: all from the diagonal on, or
  // with the split the upper (half 0) or lower (half 1) part of them
  int qlo = qt0, qhi = nqt;
  if (a.kv_split == 2) {
    const int mid = qt0 + (nqt - qt0 + 1) / 2;
    if (half == 0)
      qlo = mid;
    else
      qhi = mid;
  }
  const int per_head = qhi - qlo;
  const int niter = (h_hi - h_lo) * per_head;
  // Loop state, the same in every wave: tile t is query tile
  // qhi - 1 - t % per_head of head h_lo + t / per_head.  The query tiles are
  // walked from the end of the sequence down to the diagonal, so the key
  // tiles running together on one XCD (32 consecutive ones) all start on the
  // same query tile and stream the same Q / dO rows at once; walking up from
  // their diagonals kept 63 tiles (8 MB) in flight per XCD and fetched 11 GB
  // per launch instead of 7.  Cursors step through (head, query tile)
  // without divisions; slot counters track t % NQ and t % NG.
  struct Cur {
    int h, qt;
  };
  auto adv = [&](Cur& x) {
    if (--x.qt < qlo) {
      x.qt = qhi - 1;
      ++x.h;
    }
  };

  // Tile t + 1 is copied into LDS during tile t, by the second waves of the
  // pairs only (the first waves' S and exponentials are the round's critical
  // path): wave 4 + w copies rows 16w..16w+15 of the swizzled Q and dO tiles,
  // four rows per direct copy; waves 4 and 5 copy the tile's LSE and D (one
  // 256-byte row each).  A tile that runs past S goes through registers
  // instead, by every wave, with zero rows (and LSE = +inf, D = 0) beyond S.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const unsigned lane4 = 4u * lane;
  const int srow = tid >> 4, sc = tid & 15;
  // per-lane parts of the 4-row copies: row lane / 16 of the four, chunk
  // (lane % 16) ^ (4 (lane / 16) + q) of it (the swizzle of the tile)
  const unsigned swx = 16u * ((lane & 15) ^ (4 * (lane >> 4)));
  const unsigned rq = (lane >> 4) * 256u, rg = (lane >> 4) * static_cast<unsigned>(ldo * 2);
  auto issue = [&](const Cur& x, int slq, int slg) {
    const int u = x.h - a.q_head0;
    const int64_t q0 = static_cast<int64_t>(x.qt) * BM;
    const u16* qb = static_cast<const u16*>(a.q) + (static_cast<int64_t>(u) * S + q0) * DH;
    const u16* gb = static_cast<const u16*>(a.dO) + (x.h - a.do_h0) * a.do_hs + q0 * ldo;
    u16* qd = qs + slq * TILE;
    u16* gd = gs + slg * TILE;
    if (q0 + BM <= S) {
      if (wv >= 4) {  // the second waves copy: rows 16 w'..16 w'+15, w' = wv - 4, four rows per copy
        const int w2 = wv - 4;
        const unsigned qa = lds_byte_addr(qd) + static_cast<unsigned>(16 * w2 * 256);
        const unsigned ga = lds_byte_addr(gd) + static_cast<unsigned>(16 * w2 * 256);
        const u16* qr = qb + 16 * w2 * DH;
        const u16* gr = gb + 16 * w2 * ldo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned sw = swx ^ (16u * q);  // 16 ((lane % 16) ^ (4 (lane / 16) + q))
          dma_rows4(qr + 4 * q * DH, qa + 1024u * q, rq + sw);
          dma_rows4(gr + 4 * q * ldo, ga + 1024u * q, rg + sw);
        }
        if (wv == 4) dma_row(a.lse2 + static_cast<int64_t>(u) * S + q0, lds_byte_addr(&stat[slg][0][0]), lane4);
        if (wv == 5) dma_row(a.dd + static_cast<int64_t>(u) * S + q0, lds_byte_addr(&stat[slg][1][0]), lane4);
      }
    } else {
      const int64_t left = S - q0 - srow;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x4 vq = 32 * m < left ? ld16(qb + (srow + 32 * m) * DH + sc * 8) : u32x4{0, 0, 0, 0};
        const u32x4 vg = 32 * m < left ? ld16(gb + (srow + 32 * m) * ldo + sc * 8) : u32x4{0, 0, 0, 0};
        st16(qd + swz_off(srow + 32 * m, sc), vq);
        st16(gd + swz_off(srow + 32 * m, sc), vg);
      }
      if (tid < 2 * BM) {
        const int r = tid % BM;
        const bool in = q0 + r < S;
        const int64_t q = in ? q0 + r : S - 1;
        stat[slg][tid / BM][r] = tid < BM ? (in ? a.lse2[static_cast<int64_t>(u) * S + q] : INFINITY)
                                          : (in ? a.dd[static_cast<int64_t>(u) * S + q] : 0.f);
      }
    }
  };
  Cur cc{h_lo, qhi - 1};  // tile it
  Cur nc = cc;        // tile it + 1
  adv(nc);
  int sq = 0, sg = 0;  // it % NQ, it % NG
  auto next_tile = [&]() {  // end of a round: tile it + 1 becomes current
    adv(cc);
    adv(nc);
    sq = sq + 1 == NQ ? 0 : sq + 1;
    sg ^= 1;
  };

  // 32x64 C blocks of one tile: rows (query) x keys of this wave, two chains
  // over the 128 head columns; row operands from LDS two steps ahead.
  auto row_pass = [&](const SwzAddr& xa, f32x16 (&sv)[2]) {
    bf16x8 fa[3][2];
    auto row_ops = [&](int t, bf16x8 (&f)[2]) {
      f[0] = swz_row_frag(xa, 0, t);
      f[1] = swz_row_frag(xa, 1, t);
    };
    row_ops(0, fa[0]);
    row_ops(1, fa[1]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t + 2 < 8) row_ops(t + 2, fa[(t + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      sv[0] = mfma(fa[t % 3][0], kvf[t], sv[0]);
      sv[1] = mfma(fa[t % 3][1], kvf[t], sv[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc += op^T Y over the 64 rows of a tile: Y read as column operands,
  // step k4 outermost so the four accumulators alternate (each sums
  // k4 = 0..3 in order); operands requested two groups ahead.
  auto col_pass = [&](const SwzAddr& ya, const bf16x8 (&op)[4]) {
    bf16x8 fc[3];
    auto col_op = [&](int gi) { return swz_col_frag(ya, 16 * (gi / 4), 32 * (gi % 4)); };
    fc[0] = col_op(0);
    fc[1] = col_op(1);
#pragma unroll
    for (int gi = 0; gi < 16; ++gi) {
      if (gi + 2 < 16) fc[(gi + 2) % 3] = col_op(gi + 2);
      __builtin_amdgcn_sched_barrier(0);
      acc[gi % 4] = mfma(op[gi / 4], fc[gi % 3], acc[gi % 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (niter > 0) issue(cc, 0, 0);
  dma_wait();
  __syncthreads();

  // Both waves of a pair run niter + 1 rounds of two barriers each.
  if (pwave) {
    for (int it = 0; it <= niter; ++it) {
      bf16x8 op[4];  // P of tile it, packed
      __builtin_amdgcn_s_setprio(1);  // the first wave's S and exponentials are the round's critical path
      if (it + 1 < niter) issue(nc, sq + 1 == NQ ? 0 : sq + 1, sg ^ 1);
      if (it < niter) {
        // S = Q K^T; P = exp(S - LSE), masked above the diagonal; fp32 P to the partner
        f32x16 sv[2];
        f32x4 l4[8];  // requested before the S MFMAs, so they are ready for the exponentials
#pragma unroll
        for (int j = 0; j < 8; ++j) l4[j] = *reinterpret_cast<const f32x4*>(&stat[sg][0][8 * j + 4 * hf]);
        sv[0] = sv[1] = zero16();
        row_pass(swz_addr(qs + sq * TILE, lane), sv);
        const int64_t q0 = static_cast<int64_t>(cc.qt) * BM;
        // the diagonal test as a scalar, so the masking below is skipped by a
        // branch (as a per-lane condition it ran, exec-masked, on every tile)
        const bool need_mask = __builtin_amdgcn_readfirstlane(static_cast<int>(a.causal && q0 < wk0 + 31)) != 0;
        const int mlim = static_cast<int>(myk - q0);  // tile row r is masked when r < mlim
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int j = 4 * qb + g4, r0 = 8 * j + 4 * hf;  // tile rows r0..r0+3 = registers 4*g4..4*g4+3
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[qb][4 * g4 + e] = ex2(__builtin_fmaf(sv[qb][4 * g4 + e], c, -l4[j][e]));
            if (need_mask) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (r0 + e < mlim) sv[qb][4 * g4 + e] = 0.f;
            }
            pxch[kb][j][lane] = f32x4{sv[qb][4 * g4], sv[qb][4 * g4 + 1], sv[qb][4 * g4 + 2], sv[qb][4 * g4 + 3]};
          }
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) op[k4] = pack8(sv[k4 / 2], k4 % 2);
      }
      __syncthreads();
      __builtin_amdgcn_s_setprio(0);
      if (it < niter) col_pass(swz_addr(gs + sg * TILE, lane), op);  // dV += P^T dO
      dma_wait();
      __syncthreads();
      next_tile();
    }
  } else {
    bf16x8 op[4];  // dS of the previous tile, packed
    f32x16 sv[2];  // dP of the current tile
    for (int it = 0; it <= niter; ++it) {
      if (it + 1 < niter) issue(nc, sq + 1 == NQ ? 0 : sq + 1, sg ^ 1);
      if (it < niter) {
        // dP - D = dO V^T with the accumulators starting from -D (rows in C layout)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[sg][1][8 * j + 4 * hf]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[j / 4][4 * (j % 4) + e] = -d4[e];
        }
        row_pass(swz_addr(gs + sg * TILE, lane), sv);
      }
      if (it >= 1) col_pass(swz_addr(qs + (sq == 0 ? NQ - 1 : sq - 1) * TILE, lane), op);  // dK += dS^T Q, tile it - 1
      __syncthreads();
      if (it < niter) {
        // dS = P (dP - D) with the partner's fp32 P
        f32x4 p4[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p4[j] = pxch[kb][j][lane];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int j = 4 * qb + g4;
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[qb][4 * g4 + e] = p4[j][e] * sv[qb][4 * g4 + e];
          }
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) op[k4] = pack8(sv[k4 / 2], k4 % 2);
      }
      dma_wait();
      __syncthreads();
      next_tile();
    }
  }

  if (part) {  // split: this half's sum as it stands; dkv_combine_kernel finishes the group
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t kr = wk0 + 8 * (i / 4) + 4 * hf + (i % 4);
        if (kr < S) part[kr * DH + 32 * d4 + col] = acc[d4][i];
      }
  } else {
    float* carry = pwave ? a.dv_acc : a.dk_acc;
    u16* out = static_cast<u16*>(pwave ? a.dv : a.dk);
    const float scale = pwave ? 1.f : tau;
    if (a.last_of_group) {
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[d4][i] *= scale;
      if (!pwave && a.rope.on) {
        // gradient of the unrotated key (the group's finished sum): the
        // transposed rotation of the pairs (c, c + 64) = blocks d4, d4 + 2
#pragma unroll
        for (int d4 = 0; d4 < 2; ++d4) {
          const double fw = a.rope.fw[32 * d4 + col];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float cs, sn;
            rope_cs(wk0 + 8 * (i / 4) + 4 * hf + (i % 4), fw, cs, sn);
            float lo = acc[d4][i], hi = acc[d4 + 2][i];
            rope_bwd(lo, hi, cs, sn);
            acc[d4][i] = lo;
            acc[d4 + 2][i] = hi;
          }
        }
      }
    }
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t kr = wk0 + 8 * (i / 4) + 4 * hf + (i % 4);
        if (kr >= S) continue;
        const int64_t off = (static_cast<int64_t>(gl) * S + kr) * DH + 32 * d4 + col;
        if (a.last_of_group && !pwave && a.dk32)
          a.dk32[off] = acc[d4][i];  // QK-norm: fp32, for the normalisation's backward
        else if (a.last_of_group)
          out[off] = __builtin_bit_cast(u16, static_cast<__bf16>(acc[d4][i]));
        else
          carry[off] = acc[d4][i];
      }
  }
}

// Split dK/dV of one KV head, its group finished: dK = tau (upper + lower),
// then the transposed rotation of the pairs (c, c + 64) with the rotary
// embedding, rounded to bf16 (or kept in fp32 for the QK-norm backward);
// dV = upper + lower, rounded.  One thread per (key row, pair).
__global__ __launch_bounds__(256) void dkv_combine_kernel(AttnArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = idx / 64;
  const int c = static_cast<int>(idx % 64);
  if (row >= a.S) return;
  const int64_t Sd = a.S * DH, o = row * DH + c;
  const float* P = a.kvp;  // [half][dK, dV][S][d]
  const float tau = 1.f / sqrtf(static_cast<float>(DH));
  float klo = (P[o] + P[2 * Sd + o]) * tau, khi = (P[o + 64] + P[2 * Sd + o + 64]) * tau;
  if (a.rope.on) {
    float cs, sn;
    rope_cs(row, a.rope.fw[c], cs, sn);
    rope_bwd(klo, khi, cs, sn);
  }
  if (a.dk32) {
    a.dk32[o] = klo;
    a.dk32[o + 64] = khi;
  } else {
    static_cast<u16*>(a.dk)[o] = __builtin_bit_cast(u16, static_cast<__bf16>(klo));
    static_cast<u16*>(a.dk)[o + 64] = __builtin_bit_cast(u16, static_cast<__bf16>(khi));
  }
  const float vlo = P[Sd + o] + P[3 * Sd + o], vhi = P[Sd + o + 64] + P[3 * Sd + o + 64];
  static_cast<u16*>(a.dv)[o] = __builtin_bit_cast(u16, static_cast<__bf16>(vlo));
  static_cast<u16*>(a.dv)[o + 64] = __builtin_bit_cast(u16, static_cast<__bf16>(vhi));
}

}  // namespace

namespace bf16 {

hipError_t attn_dkv(const AttnArgs& a, hipStream_t st) {
  if (a.d != DH) return hipErrorInvalidValue;
  const int nkv = a.nq >= a.r ? a.nq / a.r : 1;
  const unsigned nkt = static_cast<unsigned>((a.S + kv::BN - 1) / kv::BN);
  if (a.kv_split != 2) {
    hipLaunchKernelGGL(attn_dkv_kernel, dim3(nkt * nkv), dim3(512), 0, st, a, nkv);
    return hipGetLastError();
  }
  // split: one launch per KV group of the stage (the two halves' sums of one
  // KV head at a time), then the combine when the group is finished
  if (!a.kvp || a.kv_split != dkv_split(a.S)) return hipErrorInvalidValue;
  const int64_t Sd = a.S * DH;
  for (int g = 0; g < nkv; ++g) {
    AttnArgs b = a;
    if (nkv > 1) {  // the stage holds whole groups: group g's r query heads
      b.nq = a.r;
      b.q_head0 = a.q_head0 + g * a.r;
      b.kv_head0 = a.kv_head0 + g;
      b.q = static_cast<const u16*>(a.q) + static_cast<int64_t>(g) * a.r * Sd;
      b.k = static_cast<const u16*>(a.k) + g * Sd;
      b.v = static_cast<const u16*>(a.v) + g * Sd;
      b.dd = a.dd + static_cast<int64_t>(g) * a.r * a.S;
      b.lse2 = a.lse2 + static_cast<int64_t>(g) * a.r * a.S;
      b.dk = static_cast<u16*>(a.dk) + g * Sd;
      b.dv = static_cast<u16*>(a.dv) + g * Sd;
      b.dk32 = a.dk32 ? a.dk32 + g * Sd : nullptr;
    }
    hipLaunchKernelGGL(attn_dkv_kernel, dim3(nkt * 2), dim3(512), 0, st, b, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (b.last_of_group && a.S > 0) {
      hipLaunchKernelGGL(dkv_combine_kernel, dim3(static_cast<unsigned>((a.S * 64 + 255) / 256)), dim3(256),
                         0, st, b);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace bf16
}  // namespace upipe
