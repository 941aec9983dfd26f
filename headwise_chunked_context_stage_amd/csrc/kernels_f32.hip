// kernels_f32.hip -- fp32 kernels of the stage loop (gfx950).
//
// The fp32 variant serves small layers stored in fp32 (the exact-precision
// configuration); its kernels are plain FMA loops, one output element or one
// row per thread, with fixed summation orders so that results are
// deterministic and identical for every stage size U.  The bf16 variant in
// kernels_bf16.hip is the performance path.
//
// Attention follows the flash formulation: scores are scaled by
// log2(e)/sqrt(d) and exponentiated with the hardware exp2; LSE is returned in
// natural log.  Backward: D_i = <dO_i, O_i>, P_ij = exp(s_ij - LSE_i),
// dS_ij = P_ij (dP_ij - D_i), dQ = tau dS K, dK = tau dS^T Q, dV = P^T dO.
#include <hip/hip_runtime.h>

#include "upipe_internal.h"
#include "rope_device.h"

namespace upipe {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ fill
__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// ------------------------------------------------------------------ GEMMs
// out[i][c] = sum_k X[i][k] * W[c][k] for one chunk (blockIdx.z).
// 64x64 output tile, 16-wide k slices staged in LDS, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void proj_kernel(const float* __restrict__ X, int64_t S, int64_t D,
                                                   int d, ChunkTable t) {
  __shared__ float xs[16][64 + 1];
  __shared__ float ws[16][64 + 1];
  const float* W = static_cast<const float*>(t.w[blockIdx.z]);
  float* out = static_cast<float*>(t.a[blockIdx.z]);
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < D; k0 += 16) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      int row = e / 16, kk = e % 16;
      int64_t gi = i0 + row;
      xs[kk][row] = gi < S ? X[gi * D + k0 + kk] : 0.f;
      ws[kk][row] = W[static_cast<int64_t>(c0 + row) * D + k0 + kk];
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk)
      for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b) acc[a][b] += xs[kk][ty * 4 + a] * ws[kk][tx * 4 + b];
    __syncthreads();
  }
  for (int a = 0; a < 4; ++a) {
    int64_t gi = i0 + ty * 4 + a;
    if (gi >= S) continue;
    for (int b = 0; b < 4; ++b) out[gi * d + c0 + tx * 4 + b] = acc[a][b];
  }
}

// dW[c][k] = sum_i A[i][c] * X[i][k]; one thread per output element, i ascending.
__global__ __launch_bounds__(256) void dw_kernel(const float* __restrict__ X, int64_t S, int64_t D,
                                                 int d, ChunkTable t) {
  const float* A = static_cast<const float*>(t.a[blockIdx.z]);
  float* dW = t.dw[blockIdx.z];
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (k >= D) return;
  float acc = 0.f;
  for (int64_t i = 0; i < S; ++i) acc += A[i * d + c] * X[i * D + k];
  dW[static_cast<int64_t>(c) * D + k] = acc;
}

// dX[i][k] += sum over chunks (table order) of sum_c A[i][c] * W[c][k].
__global__ __launch_bounds__(256) void dx_kernel(float* __restrict__ dX, int64_t S, int64_t D, int d,
                                                 ChunkTable t) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (k >= D || i >= S) return;
  float acc = t.czero ? 0.f : dX[i * D + k];
  for (int ch = 0; ch < t.n; ++ch) {
    const float* A = static_cast<const float*>(t.a[ch]);
    const float* W = static_cast<const float*>(t.w[ch]);
    for (int c = 0; c < d; ++c) acc += A[i * d + c] * W[static_cast<int64_t>(c) * D + k];
  }
  dX[i * D + k] = acc;
}

// ------------------------------------------------------------------ attention
// One thread per (head, query row).  Pass 1: running max and sum; pass 2:
// O = sum_j exp2(x_ij - lse2) V_j.
template <int DH>
__global__ __launch_bounds__(128) void attn_fwd_kernel(AttnArgs a) {
  const int u = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x;
  if (i >= a.S) return;
  const int h = a.q_head0 + u;
  const int g = h / a.r - a.kv_head0;
  const float* Q = static_cast<const float*>(a.q) + (static_cast<int64_t>(u) * a.S + i) * DH;
  const float* K = static_cast<const float*>(a.k) + static_cast<int64_t>(g) * a.S * DH;
  const float* V = static_cast<const float*>(a.v) + static_cast<int64_t>(g) * a.S * DH;
  const float c = kLog2e / sqrtf(static_cast<float>(DH));
  float q[DH];
  for (int e = 0; e < DH; ++e) q[e] = Q[e];
  const int64_t last = a.causal ? i : a.S - 1;
  float m = -INFINITY, l = 0.f;
  for (int64_t j = 0; j <= last; ++j) {
    float s = 0.f;
    for (int e = 0; e < DH; ++e) s += q[e] * K[j * DH + e];
    float x = s * c;
    float mn = fmaxf(m, x);
    l = l * exp2f(m - mn) + exp2f(x - mn);
    m = mn;
  }
  const float lse2 = m + log2f(l);
  float o[DH];
  for (int e = 0; e < DH; ++e) o[e] = 0.f;
  for (int64_t j = 0; j <= last; ++j) {
    float s = 0.f;
    for (int e = 0; e < DH; ++e) s += q[e] * K[j * DH + e];
    float p = exp2f(s * c - lse2);
    for (int e = 0; e < DH; ++e) o[e] += p * V[j * DH + e];
  }
  float* O = static_cast<float*>(a.o) + i * static_cast<int64_t>(a.H) * DH + static_cast<int64_t>(h) * DH;
  for (int e = 0; e < DH; ++e) O[e] = o[e];
  a.lse[static_cast<int64_t>(h) * a.S + i] = lse2 * kLn2;
}

// D[u][i] = <dO_i, O_i> for the stage's heads.
template <int DH>
__global__ __launch_bounds__(256) void bwd_pre_kernel(AttnArgs a) {
  const int u = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.S) return;
  const int h = a.q_head0 + u;
  const int64_t off = i * static_cast<int64_t>(a.H) * DH + static_cast<int64_t>(h) * DH;
  const float* dO = static_cast<const float*>(a.dO) + (h - a.do_h0) * a.do_hs + i * a.ldo;
  const float* O = static_cast<const float*>(a.o_in) + off;
  float acc = 0.f;
  for (int e = 0; e < DH; ++e) acc += dO[e] * O[e];
  a.dd[static_cast<int64_t>(u) * a.S + i] = acc;
}

// dQ_i = tau * sum_j dS_ij K_j; one thread per (head, query row).
template <int DH>
__global__ __launch_bounds__(128) void attn_dq_kernel(AttnArgs a) {
  const int u = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x;
  if (i >= a.S) return;
  const int h = a.q_head0 + u;
  const int g = h / a.r - a.kv_head0;
  const float* Q = static_cast<const float*>(a.q) + (static_cast<int64_t>(u) * a.S + i) * DH;
  const float* K = static_cast<const float*>(a.k) + static_cast<int64_t>(g) * a.S * DH;
  const float* V = static_cast<const float*>(a.v) + static_cast<int64_t>(g) * a.S * DH;
  const float* dO = static_cast<const float*>(a.dO) + (h - a.do_h0) * a.do_hs + i * a.ldo;
  const float tau = 1.f / sqrtf(static_cast<float>(DH));
  const float c = kLog2e * tau;
  const float lse2 = a.lse_in[static_cast<int64_t>(h) * a.S + i] * kLog2e;
  const float Di = a.dd[static_cast<int64_t>(u) * a.S + i];
  float q[DH], go[DH], dq[DH];
  for (int e = 0; e < DH; ++e) {
    q[e] = Q[e];
    go[e] = dO[e];
    dq[e] = 0.f;
  }
  const int64_t last = a.causal ? i : a.S - 1;
  for (int64_t j = 0; j <= last; ++j) {
    float s = 0.f, dp = 0.f;
    for (int e = 0; e < DH; ++e) {
      s += q[e] * K[j * DH + e];
      dp += go[e] * V[j * DH + e];
    }
    const float p = exp2f(s * c - lse2);
    const float ds = p * (dp - Di);
    for (int e = 0; e < DH; ++e) dq[e] += ds * K[j * DH + e];
  }
  float* out = static_cast<float*>(a.dq) + (static_cast<int64_t>(u) * a.S + i) * DH;
  for (int e = 0; e < DH; ++e) out[e] = dq[e] * tau;
}

// dK_j, dV_j for one KV head: one thread per key row, the stage's query heads
// of this group in ascending order, query rows ascending.  The fp32 sums are
// carried through dk/dv (unscaled) between the stages of a group.
template <int DH>
__global__ __launch_bounds__(128) void attn_dkv_kernel(AttnArgs a) {
  const int gl = blockIdx.y;  // KV head within the stage
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x;
  if (j >= a.S) return;
  const int g = a.kv_head0 + gl;
  const float* K = static_cast<const float*>(a.k) + (static_cast<int64_t>(gl) * a.S + j) * DH;
  const float* V = static_cast<const float*>(a.v) + (static_cast<int64_t>(gl) * a.S + j) * DH;
  float* dK = static_cast<float*>(a.dk) + (static_cast<int64_t>(gl) * a.S + j) * DH;
  float* dV = static_cast<float*>(a.dv) + (static_cast<int64_t>(gl) * a.S + j) * DH;
  const float tau = 1.f / sqrtf(static_cast<float>(DH));
  const float c = kLog2e * tau;
  float k[DH], v[DH], dk[DH], dv[DH];
  for (int e = 0; e < DH; ++e) {
    k[e] = K[e];
    v[e] = V[e];
    dk[e] = a.first_of_group ? 0.f : dK[e];
    dv[e] = a.first_of_group ? 0.f : dV[e];
  }
  // query heads of group g inside this stage
  const int h_lo = max(a.q_head0, g * a.r);
  const int h_hi = min(a.q_head0 + a.nq, (g + 1) * a.r);
  for (int h = h_lo; h < h_hi; ++h) {
    const int u = h - a.q_head0;
    const float* Q = static_cast<const float*>(a.q) + static_cast<int64_t>(u) * a.S * DH;
    const float* dO = static_cast<const float*>(a.dO) + (h - a.do_h0) * a.do_hs;
    const int64_t ldo = a.ldo;
    for (int64_t i = a.causal ? j : 0; i < a.S; ++i) {
      float s = 0.f, dp = 0.f;
      for (int e = 0; e < DH; ++e) {
        s += Q[i * DH + e] * k[e];
        dp += dO[i * ldo + e] * v[e];
      }
      const float p = exp2f(s * c - a.lse_in[static_cast<int64_t>(h) * a.S + i] * kLog2e);
      const float ds = p * (dp - a.dd[static_cast<int64_t>(u) * a.S + i]);
      for (int e = 0; e < DH; ++e) {
        dk[e] += ds * Q[i * DH + e];
        dv[e] += p * dO[i * ldo + e];
      }
    }
  }
  for (int e = 0; e < DH; ++e) {
    dK[e] = a.last_of_group ? dk[e] * tau : dk[e];
    dV[e] = dv[e];
  }
}

// Rotary embedding in place: one thread per (buffer, row, pair c < d/2).
// sign +1 rotates, -1 applies the transposed rotation (gradients).  fp32
// storage holds the kernels' results exactly, so rotating after the producer
// gives the same values as rotating in its epilogue.
__global__ __launch_bounds__(256) void rope_kernel(float* __restrict__ buf, int64_t S, int d,
                                                   Rope r, int sign) {
  const int half = d / 2;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= S * half) return;
  const int64_t i = e / half;
  const int c = static_cast<int>(e % half);
  float* row = buf + static_cast<int64_t>(blockIdx.y) * S * d + i * d;
  float cs, sn;
  rope_cs(i, r.fw[c], cs, sn);
  if (sign > 0)
    rope_fwd(row[c], row[c + half], cs, sn);
  else
    rope_bwd(row[c], row[c + half], cs, sn);
}

// Output projection, one thread per output element with fixed loop orders.
// Y[i][k] += sum over chunks (heads ascending), then c ascending, of
// O[i][c] Wo[k][c]; Y is the running sum across stages, so every U adds the
// same terms in the same order.
__global__ __launch_bounds__(256) void oproj_kernel(float* __restrict__ Y, int64_t S, int64_t D,
                                                    int d, ChunkTable t, int64_t ld) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (k >= D) return;
  float acc = t.czero ? 0.f : Y[i * D + k];
  for (int ch = 0; ch < t.n; ++ch) {
    const float* o = static_cast<const float*>(t.a[ch]) + i * ld;
    const float* w = static_cast<const float*>(t.w[ch]) + k * ld;
    for (int c = 0; c < d; ++c) acc += o[c] * w[c];
  }
  Y[i * D + k] = acc;
}

// out[i][c] = sum_k dY[i][k] Wo[k][c] (k ascending), for chunk blockIdx.z.
__global__ __launch_bounds__(256) void dout_kernel(const float* __restrict__ dY, int64_t S,
                                                   int64_t D, int d, ChunkTable t, int64_t ld) {
  const int c = threadIdx.x % 64 + 64 * blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (i >= S || c >= d) return;
  const float* w = static_cast<const float*>(t.w[blockIdx.z]) + c;
  float acc = 0.f;
  for (int64_t k = 0; k < D; ++k) acc += dY[i * D + k] * w[k * ld];
  static_cast<float*>(t.a[blockIdx.z])[i * d + c] = acc;
}

// dWo[k][c] = sum_i dY[i][k] O[i][c] (i ascending), for chunk blockIdx.z.
__global__ __launch_bounds__(256) void dwo_kernel(const float* __restrict__ dY, int64_t S,
                                                  int64_t D, int d, ChunkTable t, int64_t ld) {
  const int c = threadIdx.x % 64 + 64 * blockIdx.y;
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (k >= D || c >= d) return;
  const float* o = static_cast<const float*>(t.a[blockIdx.z]) + c;
  float acc = 0.f;
  for (int64_t i = 0; i < S; ++i) acc += dY[i * D + k] * o[i * ld];
  t.dw[blockIdx.z][k * ld + c] = acc;
}

inline unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

hipError_t fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<uint4*>(p), n16, static_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

namespace f32 {

hipError_t proj(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, hipStream_t st) {
  hipLaunchKernelGGL(proj_kernel, dim3(cdiv(S, 64), d / 64, t.n), dim3(256), 0, st,
                     static_cast<const float*>(X), S, D, d, t);
  return hipGetLastError();
}

hipError_t dw(const void* X, int64_t S, int64_t D, int d, const ChunkTable& t, float* /*scratch*/,
              hipStream_t st) {
  hipLaunchKernelGGL(dw_kernel, dim3(cdiv(D, 256), d, t.n), dim3(256), 0, st,
                     static_cast<const float*>(X), S, D, d, t);
  return hipGetLastError();
}

hipError_t dx(float* dX, int64_t S, int64_t D, int d, const ChunkTable& t, hipStream_t st) {
  hipLaunchKernelGGL(dx_kernel, dim3(cdiv(D, 256), static_cast<unsigned>(S)), dim3(256), 0, st, dX,
                     S, D, d, t);
  return hipGetLastError();
}

hipError_t rope(float* buf, int n, int64_t S, int d, const Rope& r, int sign, hipStream_t st) {
  if (n <= 0 || S <= 0) return hipSuccess;
  if (!r.on || d % 2 != 0 || d / 2 > kMaxRopePairs) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_kernel, dim3(cdiv(S * (d / 2), 256), n), dim3(256), 0, st, buf, S, d, r,
                     sign);
  return hipGetLastError();
}

hipError_t oproj(float* Y, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                 hipStream_t st) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(oproj_kernel, dim3(cdiv(D, 256), static_cast<unsigned>(S)), dim3(256), 0, st,
                     Y, S, D, d, t, ld);
  return hipGetLastError();
}

hipError_t dout(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
                hipStream_t st) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(dout_kernel, dim3(cdiv(S, 4), cdiv(d, 64), t.n), dim3(256), 0, st,
                     static_cast<const float*>(dY), S, D, d, t, ld);
  return hipGetLastError();
}

hipError_t dwo(const void* dY, int64_t S, int64_t D, int d, const ChunkTable& t, int64_t ld,
               float* /*scratch*/, hipStream_t st) {
  hipLaunchKernelGGL(dwo_kernel, dim3(cdiv(D, 4), cdiv(d, 64), t.n), dim3(256), 0, st,
                     static_cast<const float*>(dY), S, D, d, t, ld);
  return hipGetLastError();
}

#define UPIPE_F32_DISPATCH(kern, grid, block)                                          \
  do {                                                                                 \
    if (a.d == 64)                                                                     \
      hipLaunchKernelGGL(kern<64>, grid, block, 0, st, a);                             \
    else                                                                               \
      hipLaunchKernelGGL(kern<128>, grid, block, 0, st, a);                            \
    return hipGetLastError();                                                          \
  } while (0)

hipError_t attn_fwd(const AttnArgs& a, hipStream_t st) {
  UPIPE_F32_DISPATCH(attn_fwd_kernel, dim3(cdiv(a.S, 128), a.nq), dim3(128));
}
hipError_t bwd_pre(const AttnArgs& a, hipStream_t st) {
  UPIPE_F32_DISPATCH(bwd_pre_kernel, dim3(cdiv(a.S, 256), a.nq), dim3(256));
}
hipError_t attn_dq(const AttnArgs& a, hipStream_t st) {
  UPIPE_F32_DISPATCH(attn_dq_kernel, dim3(cdiv(a.S, 128), a.nq), dim3(128));
}
hipError_t attn_dkv(const AttnArgs& a, hipStream_t st) {
  const int nkv = a.nq >= a.r ? a.nq / a.r : 1;
  UPIPE_F32_DISPATCH(attn_dkv_kernel, dim3(cdiv(a.S, 128), nkv), dim3(128));
}

}  // namespace f32
}  // namespace upipe
