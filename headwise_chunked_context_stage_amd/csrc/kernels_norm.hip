// kernels_norm.hip -- QK-norm of the projected queries and keys for gfx950.
//
// Not on the pages (the Qwen3 attention whose shape the pages train uses it):
// each projected query or key row x of a head (d values) becomes
//   y_c = gamma_c * xhat_c,  xhat = x * r,  r = 1 / sqrt(sum_c x_c^2 / d + eps),
// before the rotary embedding.  Its backward, for the gradient gy of y:
//   gx_c = r * (gamma_c * gy_c - xhat_c * (sum_e gamma_e gy_e xhat_e) / d),
//   dgamma_c = sum over heads and rows of gy_c * xhat_c.
// The bf16 forward runs in the projection's epilogue (before its rounding);
// fp32 plans normalise in place here.  The backward always runs here, on the
// fp32 gradients the attention backward leaves, and writes the gradient the
// weight- and input-gradient GEMMs read.
//
// One wave per row: lane l holds columns l and l + 64 (d = 128) or l (d = 64).
// Row sums use an xor butterfly, which gives every lane the same value (each
// step adds two values in either order, and fp32 addition is commutative).
// dgamma is reduced deterministically: per 256-token block in a fixed order
// (a wave's 64 rows in order, then the four waves in order), then the blocks
// in order by gamma_sum, heads ascending -- no atomics, the same bits for
// every U.
#include <hip/hip_runtime.h>

#include "upipe_internal.h"

namespace upipe {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ float gamma_at(const void* g, int bf, int c) {
  if (bf) {
    const unsigned short h = static_cast<const unsigned short*>(g)[c];
    return __uint_as_float(static_cast<unsigned>(h) << 16);
  }
  return static_cast<const float*>(g)[c];
}

// fp32 plans: rows of n * S, in place.
__global__ __launch_bounds__(256) void norm_fwd_f32_kernel(float* __restrict__ x, int64_t rows,
                                                           int d, const float* __restrict__ gamma,
                                                           float eps, float* __restrict__ xhat,
                                                           float* __restrict__ rinv) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;
  const int nc = d / 64;  // columns per lane
  float* xr = x + row * d;
  float v[2] = {0.f, 0.f};
  float ss = 0.f;
  for (int k = 0; k < nc; ++k) {
    v[k] = xr[lane + 64 * k];
    ss += v[k] * v[k];
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss * (1.f / static_cast<float>(d)) + eps);
  for (int k = 0; k < nc; ++k) {
    const int c = lane + 64 * k;
    const float xh = v[k] * r;
    if (xhat) xhat[row * d + c] = xh;
    xr[c] = gamma[c] * xh;
  }
  if (rinv && lane == 0) rinv[row] = r;
}

// Backward: grid (blocks of kNormBlock tokens, n row blocks of S), 4 waves.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void norm_bwd_kernel(const float* g, const float* __restrict__ xhat,
                                                       const float* __restrict__ rinv,
                                                       const void* __restrict__ gamma, int gamma_bf16,
                                                       void* out, float* __restrict__ part,
                                                       int64_t S, int d) {
  __shared__ float wpart[4][128];
  const int b = blockIdx.x, u = blockIdx.y, nb = gridDim.x;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int nc = d / 64;
  float gam[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
  for (int k = 0; k < nc; ++k) gam[k] = gamma_at(gamma, gamma_bf16, lane + 64 * k);
  const float inv_d = 1.f / static_cast<float>(d);
  const int64_t r0 = static_cast<int64_t>(b) * kNormBlock + 64 * wave;
  for (int i = 0; i < 64; ++i) {
    const int64_t row = r0 + i;
    if (row >= S) break;
    const int64_t off = (static_cast<int64_t>(u) * S + row) * d;
    const float r = rinv[static_cast<int64_t>(u) * S + row];
    float gv[2] = {0.f, 0.f}, xv[2] = {0.f, 0.f};
    float t = 0.f;
    for (int k = 0; k < nc; ++k) {
      gv[k] = g[off + lane + 64 * k];
      xv[k] = xhat[off + lane + 64 * k];
      t += gam[k] * gv[k] * xv[k];
      acc[k] += gv[k] * xv[k];
    }
    t = wave_sum(t) * inv_d;
    for (int k = 0; k < nc; ++k) {
      const float o = r * (gam[k] * gv[k] - xv[k] * t);
      if (OUT_BF16)
        static_cast<__bf16*>(out)[off + lane + 64 * k] = static_cast<__bf16>(o);
      else
        static_cast<float*>(out)[off + lane + 64 * k] = o;
    }
  }
  for (int k = 0; k < nc; ++k) wpart[wave][lane + 64 * k] = acc[k];
  __syncthreads();
  const int c = threadIdx.x;
  if (c < d) {
    const float s = ((wpart[0][c] + wpart[1][c]) + wpart[2][c]) + wpart[3][c];
    part[(static_cast<int64_t>(u) * nb + b) * d + c] = s;
  }
}

__global__ __launch_bounds__(128) void gamma_sum_kernel(float* dg, const float* __restrict__ part,
                                                        int64_t nrows, int d, int first) {
  const int c = threadIdx.x;
  if (c >= d) return;
  float acc = first ? 0.f : dg[c];
  for (int64_t i = 0; i < nrows; ++i) acc += part[i * d + c];
  dg[c] = acc;
}

}  // namespace

namespace norm {

hipError_t fwd_f32(float* x, int n, int64_t S, int d, const float* gamma, float eps, float* xhat,
                   float* rinv, hipStream_t st) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  const int64_t rows = static_cast<int64_t>(n) * S;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(norm_fwd_f32_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
                     st, x, rows, d, gamma, eps, xhat, rinv);
  return hipGetLastError();
}

hipError_t bwd(const float* g, const float* xhat, const float* rinv, const void* gamma,
               int gamma_bf16, void* out, int out_bf16, float* part, int n, int64_t S, int d,
               hipStream_t st) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  const int64_t nb = (S + kNormBlock - 1) / kNormBlock;
  if (nb == 0 || n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>(n));
  if (out_bf16)
    hipLaunchKernelGGL(norm_bwd_kernel<true>, grid, dim3(256), 0, st, g, xhat, rinv, gamma,
                       gamma_bf16, out, part, S, d);
  else
    hipLaunchKernelGGL(norm_bwd_kernel<false>, grid, dim3(256), 0, st, g, xhat, rinv, gamma,
                       gamma_bf16, out, part, S, d);
  return hipGetLastError();
}

hipError_t gamma_sum(float* dg, const float* part, int n, int64_t S, int d, int first,
                     hipStream_t st) {
  const int64_t nb = (S + kNormBlock - 1) / kNormBlock;
  hipLaunchKernelGGL(gamma_sum_kernel, dim3(1), dim3(128), 0, st, dg, part,
                     static_cast<int64_t>(n) * nb, d, first);
  return hipGetLastError();
}

}  // namespace norm
}  // namespace upipe
