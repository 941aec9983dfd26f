// rope_device.h -- rotary position embedding on the device (rotate-half form,
// as in the Llama and Qwen model families that run this layer): the pair
// (c, c + d/2) of a query or key row at token position i turns by the angle
// i * w_c, w_c = theta^(-2c/d).  Included by each kernel source.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace upipe {
namespace {

// Cosine and sine of the angle pos * w for fw = w / (2 pi) (turns per
// position, fp64).  The product and its fractional part are taken in fp64
// (exact to ~1e-10 turns for positions below 2^31), so the hardware sine and
// cosine (v_sin_f32 / v_cos_f32, whose argument is in turns) only ever see a
// value in [0, 1).
__device__ __forceinline__ void rope_cs(int64_t pos, double fw, float& cs, float& sn) {
  double t = static_cast<double>(pos) * fw;
  t -= __builtin_floor(t);
  const float tf = static_cast<float>(t);
  cs = __builtin_amdgcn_cosf(tf);
  sn = __builtin_amdgcn_sinf(tf);
}

// Forward rotation of the pair (lo, hi) = (x[c], x[c + d/2]).
__device__ __forceinline__ void rope_fwd(float& lo, float& hi, float cs, float sn) {
  const float a = lo, b = hi;
  lo = a * cs - b * sn;
  hi = b * cs + a * sn;
}

// Transposed rotation, for the gradients of rotated rows.
__device__ __forceinline__ void rope_bwd(float& lo, float& hi, float cs, float sn) {
  const float a = lo, b = hi;
  lo = a * cs + b * sn;
  hi = b * cs - a * sn;
}

}  // namespace
}  // namespace upipe
