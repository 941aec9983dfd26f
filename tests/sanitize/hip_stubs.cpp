// Host-only stand-ins for the HIP runtime calls and kernel launchers that the
// C ABI's host code (capi.cpp, plan.cpp) links against, so that code can be
// built with g++ and AddressSanitizer / UndefinedBehaviorSanitizer on a
// machine without a GPU.  TEST INFRASTRUCTURE ONLY: nothing here computes or
// touches the pointers it is given.  Every launcher counts its call; with
// g_ok clear it reports failure (host_driver.cpp checks that validation
// rejects bad calls before any launcher runs), with g_ok set it reports
// success, so the whole host side of a call (stage loops, chunk tables,
// stream and event ordering) runs under the sanitizers.
#include <hip/hip_runtime.h>

#include "../../headwise_chunked_context_stage_amd/csrc/upipe_internal.h"

int g_launches = 0;  // kernel launchers reached
int g_fills = 0;     // zero fills reached (the empty-sequence path)
int g_hip_calls = 0; // HIP runtime calls reached
bool g_ok = false;   // launchers and runtime calls succeed

namespace {
hipError_t launched() {
  ++g_launches;
  return g_ok ? hipSuccess : hipErrorNotSupported;
}
hipError_t hip_call() {
  ++g_hip_calls;
  return g_ok ? hipSuccess : hipErrorNotSupported;
}
// distinct fake handles (never dereferenced by the code under test)
char g_handles[64];
int g_next_handle = 0;
template <typename T>
T fake_handle() {
  return reinterpret_cast<T>(&g_handles[(g_next_handle++) % 64]);
}
}  // namespace

namespace upipe {
namespace bf16 {
hipError_t proj(const void*, int64_t, int64_t, int, const ChunkTable&, const Rope&, const NormArgs&,
                hipStream_t) { return launched(); }
hipError_t attn_fwd(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t bwd_pre(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t attn_dkv(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t attn_dq(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t dw(const void*, int64_t, int64_t, int, const ChunkTable&, float*, hipStream_t) { return launched(); }
hipError_t dx(float*, int64_t, int64_t, int, const ChunkTable&, hipStream_t) { return launched(); }
hipError_t oproj(float*, int64_t, int64_t, int, const ChunkTable&, int64_t, hipStream_t) { return launched(); }
hipError_t dout(const void*, int64_t, int64_t, int, const ChunkTable&, int64_t, hipStream_t) { return launched(); }
hipError_t dwo(const void*, int64_t, int64_t, int, const ChunkTable&, int64_t, float*, hipStream_t) { return launched(); }
hipError_t mfma_ceiling(int, int, double*, hipStream_t) { return launched(); }
}  // namespace bf16
namespace f32 {
hipError_t proj(const void*, int64_t, int64_t, int, const ChunkTable&, hipStream_t) { return launched(); }
hipError_t attn_fwd(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t bwd_pre(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t attn_dkv(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t attn_dq(const AttnArgs&, hipStream_t) { return launched(); }
hipError_t dw(const void*, int64_t, int64_t, int, const ChunkTable&, float*, hipStream_t) { return launched(); }
hipError_t dx(float*, int64_t, int64_t, int, const ChunkTable&, hipStream_t) { return launched(); }
hipError_t rope(float*, int, int64_t, int, const Rope&, int, hipStream_t) { return launched(); }
hipError_t oproj(float*, int64_t, int64_t, int, const ChunkTable&, int64_t, hipStream_t) { return launched(); }
hipError_t dout(const void*, int64_t, int64_t, int, const ChunkTable&, int64_t, hipStream_t) { return launched(); }
hipError_t dwo(const void*, int64_t, int64_t, int, const ChunkTable&, int64_t, float*, hipStream_t) { return launched(); }
}  // namespace f32
namespace norm {
hipError_t fwd_f32(float*, int, int64_t, int, const float*, float, float*, float*, hipStream_t) { return launched(); }
hipError_t bwd(const float*, const float*, const float*, const void*, int, void*, int, float*, int,
               int64_t, int, hipStream_t) { return launched(); }
hipError_t gamma_sum(float*, const float*, int, int64_t, int, int, hipStream_t) { return launched(); }
}  // namespace norm
hipError_t fill_zero(void*, size_t, hipStream_t) {
  ++g_fills;
  return hipSuccess;
}
}  // namespace upipe

extern "C" {
hipError_t hipEventCreate(hipEvent_t* e) {
  if (g_ok) *e = fake_handle<hipEvent_t>();
  return hip_call();
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  if (g_ok) *e = fake_handle<hipEvent_t>();
  return hip_call();
}
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  if (g_ok) *ms = 1.f;
  return hip_call();
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hip_call(); }
hipError_t hipEventSynchronize(hipEvent_t) { return hip_call(); }
hipError_t hipGetDevice(int* d) {
  if (g_ok) *d = 0;
  return hip_call();
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
  if (g_ok) *s = fake_handle<hipStream_t>();
  return hip_call();
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned) { return hip_call(); }
}
