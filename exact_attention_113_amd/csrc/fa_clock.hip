// Clock probe, a measurement aid outside the attention path: the shader
// clock the chip runs at while other kernels occupy it. One wave spins on a
// dependent chain of fused multiply-adds between two reads each of the
// shader cycle counter (s_memtime) and of the 100 MHz constant clock
// (s_memrealtime); their deltas give the clock over the spin. The wave uses
// no LDS and a few registers, so it fits beside a kernel that fills the
// CUs' LDS, and the clock it sees is the one that kernel runs at.
#include "fa_internal.h"

namespace fa {
namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* out, int iters) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  float x = (float)threadIdx.x * 1e-3f, y = 1.0001f;
  for (int i = 0; i < iters; ++i) {
    x = fmaf(x, y, 1e-7f);
    y = fmaf(y, 0.99999f, 1e-6f);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = t1 - t0;
    // Keeps the chain live; the value means nothing.
    out[2] = (uint64_t)__float_as_uint(x + y);
  }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t* out, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace fa
