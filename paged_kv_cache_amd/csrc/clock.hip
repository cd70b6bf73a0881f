// clock.hip -- pa_clock_probe: the shader clock the chip sustains while every
// SIMD issues bf16 matrix products, for quoting MFMA throughput against the
// peak at the measured clock as well as the peak at the rated 2.4 GHz.
//
// Each wave runs four independent chains of v_mfma_f32_32x32x16_bf16 for a
// fixed number of steps and reads two counters before and after: the core
// clock counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime).  Its clock is cycles / (ticks / 100 MHz).

#include "device.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void clock_probe_kernel(float *ghz, int n_waves, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f / (1 + ((lane + i) & 7)));
    b[i] = (__bf16)(0.5f / (1 + ((lane * 3 + i) & 7)));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (lane == 0 && wave < n_waves) {
    const double ticks = (double)(r1 - r0);
    // the sum is finite and small: adding 0 * s keeps the products live
    ghz[wave] = ticks > 0 ? (float)((double)(t1 - t0) / (ticks * 10.0)) + 0.f * s : 0.f;
  }
}

}  // namespace

int launch_clock_probe(float *ghz, int n_waves, int iters, hipStream_t stream) {
  const int blocks = (n_waves + kProbeThreads / 64 - 1) / (kProbeThreads / 64);
  hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, ghz,
                     n_waves, iters);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
