// peak.hip -- achievable-peak probe for the measurement harness (not part of
// the attention path): a dense loop of independent v_mfma_f32_32x32x16_bf16
// with two waves per SIMD, the rate the matrix cores reach on this device
// with no memory traffic.  bench.py reports kernel throughput against both
// the published peak and this measured one.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;  // independent accumulators per wave

__global__ __launch_bounds__(512) void mfma_loop(int iters, float* out) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(t + i));
    b[i] = (__bf16)(0.002f * (float)(t - i));
  }
  f32x16 acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = (f32x16){};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kAcc; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  out[blockIdx.x * 512 + t] = s;  // keeps the loop; the values are not used
}

}  // namespace

// Runs blocks x 512 threads, each wave issuing iters x 8 MFMAs (32,768 flops
// each) on `stream`; out needs blocks x 512 floats.  Returns 0, or -1 on a
// bad argument or launch error.
extern "C" int nvfp4kv_mfma_peak_probe(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" double nvfp4kv_mfma_peak_probe_flops(int blocks, int iters) {
  return (double)blocks * 8 /* waves */ * iters * kAcc * 32768.0;
}
