// peak.hip -- achievable-peak probes for the measurement harness (not part of
// the hot path): a dense loop of independent v_mfma_f32_32x32x16_bf16 with two
// waves per SIMD (the rate the matrix cores reach with no memory traffic); a
// 16-byte-per-lane device copy; and the append's own data movement without
// its arithmetic (the same bf16 loads, 4-byte code stores and scale-byte
// stores, scattered through the same slot mapping).  bench.py reports kernel
// throughput against the published peaks and these measured ones.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

__global__ __launch_bounds__(256) void copy16(const uint4* __restrict__ a, uint4* __restrict__ b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) b[i] = a[i];
}

// One thread per 8 bf16 of K and of V (the append's half blocks): loads them,
// folds each 16 bytes into a 4-byte word (no quantization), and stores the
// words and one byte per even lane where the append stores codes and scales,
// with the append's cache hints.
__global__ __launch_bounds__(256) void append_traffic(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                      const int64_t* __restrict__ slots, int64_t n, int hpt,
                                                      int64_t num_slots, uint32_t* __restrict__ kc,
                                                      uint32_t* __restrict__ vc, uint8_t* __restrict__ ks,
                                                      uint8_t* __restrict__ vs) {
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (h >= n) return;
  const int64_t token = h / hpt;
  const int j = (int)(h - token * hpt);
  const int64_t slot = slots[token];
  // the append's cache hints: streaming loads, write-back stores
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k) + h);
  const u32x4 y = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v) + h);
  if (slot < 0 || slot >= num_slots) return;
  const uint32_t a = x[0] ^ x[1] ^ x[2] ^ x[3], b = y[0] ^ y[1] ^ y[2] ^ y[3];
  const int64_t o = slot * hpt + j;
  kc[o] = a;
  vc[o] = b;
  if ((j & 1) == 0) {
    ks[o >> 1] = (uint8_t)a;
    vs[o >> 1] = (uint8_t)b;
  }
}

}  // namespace

// Copies n16 16-byte words from src to dst on `stream` (both 16-byte
// aligned).  Returns 0, or -1 on a bad argument or launch error.
extern "C" int nvfp4kv_copy_probe(const void* src, void* dst, int64_t n16, void* stream) {
  if (!src || !dst || n16 <= 0 || ((uintptr_t)src | (uintptr_t)dst) % 16) return -1;
  hipLaunchKernelGGL(copy16, dim3((uint32_t)((n16 + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The append's data movement for num_tokens rows of num_kv_heads x head_dim
// bf16 K and V (16-byte aligned) through slot_mapping into caches laid out as
// the append's ([num_slots][H][D/2] code bytes, [num_slots][H][D/16] scale
// bytes; head_dim a multiple of 16).  Slots outside [0, num_slots) are
// skipped.  Returns 0, or -1 on a bad argument or launch error.
extern "C" int nvfp4kv_append_traffic_probe(const void* k, const void* v, const int64_t* slot_mapping,
                                            int64_t num_tokens, int num_kv_heads, int head_dim,
                                            int64_t num_slots, void* k_cache, void* v_cache, void* k_sf,
                                            void* v_sf, void* stream) {
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_sf || !v_sf || num_tokens <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || head_dim % 16 || ((uintptr_t)k | (uintptr_t)v) % 16 ||
      ((uintptr_t)k_cache | (uintptr_t)v_cache) % 4)
    return -1;
  const int hpt = num_kv_heads * head_dim / 8;
  const int64_t n = num_tokens * hpt;
  hipLaunchKernelGGL(append_traffic, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)k, (const uint4*)v, slot_mapping, n, hpt, num_slots, (uint32_t*)k_cache,
                     (uint32_t*)v_cache, (uint8_t*)k_sf, (uint8_t*)v_sf);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

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
