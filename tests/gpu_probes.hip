// gpu_probes.hip -- GPU checks of compiler builtins the kernels rely on.
// Built into tests/libnvfp4kv_probes.so and driven by tests/test_gpu_probes.py.
//  * e2m1 transition scan: converts every fp32 pattern of one sign in
//    [0, +inf] with the hardware conversion and with the software encoder of
//    nvfp4kv_codec.hpp, and records where the code changes;
//  * MFMA lane layouts of v_mfma_f32_32x32x16_bf16 / 16x16x32_bf16;
//  * the FP4 -> bf16 / fp32 hardware conversions with a scale operand;
//  * the E4M3 (fp8) -> fp32 pair conversion used to decode block scales;
//  * the conversions and the scaled FP4 x FP8 matrix instruction of the MX
//    score variant (f32 -> E4M3 pairs, f16 pairs -> E2M1).
#include <hip/hip_runtime.h>
#include "../nvfp4_paged_kv_amd/csrc/nvfp4kv_codec.hpp"

using namespace nvfp4kv;

constexpr uint32_t kScanEnd = 0x7F800000u;  // +inf, last pattern scanned
constexpr uint32_t kPerThread = 4096u;

__device__ __forceinline__ uint32_t code_of(uint32_t pat, int mode) {
  float y = u2f(pat);
  if (mode == 0) {
    uint32_t b = cvt_pk_e2m1<0>(0u, y, 0.0f);
    return b & 0xFFu;  // low nibble: y, high nibble: +0
  }
  return (pat >> 28 & 8u) | e2m1_mag_from_abs_bits(pat & 0x7FFFFFFFu);
}

// transitions: pairs (pattern, code) where code(pattern) != code(pattern-1)
__global__ void e2m1_scan_kernel(uint32_t sign, int mode, uint32_t* count, uint32_t* buf, uint32_t cap) {
  uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t lo = t * kPerThread;
  if (lo > kScanEnd) return;
  uint64_t hi = lo + kPerThread - 1;
  if (hi > kScanEnd) hi = kScanEnd;
  uint32_t prev = lo == 0 ? 0xFFFFFFFFu : code_of(sign | (uint32_t)(lo - 1), mode);
  for (uint64_t p = lo; p <= hi; ++p) {
    uint32_t c = code_of(sign | (uint32_t)p, mode);
    if (c != prev) {
      uint32_t i = atomicAdd(count, 1u);
      if (i < cap) { buf[2 * i] = (uint32_t)p; buf[2 * i + 1] = c; }
    }
    prev = c;
  }
}

__global__ void cvt_pairs_kernel(const float* in, int n, uint32_t* out) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = cvt_pk_e2m1<0>(0u, in[2 * i], in[2 * i + 1]);
  if (i < n) out[n + i] = cvt_pk_e2m1<2>(0u, in[2 * i], in[2 * i + 1]);
}

// byte b -> two bf16 via the scaled hardware conversion, and two fp32
__global__ void fp4_to_bf16_kernel(const float* scales, int nscale, uint32_t* out_bf16, float* out_f32) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 256 * nscale) return;
  uint32_t byte = i & 255;
  float sc = scales[i >> 8];
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte, sc, 0);
  uint32_t rb;
  __builtin_memcpy(&rb, &r, 4);
  out_bf16[i] = rb;
  auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, sc, 0);
  out_f32[2 * i] = f[0];
  out_f32[2 * i + 1] = f[1];
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One wave.  A: [M][K] fp32, B: [K][N] fp32 (values exact in bf16).
// Assumed operand layout (32x32x16): lane l holds A[l%32][8*(l/32) + j] and
// B[8*(l/32) + j][l%32], j = 0..7; result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__global__ void mfma32_kernel(const float* A, const float* B, float* D) {
  int l = threadIdx.x;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)A[(l % 32) * 16 + 8 * (l / 32) + j];
    b[j] = (__bf16)B[(8 * (l / 32) + j) * 32 + l % 32];
  }
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  for (int r = 0; r < 16; ++r) D[(8 * (r / 4) + 4 * (l / 32) + r % 4) * 32 + l % 32] = c[r];
}

// 16x16x32: lane l holds A[l%16][8*(l/16) + j], B[8*(l/16) + j][l%16];
// register r of lane l is D[4*(l/16) + r][l%16].
__global__ void mfma16_kernel(const float* A, const float* B, float* D) {
  int l = threadIdx.x;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)A[(l % 16) * 32 + 8 * (l / 16) + j];
    b[j] = (__bf16)B[(8 * (l / 16) + j) * 16 + l % 16];
  }
  f32x4 c = {};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  for (int r = 0; r < 4; ++r) D[(4 * (l / 16) + r) * 16 + l % 16] = c[r];
}

// every E4M3 byte b decoded by the pair conversion: thread t < 128 converts the
// dword holding bytes (2t, 2t+1) in its low half and (2t+1, 2t) in its high
// half, so both word selects see every byte in both positions
__global__ void fp8_pairs_kernel(float* out) {
  const uint32_t t = threadIdx.x;
  if (t >= 128) return;
  const uint32_t b0 = 2 * t, b1 = 2 * t + 1;
  const uint32_t w = b0 | (b1 << 8) | (b1 << 16) | (b0 << 24);
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const f2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  out[4 * t + 0] = lo.x;  // byte b0
  out[4 * t + 1] = lo.y;  // byte b1
  out[4 * t + 2] = hi.x;  // byte b1
  out[4 * t + 3] = hi.y;  // byte b0
}

// The scaled FP4 x FP8 product v_mfma_scale_f32_32x32x64_f8f6f4 (A in E2M1,
// B in E4M3, one E8M0 scale per lane for A and for B, byte 0 of its scale
// word): one wave, the register contents as given (a: 8 dwords per lane,
// the first 4 used for FP4; b: 8 dwords per lane; sa, sb: one word per
// lane); d: the 16 result registers of each lane.
typedef int v8i __attribute__((ext_vector_type(8)));
__global__ void mfma_scale_kernel(const int* a, const int* b, const int* sa, const int* sb, float* d) {
  const int l = threadIdx.x;
  v8i av, bv;
  for (int j = 0; j < 8; ++j) {
    av[j] = a[l * 8 + j];
    bv[j] = b[l * 8 + j];
  }
  const int xa = sa[l], xb = sb[l];
  f32x16 c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, (f32x16){}, 4, 0, 0, xa, 0, xb);
  // the sources stay live until after the instruction, so that its result
  // registers cannot overlap them
  asm volatile("" : "+v"(c) : "v"(av), "v"(bv), "v"(xa), "v"(xb));
  for (int r = 0; r < 16; ++r) d[l * 16 + r] = c[r];
}

// Every bf16 pattern through the f32 -> E4M3 pair conversion the MXFP8 query
// load uses: thread t converts patterns 4t .. 4t+3 (as f32) into the bytes
// 0 .. 3 of one word (two conversions, word select 0 then 1).
__global__ void fp8_from_bf16_kernel(uint32_t* out) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= 16384u) return;
  typedef short s2 __attribute__((ext_vector_type(2)));
  float v[4];
  for (int i = 0; i < 4; ++i) v[i] = u2f((4u * t + (uint32_t)i) << 16);
  s2 o = {};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, v[0], v[1], 1.0f, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, v[2], v[3], 1.0f, true);
  out[t] = __builtin_bit_cast(uint32_t, o);
}

// Every f16 pattern through the f16 pair -> E2M1 conversion the K
// requantization uses: thread t converts patterns 8t .. 8t+7 into the
// nibbles 0 .. 7 of one word (pair j into byte j).
__global__ void fp4_from_f16_kernel(uint32_t* out) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= 8192u) return;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v[4];
  for (int j = 0; j < 4; ++j) {
    const uint32_t bits = (8u * t + 2u * j) | ((8u * t + 2u * j + 1u) << 16);
    v[j] = __builtin_bit_cast(h2, bits);
  }
  uint32_t o = 0;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(o, v[0], 1.0f, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(o, v[1], 1.0f, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(o, v[2], 1.0f, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(o, v[3], 1.0f, 3);
  out[t] = o;
}

// The cross-row lane swaps the decode's softmax uses for its column maxima:
// one wave, x = in[lane] as both operands; out holds, per lane, the two
// results of v_permlane16_swap then those of v_permlane32_swap.
__global__ void permlane_swap_kernel(const uint32_t* in, uint32_t* out) {
  const int l = threadIdx.x;
  const uint32_t x = in[l];
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  out[l] = a[0];
  out[64 + l] = a[1];
  out[128 + l] = b[0];
  out[192 + l] = b[1];
}

extern "C" {
// All pointers are device pointers; every call synchronizes the device.
int probe_e2m1_scan(uint32_t sign, int mode, uint32_t* count, uint32_t* buf, uint32_t cap) {
  uint64_t threads = ((uint64_t)kScanEnd + kPerThread) / kPerThread;
  uint32_t blocks = (uint32_t)((threads + 255) / 256);
  e2m1_scan_kernel<<<blocks, 256>>>(sign, mode, count, buf, cap);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_cvt_pairs(const float* in, int n, uint32_t* out) {
  cvt_pairs_kernel<<<(n + 255) / 256, 256>>>(in, n, out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_fp4_to_bf16(const float* scales, int nscale, uint32_t* out_bf16, float* out_f32) {
  fp4_to_bf16_kernel<<<(256 * nscale + 255) / 256, 256>>>(scales, nscale, out_bf16, out_f32);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_mfma32(const float* A, const float* B, float* D) {
  mfma32_kernel<<<1, 64>>>(A, B, D);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_fp8_pairs(float* out) {
  fp8_pairs_kernel<<<1, 128>>>(out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_fp8_from_bf16(uint32_t* out) {  // out: 16384 words
  fp8_from_bf16_kernel<<<64, 256>>>(out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_fp4_from_f16(uint32_t* out) {  // out: 8192 words
  fp4_from_f16_kernel<<<32, 256>>>(out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_mfma_scale(const int* a, const int* b, const int* sa, const int* sb, float* d) {
  mfma_scale_kernel<<<1, 64>>>(a, b, sa, sb, d);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_permlane_swap(const uint32_t* in, uint32_t* out) {  // in: 64 words, out: 256
  permlane_swap_kernel<<<1, 64>>>(in, out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
int probe_mfma16(const float* A, const float* B, float* D) {
  mfma16_kernel<<<1, 64>>>(A, B, D);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
}
