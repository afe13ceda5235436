// append.hip -- NVFP4 quantize + paged-KV append through a slot mapping (gfx950).
//
// FlashInfer PR #6204 page ("NVFP4 KV cache append: host sync removed"):
//   * the append quantizes new K/V rows to NVFP4 and writes them to the cache
//     positions a slot mapping names (introduction, append-function section);
//   * the global decode scales arrive as device fp32 scalars and are checked
//     by the append kernel itself, only when there are rows to write, so the
//     host never reads them and never synchronizes (the
//     `_as_float32_scalar_tensors` change and the docstring change);
//   * a bad device scale surfaces as a device-side error (error-handling
//     section).  Here it sets a bit in a caller-owned device error word and
//     the kernel writes nothing.
//
// Work decomposition: one thread per half block (8 consecutive elements) of K
// and of V; lanes 2i and 2i+1 hold one 16-element block and exchange their
// partial amax.  Every load instruction of a wave then reads 1 KiB of
// contiguous bf16 (16 bytes per lane), and with the NHD cache layout the
// packed writes of one token row are one contiguous H*D/2-byte run (4 bytes
// per lane), its H*D/16 scale bytes beside it.
#include <hip/hip_runtime.h>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// Largest |x| over 8 bf16 values as a bf16 bit pattern (sign cleared).  For
// finite values the integer order of the magnitude bits is the numeric order;
// a result >= 0x7F80 means the values hold an inf or a NaN.
__device__ __forceinline__ uint32_t amax_bits8(const uint4& x) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = w[i] & 0x7FFF7FFFu;
    u16x2 v;
    __builtin_memcpy(&v, &a, 4);
    m = __builtin_elementwise_max(m, v);
  }
  return m[0] > m[1] ? m[0] : m[1];
}

// The value of the partner lane (lane ^ 1) of a block's lane pair.
__device__ __forceinline__ uint32_t pair_swap(uint32_t x) {
  // DPP quad permutation [1, 0, 3, 2]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

// Block scale from amax: sf byte and the element multiplier r.
__device__ __forceinline__ void block_scale(float a, float g, float d6, uint32_t& sf, float& r) {
  float s = a / d6;  // IEEE-correct fp32 division
  sf = e4m3_encode(s);
  float den = e4m3_decode(sf) * g;
  r = sf ? 1.0f / den : 0.0f;
}

// Rare path (both lanes of the pair take it together; inlined: a call would
// give the kernel a stack in scratch memory): the block holds
// inf/NaN, or 1/(S g) overflowed.  Element by element in software; NaN is
// ignored by the amax and encodes to magnitude 0.
__device__ __forceinline__ uint32_t quantize_half_slow(const uint4& x, float g, float d6,
                                                          uint32_t& sf_out) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float a = 0.0f;
  for (int i = 0; i < 8; ++i) {
    float m = __builtin_fabsf(u2f((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16)));
    if (m > a) a = m;  // false for NaN
  }
  a = __builtin_fmaxf(a, u2f(pair_swap(f2u(a))));
  uint32_t sf;
  float r;
  block_scale(a, g, d6, sf, r);
  uint32_t out = 0u;
  for (int i = 0; i < 8; ++i) {
    uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
    float y = u2f(bits) * r;
    uint32_t yb = f2u(y) & 0x7FFFFFFFu;
    uint32_t mag = yb > 0x7F800000u ? 0u : e2m1_mag_from_abs_bits(yb);
    out |= (((bits >> 28) & 8u) | mag) << (4 * i);
  }
  sf_out = sf;
  return out;
}

// This lane's 8 elements of a 16-element block (4 dwords of bf16 pairs,
// element 2i in the low half): 4 packed code bytes, and the block's sf byte.
__device__ __forceinline__ uint32_t quantize_half(const uint4& x, float g, float d6, uint32_t& sf) {
  uint32_t am = amax_bits8(x);
  am = max(am, pair_swap(am));
  float r;
  block_scale(u2f(am << 16), g, d6, sf, r);
  if (__builtin_expect(am >= 0x7F80u || !(r < 3.0e38f), 0)) return quantize_half_slow(x, g, d6, sf);
  // y = x * r keeps the sign of x (r >= +0, no NaN reaches here), so the
  // hardware conversion's sign bit is the input's.
  uint32_t p = 0u;
  p = cvt_pk_e2m1<0>(p, bf16_lo(x.x) * r, bf16_hi(x.x) * r);
  p = cvt_pk_e2m1<1>(p, bf16_lo(x.y) * r, bf16_hi(x.y) * r);
  p = cvt_pk_e2m1<2>(p, bf16_lo(x.z) * r, bf16_hi(x.z) * r);
  p = cvt_pk_e2m1<3>(p, bf16_lo(x.w) * r, bf16_hi(x.w) * r);
  return p;
}

__global__ __launch_bounds__(256) void append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint32_t* __restrict__ k_cache, uint32_t* __restrict__ v_cache, uint8_t* __restrict__ k_sf,
    uint8_t* __restrict__ v_sf, uint32_t total_halves, FastDiv hpt, int64_t num_slots,
    uint32_t* __restrict__ err) {
  const float gk = *k_scale, gv = *v_scale;
  if (!scale_ok(gk) || !scale_ok(gv)) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      atomicOr(err, (scale_ok(gk) ? 0u : kErrBadKScale) | (scale_ok(gv) ? 0u : kErrBadVScale));
    return;  // nothing is written for either tensor
  }
  // Half blocks per token are even, so a lane pair never straddles a token
  // and both lanes of a pair leave or stay together below.
  const uint32_t h = blockIdx.x * 256u + threadIdx.x;
  if (h >= total_halves) return;
  const uint32_t token = fastdiv(h, hpt);
  const uint32_t j = h - token * hpt.d;  // half block within the token row
  const int64_t slot = slots[token];
  // the bf16 rows are read once: streaming (non-temporal) loads
  const u32x4 kr = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k) + h);
  const u32x4 vr = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v) + h);
  const uint4 kx = make_uint4(kr[0], kr[1], kr[2], kr[3]), vx = make_uint4(vr[0], vr[1], vr[2], vr[3]);
  uint32_t ksf, vsf;
  const uint32_t kp = quantize_half(kx, gk, 6.0f * gk, ksf);
  const uint32_t vp = quantize_half(vx, gv, 6.0f * gv, vsf);
  if (slot < 0) return;  // padding
  if (slot >= num_slots) {
    atomicOr(err, kErrSlotOob);
    return;
  }
  // NHD: the cache row of a slot is [slot][H_kv][D/2] bytes (4 per half
  // block), its scale row [slot][H_kv][D/16] (1 per block).
  // Plain (write-back) stores: the scattered 512-byte rows merge in L2
  // (streaming stores measured ~2% slower here).
  const size_t o = (size_t)slot * hpt.d + j;
  k_cache[o] = kp;
  v_cache[o] = vp;
  if ((j & 1) == 0) {
    k_sf[o >> 1] = (uint8_t)ksf;
    v_sf[o >> 1] = (uint8_t)vsf;
  }
}

}  // namespace
}  // namespace nvfp4kv

using namespace nvfp4kv;

extern "C" int nvfp4_append_paged_kv(const void* k, const void* v, const int64_t* slot_mapping,
                                     int64_t num_tokens, const float* k_scale,
                                     const float* v_scale, uint8_t* k_cache, uint8_t* v_cache,
                                     uint8_t* k_sf, uint8_t* v_sf, int64_t num_pages,
                                     int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                                     uint32_t* dev_error, void* stream) {
  if (num_tokens < 0 || num_pages < 0 || page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      head_dim % 16 != 0)
    return NVFP4KV_EINVAL;
  // No rows: nothing is written, so nothing (the scales included) is checked.
  if (num_tokens == 0) return NVFP4KV_OK;
  if (!k || !v || !slot_mapping || !k_scale || !v_scale || !k_cache || !v_cache || !k_sf ||
      !v_sf || !dev_error)
    return NVFP4KV_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 4) || !aligned(v_cache, 4) ||
      !aligned(slot_mapping, 8) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(dev_error, 4))
    return NVFP4KV_EINVAL;
  const int64_t hpt = (int64_t)num_kv_heads * head_dim / 8;  // half blocks per token (even)
  const int64_t total = num_tokens * hpt;
  if (hpt >= (1ll << 31) || total >= (1ll << 31)) return NVFP4KV_EUNSUPPORTED;
  const uint32_t grid = (uint32_t)((total + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)k, (const uint4*)v, slot_mapping, k_scale, v_scale,
                     (uint32_t*)k_cache, (uint32_t*)v_cache, k_sf, v_sf, (uint32_t)total,
                     make_fastdiv((uint32_t)hpt), num_pages * page_size, dev_error);
  return hipGetLastError() == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP;
}
