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
// Work decomposition: one thread per (token, 16-element block) handles that
// block of K and of V.  Lanes of a wave cover consecutive blocks, so the bf16
// reads are fully coalesced (a wave reads 2 KiB of K and 2 KiB of V) and, with
// the NHD cache layout, the packed writes of one token row are one contiguous
// H*D/2-byte run (H*D/16 scale bytes beside it).
#include <hip/hip_runtime.h>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// Largest |x| over 16 bf16 values as a bf16 bit pattern (sign cleared).  For
// finite values the integer order of the magnitude bits is the numeric order;
// a result >= 0x7F80 means the block holds an inf or a NaN.
__device__ __forceinline__ uint32_t amax_bits16(const uint32_t (&w)[8]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t a = w[i] & 0x7FFF7FFFu;
    u16x2 v;
    __builtin_memcpy(&v, &a, 4);
    m = __builtin_elementwise_max(m, v);
  }
  return m[0] > m[1] ? m[0] : m[1];
}

// Block scale from amax: sf byte and the element multiplier r.
__device__ __forceinline__ void block_scale(float a, float g, float d6, uint32_t& sf, float& r) {
  float s = a / d6;  // IEEE-correct fp32 division
  sf = e4m3_encode(s);
  float den = e4m3_decode(sf) * g;
  r = sf ? 1.0f / den : 0.0f;
}

// Rare path: the block holds inf/NaN, or 1/(S g) overflowed.  Element by
// element in software; NaN is ignored by the amax and encodes to magnitude 0.
__device__ __attribute__((noinline)) uint2 quantize_block_slow(const uint32_t (&w)[8], float g,
                                                               float d6, uint32_t& sf_out) {
  float a = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float x = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    float m = __builtin_fabsf(x);
    if (m > a) a = m;
  }
  uint32_t sf;
  float r;
  block_scale(a, g, d6, sf, r);
  uint32_t out[2] = {0u, 0u};
  for (int i = 0; i < 16; ++i) {
    uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
    float y = u2f(bits) * r;
    uint32_t yb = f2u(y) & 0x7FFFFFFFu;
    uint32_t mag = yb > 0x7F800000u ? 0u : e2m1_mag_from_abs_bits(yb);
    uint32_t code = ((bits >> 28) & 8u) | mag;
    out[i >> 3] |= code << (4 * (i & 7));
  }
  sf_out = sf;
  return make_uint2(out[0], out[1]);
}

// One 16-element block: 8 dwords of bf16 pairs (element 2i in the low half).
__device__ __forceinline__ uint2 quantize_block(const uint4& lo, const uint4& hi, float g, float d6,
                                                uint32_t& sf) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t am = amax_bits16(w);
  float r;
  block_scale(u2f(am << 16), g, d6, sf, r);
  if (__builtin_expect(am >= 0x7F80u || !(r < 3.0e38f), 0)) return quantize_block_slow(w, g, d6, sf);
#if NVFP4KV_E2M1_SOFTWARE
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
    uint32_t yb = f2u(u2f(bits) * r);
    uint32_t code = ((yb >> 28) & 8u) | e2m1_mag_from_abs_bits(yb & 0x7FFFFFFFu);
    out[i >> 3] |= code << (4 * (i & 7));
  }
  return make_uint2(out[0], out[1]);
#else
  // y = x * r keeps the sign of x (r >= +0, no NaN reaches here), so the
  // hardware conversion's sign bit is the input's.
  uint32_t p0 = 0u, p1 = 0u;
  p0 = cvt_pk_e2m1<0>(p0, bf16_lo(w[0]) * r, bf16_hi(w[0]) * r);
  p0 = cvt_pk_e2m1<1>(p0, bf16_lo(w[1]) * r, bf16_hi(w[1]) * r);
  p0 = cvt_pk_e2m1<2>(p0, bf16_lo(w[2]) * r, bf16_hi(w[2]) * r);
  p0 = cvt_pk_e2m1<3>(p0, bf16_lo(w[3]) * r, bf16_hi(w[3]) * r);
  p1 = cvt_pk_e2m1<0>(p1, bf16_lo(w[4]) * r, bf16_hi(w[4]) * r);
  p1 = cvt_pk_e2m1<1>(p1, bf16_lo(w[5]) * r, bf16_hi(w[5]) * r);
  p1 = cvt_pk_e2m1<2>(p1, bf16_lo(w[6]) * r, bf16_hi(w[6]) * r);
  p1 = cvt_pk_e2m1<3>(p1, bf16_lo(w[7]) * r, bf16_hi(w[7]) * r);
  return make_uint2(p0, p1);
#endif
}

__global__ __launch_bounds__(256) void append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint2* __restrict__ k_cache, uint2* __restrict__ v_cache, uint8_t* __restrict__ k_sf,
    uint8_t* __restrict__ v_sf, uint32_t total_blocks, FastDiv bpt, int64_t num_slots,
    uint32_t* __restrict__ err) {
  const float gk = *k_scale, gv = *v_scale;
  if (!scale_ok(gk) || !scale_ok(gv)) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      atomicOr(err, (scale_ok(gk) ? 0u : kErrBadKScale) | (scale_ok(gv) ? 0u : kErrBadVScale));
    return;  // nothing is written for either tensor
  }
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  if (gid >= total_blocks) return;
  const uint32_t token = fastdiv(gid, bpt);
  const uint32_t j = gid - token * bpt.d;
  const int64_t slot = slots[token];
  if (slot < 0) return;  // padding
  if (slot >= num_slots) {
    atomicOr(err, kErrSlotOob);
    return;
  }
  const uint4 k0 = k[2 * (size_t)gid], k1 = k[2 * (size_t)gid + 1];
  const uint4 v0 = v[2 * (size_t)gid], v1 = v[2 * (size_t)gid + 1];
  uint32_t ksf, vsf;
  const uint2 kp = quantize_block(k0, k1, gk, 6.0f * gk, ksf);
  const uint2 vp = quantize_block(v0, v1, gv, 6.0f * gv, vsf);
  // NHD: the cache row of a slot is [slot][H_kv][D/2] bytes, its scale row
  // [slot][H_kv][D/16]; block j of the token is block j of that row.
  const size_t o = (size_t)slot * bpt.d + j;
  // one 8-byte store per lane: a wave covers whole cache lines of the row
  __builtin_nontemporal_store(((uint64_t)kp.y << 32) | kp.x, (uint64_t*)&k_cache[o]);
  __builtin_nontemporal_store(((uint64_t)vp.y << 32) | vp.x, (uint64_t*)&v_cache[o]);
  k_sf[o] = (uint8_t)ksf;
  v_sf[o] = (uint8_t)vsf;
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
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 8) || !aligned(v_cache, 8) ||
      !aligned(slot_mapping, 8) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(dev_error, 4))
    return NVFP4KV_EINVAL;
  const int64_t bpt = (int64_t)num_kv_heads * head_dim / 16;
  const int64_t total = num_tokens * bpt;
  if (bpt >= (1ll << 31) || total >= (1ll << 31)) return NVFP4KV_EUNSUPPORTED;
  const uint32_t grid = (uint32_t)((total + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)k, (const uint4*)v, slot_mapping, k_scale, v_scale,
                     (uint2*)k_cache, (uint2*)v_cache, k_sf, v_sf, (uint32_t)total,
                     make_fastdiv((uint32_t)bpt), num_pages * page_size, dev_error);
  return hipGetLastError() == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP;
}
