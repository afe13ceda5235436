// peak.hip -- achievable-peak probes for the measurement harness (not part of
// the hot path): a dense loop of independent v_mfma_f32_32x32x16_bf16 with two
// waves per SIMD (the rate the matrix cores reach with no memory traffic, with
// smooth or with random operand bits); a
// 16-byte-per-lane device copy; the append's own data movement without its
// arithmetic (the same bf16 loads, 4-byte code stores and scale-byte stores,
// scattered through the same slot mapping); and the decode's loads without
// its arithmetic (the same waves, page lookups and per-lane code and scale
// loads, one or two tiles ahead).  bench.py reports kernel throughput
// against the published peaks and these measured ones.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;  // independent accumulators per wave

// RANDOM: operands of random sign, exponent and mantissa bits (each lane's
// own, like real data) instead of smooth ramps: the matrix cores' power, and
// with it the clock the part holds, depends on the operand bits.
template <bool RANDOM>
__global__ __launch_bounds__(512) void mfma_loop(int iters, float* out) {
  const int t = threadIdx.x;
  bf16x8 a, b;
  uint32_t x = (uint32_t)(blockIdx.x * 512 + t) * 2654435761u + 12345u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (RANDOM) {
      // bf16 bit patterns with exponents in [2^-4, 2^4): finite, nonzero
      x = x * 1664525u + 1013904223u;
      const uint16_t ha = (uint16_t)((x >> 16) & 0x807Fu) | (uint16_t)((123u + ((x >> 8) & 7u)) << 7);
      x = x * 1664525u + 1013904223u;
      const uint16_t hb = (uint16_t)((x >> 16) & 0x807Fu) | (uint16_t)((123u + ((x >> 8) & 7u)) << 7);
      a[i] = __builtin_bit_cast(__bf16, ha);
      b[i] = __builtin_bit_cast(__bf16, hb);
    } else {
      a[i] = (__bf16)(0.001f * (float)(t + i));
      b[i] = (__bf16)(0.002f * (float)(t - i));
    }
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

// The decode's reads for head_dim 128 with two KV heads per wave: one wave
// per (request, chunk, head pair), 8 waves per workgroup, the same item
// order; per 32-key tile and lane (key k of a 16-key block, quarter q) the
// 32 code bytes of K and of V at byte 32q of the pair's 128-byte line and
// the dword of the pair's scale row that holds the quarter's four scales;
// page ids two tiles ahead of the codes.  The codes of tile t + AHEAD are
// issued before tile t is folded (XOR) into one word per lane, which is
// stored at the end.
struct DecodeTraffic {
  const int32_t* kvp;
  const int32_t* pt;
  const int32_t* kvl;
  const uint8_t* kc;
  const uint8_t* vc;
  const uint8_t* ksf;
  const uint8_t* vsf;
  uint32_t* out;
  int64_t num_items, num_pages;
  int Hk, ps, chunk_len, max_chunks;
};

struct TileRaw {
  u32x4 k[2][2], v[2][2];
  uint32_t ks[2], vs[2];
};

template <int AHEAD>
__global__ __launch_bounds__(512) void decode_traffic(DecodeTraffic a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 6);
  if (item >= a.num_items) return;
  const int ngr = a.Hk / 2;
  const int hk0 = (int)(item % ngr) * 2;
  const int64_t bc = item / ngr;
  const int chunk = (int)(bc % a.max_chunks), b = (int)(bc / a.max_chunks);
  const int Lk = a.kvl[b];
  const int k0 = chunk * a.chunk_len;
  if (k0 >= Lk) return;
  const int k1 = min(Lk, k0 + a.chunk_len);
  const int ntiles = (k1 - k0 + 31) / 32;
  const int k16 = lane & 15, qq = lane >> 4;
  const int32_t* ptb = a.pt + a.kvp[b];
  auto lookup = [&](int t, int (&pg)[2]) {
    for (int kb = 0; kb < 2; ++kb) pg[kb] = ptb[min(k0 + 32 * t + 16 * kb + k16, k1 - 1) / a.ps];
  };
  auto load = [&](int t, const int (&pg)[2], TileRaw& r) {
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(k0 + 32 * t + 16 * kb + k16, k1 - 1);
      const int64_t page = (uint32_t)pg[kb] < (uint64_t)a.num_pages ? pg[kb] : 0;
      const int64_t row = (page * a.ps + key % a.ps) * a.Hk + hk0;
      const int64_t co = row * 64 + 32 * qq;
      r.k[kb][0] = *(const u32x4*)(a.kc + co);
      r.k[kb][1] = *(const u32x4*)(a.kc + co + 16);
      r.v[kb][0] = *(const u32x4*)(a.vc + co);
      r.v[kb][1] = *(const u32x4*)(a.vc + co + 16);
      r.ks[kb] = *(const uint32_t*)(a.ksf + row * 8 + 4 * qq);
      r.vs[kb] = *(const uint32_t*)(a.vsf + row * 8 + 4 * qq);
    }
  };
  auto fold = [](const TileRaw& r) {
    uint32_t x = 0;
    for (int kb = 0; kb < 2; ++kb) {
      for (int h = 0; h < 2; ++h)
        for (int c = 0; c < 4; ++c) x ^= r.k[kb][h][c] ^ r.v[kb][h][c];
      x ^= r.ks[kb] ^ r.vs[kb];
    }
    return x;
  };
  TileRaw ring[AHEAD + 1];
  int pg[2];
  for (int t = 0; t < AHEAD; ++t) {
    lookup(t, pg);
    load(t, pg, ring[t]);
  }
  uint32_t acc = 0;
  for (int t = 0; t < ntiles; t += AHEAD + 1) {
#pragma unroll
    for (int u = 0; u <= AHEAD; ++u) {  // the ring slot of tile t + u is u
      if (t + u >= ntiles) break;
      lookup(t + u + AHEAD, pg);  // past the last tile: clamped, unused
      load(t + u + AHEAD, pg, ring[(u + AHEAD) % (AHEAD + 1)]);
      acc ^= fold(ring[u]);
    }
  }
  a.out[item * 64 + lane] = acc;
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

// The decode's reads (head_dim 128, two KV heads per wave) for the items of
// a decode plan (num_items waves; chunk_len a multiple of 32), over caches
// and page tables laid out as the library's; out needs num_items x 64 words.
// ahead = 1 or 2: tiles whose codes are in flight while one is folded.
// Returns 0, or -1 on a bad argument or launch error.
extern "C" int nvfp4kv_decode_traffic_probe(const int32_t* kv_indptr, const int32_t* page_table,
                                            const int32_t* kv_lens, int64_t num_items, int num_kv_heads,
                                            int page_size, int64_t num_pages, int chunk_len, int max_chunks,
                                            const void* k_cache, const void* v_cache, const void* k_sf,
                                            const void* v_sf, uint32_t* out, int ahead, void* stream) {
  if (!kv_indptr || !page_table || !kv_lens || !k_cache || !v_cache || !k_sf || !v_sf || !out ||
      num_items <= 0 || num_kv_heads <= 0 || num_kv_heads % 2 || page_size <= 0 || num_pages <= 0 ||
      chunk_len <= 0 || chunk_len % 32 || max_chunks <= 0 || (ahead != 1 && ahead != 2) ||
      ((uintptr_t)k_cache | (uintptr_t)v_cache) % 16 || ((uintptr_t)k_sf | (uintptr_t)v_sf) % 4)
    return -1;
  DecodeTraffic a{kv_indptr, page_table, kv_lens, (const uint8_t*)k_cache, (const uint8_t*)v_cache,
                  (const uint8_t*)k_sf, (const uint8_t*)v_sf, out, num_items, num_pages,
                  num_kv_heads, page_size, chunk_len, max_chunks};
  const dim3 grid((uint32_t)((num_items + 7) / 8));
  if (ahead == 1)
    hipLaunchKernelGGL(decode_traffic<1>, grid, dim3(512), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(decode_traffic<2>, grid, dim3(512), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Runs blocks x 512 threads, each wave issuing iters x 8 MFMAs (32,768 flops
// each) on `stream`; out needs blocks x 512 floats.  Returns 0, or -1 on a
// bad argument or launch error.
extern "C" int nvfp4kv_mfma_peak_probe(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_loop<false>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The same loop with random operand bits (see mfma_loop).
extern "C" int nvfp4kv_mfma_random_peak_probe(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_loop<true>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" double nvfp4kv_mfma_peak_probe_flops(int blocks, int iters) {
  return (double)blocks * 8 /* waves */ * iters * kAcc * 32768.0;
}
