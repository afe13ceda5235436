// prefill.hip -- batched causal prefill attention over the NVFP4 paged KV
// cache (gfx950, wave64, f16 MFMA).
//
// Design points taken from the pages, re-made for CDNA4:
//  * FlashInfer PR #4769 page (NVFP4 KV tile repack; code analysis and "why"
//    sections): decoding NVFP4 inside the matrix-multiply loop made the
//    kernel instruction-bound; each KV tile is instead dequantized ONCE into a
//    16-bit staging tile that the matrix cores then read natively.  Here: the
//    whole workgroup decodes the tile into LDS as f16 (E2M1 x E4M3 is exact
//    in f16, and the packed f16 multiply makes the decode one instruction
//    per element), K and V both staged [key][d]; K feeds
//    v_mfma_f32_32x32x16_f16 with 16-byte LDS reads, V with gfx950 LDS
//    transpose reads.  Q enters as f16 after an exact per-row power-of-two
//    rescale, P as f16 (11 significant bits).  The raw NVFP4
//    bytes of the next tile are loaded into registers while the current tile
//    is computed.  The global scales are not applied in the staging tile: g_k
//    folds into the softmax scale and g_v into the epilogue.
//  * FlashInfer PR #3575 page (FP8 causal attention): section 1, O(1) tile
//    decode when every request has the same query length (uniform flag from
//    the plan); section 2, the heaviest causal Q tiles of all requests and
//    heads are issued first; section 3, that global order only when the KV
//    working set fits in L2 (here the sum of the 8 XCD L2s; tiles of one
//    (request, KV head) stream stay on one XCD).  Ragged batches use a work
//    list sorted by tile cost on the device.
//
// Tile = 128 query rows: block_q = 128/G consecutive tokens x the G query
// heads sharing one KV head (GQA packing).  4 waves x 32 rows.  KV tile = 64
// keys.  The score tile is computed transposed, S^T = K Q^T, so every lane
// owns one query row (lane % 32) and its softmax state stays in registers;
// O^T = V^T P^T then keeps the same row per lane, and P^T comes straight out
// of the S^T accumulators without any data movement.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

#ifndef NVFP4KV_PREFILL_SHARD
#define NVFP4KV_PREFILL_SHARD 0
#endif

namespace nvfp4kv {

// Arguments of one prefill launch (the kernels' only parameter).
struct PrefillArgs;

// The kernel templates below are compiled in three translation units (this
// file built once per shard, the shards in parallel): shard k instantiates
// the kernels prefill_shard_of assigns it and exports
// launch_prefill_shard<k>, which launches the kernel of a shape if it holds
// it; shard 0 also holds the work-list kernel, the C entry points and the
// no-allocation scratch array.
constexpr int prefill_shard_of(int head_dim, bool paired) { return head_dim == 64 ? 2 : paired ? 1 : 0; }
bool launch_prefill_shard0(const PrefillArgs& a, int D, int G, int W, int dq, bool paired, hipStream_t s);
bool launch_prefill_shard1(const PrefillArgs& a, int D, int G, int W, int dq, bool paired, hipStream_t s);
bool launch_prefill_shard2(const PrefillArgs& a, int D, int G, int W, int dq, bool paired, hipStream_t s);

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* qo;
  const int32_t* kvp;
  const int32_t* pt;
  const int32_t* kvl;
  const uint8_t* kc;
  const uint8_t* vc;
  const uint8_t* ksf;
  const uint8_t* vsf;
  const float* kscale;
  const float* vscale;
  uint16_t* out;
  const int4* worklist;  // ragged or split batches; null for the uniform O(1) decode
  int* counters;         // split tiles: [arrivals, partials written] per split tile
  float* partials;       // split tiles: max_chunks partial results each
  int64_t partial_floats;  // floats of one partial (rows x D for O, then m and l)
  int max_chunks;
  uint32_t* err;
  int64_t num_pages;
  FastDiv ps_div;
  int Hq, Hk;
  float sm_scale_log2;  // sm_scale * log2(e)
  int B, QT, order, nxcd;  // order: kOrderHeaviest, kOrderStream or kOrderRequest
  int snake;  // every tile is resident at once: pair heavy with light tiles
  uint32_t num_tiles, num_items;
};

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


template <int D, int G, int W>
struct Cfg {
  static constexpr int NT = 64 * W;         // threads (W waves of 32 rows each)
  static constexpr int BQ = 32 * W / G;     // query tokens per tile
  static constexpr int BN = kBlockN;        // keys per KV tile
  // Staged rows are padded so that the column-wise MFMA operand reads of 16
  // lanes hit distinct LDS banks: +16 bytes for K (16-byte reads of 16
  // consecutive keys), +32 bytes for V (transpose reads: 4 keys x 32 bytes).
  static constexpr int KROW = D * 2 + 16;
  static constexpr int VROW = D * 2 + 32;
  static constexpr int K_STAGE = BN * KROW;
  // Raw K row of the in-loop decode ablation: 64 code bytes + 8 scale bytes
  // (4-byte code reads of 32 keys x 2 halves hit 64 distinct banks)
  static constexpr int KRAW = 72;
  static constexpr int V_STAGE = BN * VROW;
  static constexpr int NDC = D / 16;        // MFMA k-steps over head_dim
  static constexpr int NDB = D / 32;        // 32-wide head_dim blocks of O^T
  static constexpr int PARTS = D / 32;      // 32-element dequant jobs per key row
  static constexpr int JOBS_PER_THREAD = 2 * BN * PARTS / NT;  // K and V
  // VALU instructions of a tile's staging and prefetch (about 70 per job plus
  // addressing), spread over the 2 * NDC MFMAs of S^T = K Q^T
  static constexpr int STAGE_VALU_PER_MFMA = (JOBS_PER_THREAD * 70 + 24 + 2 * NDC - 1) / (2 * NDC);
};

// Online-softmax reference max slack (log2 domain): probabilities are formed
// against a max that may lag the true running max by up to this much.
constexpr float kRescaleSlack = 8.0f;

// Scores are formed in two ways.  Normally p = exp2(fma(s, c, -m)) with the
// reference m in log2 units (s the raw matrix-core score, c the row's score
// scale): m's rounding error is a factor common to every p of the row and
// cancels.  When |s c| can reach 2^24 (a row of enormous queries), half an
// ulp of m is no longer small and exp2 would overflow; such rows use the
// exact form p = exp2((s - m) c) with m in raw score units.  A row may take
// the exact form when c times the largest possible raw score (head_dim x
// 2^15 x the largest key: a query rescaled below 2^15 times 6 x 448 staged,
// or at most 6 x 512 requantized to MXFP4 or MXFP8) reaches 2^24.
template <int D, int DQ>
__device__ __forceinline__ bool exact_scores(float c) {
  constexpr float kMaxRaw = (float)D * 32768.0f * (DQ >= 4 ? 3072.0f : 2688.0f);
  return c * kMaxRaw >= 16777216.0f;
}

// Two E2M1 codes (byte SEL of x) times one E4M3 block scale, as an f16 pair:
// the products (at most 5 significant bits, magnitudes 2^-10 .. 2688) are
// exact in f16, so the packed f16 multiply rounds nothing.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_times(uint32_t x, f16x2 S) {
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, c * S);
}

// Device-coherent access to the split-tile partials: raw buffer loads and
// stores with the device-scope cache policy (sc1), the policy of relaxed
// device-scope atomic loads and stores.  Each XCD's L2 is its own cache, so a
// partial written on one XCD is read on another through this policy.
// Offsets are bytes from the resource base; the resource range bounds them.
constexpr int kDeviceScopePolicy = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDeviceScopePolicy);
}
__device__ __forceinline__ void coherent_store1(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kDeviceScopePolicy);
}
__device__ __forceinline__ f32x4 coherent_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScopePolicy));
}
__device__ __forceinline__ float coherent_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kDeviceScopePolicy));
}

// max(x, x of lane l ^ 32) in every lane: one v_permlane32_swap exchanges
// the wave's halves in registers (no LDS round trip).  The swap is given
// two registers that hold x: its results are x and the other half's x.  The
// second copy goes through an empty asm so that the optimizer cannot see the
// two operands are the same value (it then takes the swap's two results for
// equal and drops the max).
__device__ __forceinline__ float half_max(float x) {
  uint32_t y = f2u(x);
  asm volatile("" : "+v"(y));
  const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), y, false, false);
  return __builtin_fmaxf(u2f(r[0]), u2f(r[1]));
}

// Instruction classes of the scheduling-group hints.
constexpr int kSchedValu = 0x2 | 0x400;  // VALU and transcendental
constexpr int kSchedMfma = 0x8;
constexpr int kSchedDsRead = 0x100;

constexpr f16x2 kOnesF16x2 = {(_Float16)1.0f, (_Float16)1.0f};
constexpr bf16x2 kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Dequantization kinds (the dequant-placement ablation; 0 is the kernel's own):
//  0: each KV tile decoded once per workgroup into the f16 staging tile, with
//     the hardware FP4 conversion;
//  1: K codes and scales staged raw, each wave decoding its K fragments in
//     registers inside the matrix loop (the page's "before" design); V as 0;
//  2: as 0, with a byte-table decode of the codes instead of the hardware
//     conversion;
//  3: as 0, with a bf16 staging tile, bf16 queries and probabilities and the
//     bf16 matrix instructions (the kernel's own 16-bit format is f16);
//  4: native low-precision scores in the OCP MX formats that gfx950's scaled
//     matrix instruction consumes: K requantized from NVFP4 (E4M3 scale per
//     16) to MXFP4 (E8M0 scale per 32) while it is staged, the queries in
//     MXFP8, S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4; V, P and O^T
//     as in 0.  Both requantizations round, so this mode is held to a looser
//     accuracy contract than the others;
//  5: as 4 with K requantized to MXFP8 (E4M3 elements) instead: twice the
//     staged K bytes of 4, the same instruction rate (the FP8 queries set
//     it), a much smaller requantization error.
// The 16-bit operands travel as raw bits in f16x8 registers either way.
// Eight codes (one dword) times the f16 scale pair SS, as four f16 pairs.
// The 32x32x16 matrix instruction on 16-bit operands: f16, or bf16 for the
// bf16 ablation (DQ 3).
template <int DQ>
__device__ __forceinline__ f32x16 mma16(f16x8 a, f16x8 b, f32x16 c) {
  if constexpr (DQ == 3)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// lo, hi exactly representable in bf16: keep their upper halves
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
}
// 8 codes (one dword) times their block scale S as bf16 pairs: each code
// pair to f32, one f32 multiply per element (exact), the upper halves kept.
__device__ __forceinline__ u32x4 decode8_bf16(uint32_t x, float S) {
  u32x4 r;
  static_for<0, 4>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, j);
    r[j] = bf16_pair(f[0] * S, f[1] * S);
  });
  return r;
}
template <int DQ>
__device__ __forceinline__ u32x4 decode8(uint32_t x, f16x2 SS) {
  if constexpr (DQ == 3) {
    return decode8_bf16(x, (float)SS[0]);
  } else if constexpr (DQ != 2) {
    return (u32x4){fp4x2_times<0>(x, SS), fp4x2_times<1>(x, SS), fp4x2_times<2>(x, SS),
                   fp4x2_times<3>(x, SS)};
  } else {
    // high bytes of the f16 of the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
    // (their low bytes are 0): byte k of (kLutHi:kLutLo), chosen by v_perm
    constexpr uint32_t kLutLo = 0x3E3C3800u, kLutHi = 0x46444240u;
    const uint32_t ev = x & 0x07070707u, od = (x >> 4) & 0x07070707u;  // even / odd element codes
    const uint32_t hev = __builtin_amdgcn_perm(kLutHi, kLutLo, ev) | ((x & 0x08080808u) << 4);
    const uint32_t hod = __builtin_amdgcn_perm(kLutHi, kLutLo, od) | (x & 0x80808080u);
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // element pair j: f16 (hev byte j) << 8 and (hod byte j) << 8
      const uint32_t pair = __builtin_amdgcn_perm(hod, hev, 0x000C000Cu | (uint32_t)j << 8 | (uint32_t)(4 + j) << 24);
      r[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, pair) * SS);
    }
    return r;
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// ---- dequant modes 4 and 5 (MX scores).  Operand layout of the scaled
// 32x32x64 product (pinned on the device by the probe tests): an FP4 A lane
// (row m = lane % 32, half h = lane / 32) holds two 16-element chunks of its
// row, at contraction offsets 16h and 32 + 16h; an FP8 A lane, and every B
// lane (column n, half h), holds the 32 consecutive contraction elements at
// 32h.  The scales do not follow the FP8 layout: for either format the
// product of contraction element k takes the E8M0 byte of A lane (m, g) and
// of B lane (n, g), g = (k / 16) % 2.  So both operands' MX blocks are the
// 16-element chunks {g, g + 2} of a K-step: for K-step c (head_dim 64c ..
// 64c + 63) the NVFP4 blocks 4c + g and 4c + 2 + g, MX block (c, g).  A
// staged K row holds the requantized elements (FP4: for every (c, g) the
// pair's 16 code bytes at 32c + 16g; FP8: element d at byte d; block b at
// code_off(b) either way), then the E8M0 byte of (c, g) at CODES + 4g + c.
template <int D, int DQ>
struct Mx {
  static constexpr bool FP8 = DQ == 5;
  static constexpr int CODES = FP8 ? D : D / 2;  // element bytes of a staged K row
  static constexpr int KROW = CODES + 16;        // 16-byte aligned rows
  static constexpr int FRAG = FP8 ? 32 : 16;     // A-operand bytes of one lane and K-step
  __device__ static constexpr int code_off(int b) {
    return FP8 ? 16 * b : 32 * (b / 4) + 16 * (b % 2) + 8 * ((b / 2) % 2);
  }
};

// The E8M0 exponent of an MX block whose NVFP4 block scales are at most smax
// (> 0, an E4M3 value, so a normal float): the smallest e with smax <= 2^e,
// so that every requantized magnitude e2m1 x S_b / 2^e stays within E2M1's
// range.
__device__ __forceinline__ int mx_exponent_of_scale(float smax) {
  const uint32_t b = f2u(smax);
  return (int)(b >> 23) - 127 + ((b & 0x7FFFFFu) != 0u);
}

// The same for MXFP8 elements: the smallest e with 6 smax <= 448 x 2^e (6 smax
// is exact in f32; 448 = 1.75 x 2^8).
__device__ __forceinline__ int mx8_exponent_of_scale(float smax) {
  const uint32_t b = f2u(6.0f * smax);
  return (int)(b >> 23) - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u);
}

// MXFP8 query fragments: lane (row, half hh) holds for K-step c the 32
// elements q[64c + 32hh .. +31] as E4M3 bytes (q8[c], 8 dwords): 16-element
// chunks 2hh (MX block g = 0) and 2hh + 1 (g = 1) of the K-step.  The row is
// first rescaled by 2^-sh exactly as the f16 path does (largest magnitude to
// [2^14, 2^15)), so raw scores keep the same bound; then each MX block (the
// chunks {g, g + 2}: half in each lane of the pair) takes the smallest E8M0
// exponent e >= -127 with its largest magnitude a <= 448 x 2^e (nothing
// saturates), and its elements are rounded to nearest-even E4M3 after the
// exact multiplication by 2^-e.  Byte c of the returned word is e + 127 of
// block (c, hh), the one this lane's scale operand carries; sh goes into
// *cmul as 2^sh.
// (DQ and TAG only give each kernel its own instance: the host pass of this
// compiler rejects a second kernel's call to a shared instance of this
// function)
template <int DQ, int TAG, int NC>
__device__ __forceinline__ uint32_t load_q_mx(const uint16_t* qrow, int hh, i32x8 (&q8)[NC], float& cmul) {
  u32x4 qw[NC][4];
  uint32_t bm[NC][2];  // largest |bf16| bit pattern of each MX block (t: chunk 2hh + t, block t)
  uint32_t am = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bm[c][t] = 0;
#pragma unroll
      for (int k = 2 * t; k < 2 * t + 2; ++k) {
        qw[c][k] = *(const u32x4*)(qrow + 64 * c + 32 * hh + 8 * k);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bm[c][t] = max(bm[c][t], max(qw[c][k][e] & 0x7FFFu, (qw[c][k][e] >> 16) & 0x7FFFu));
      }
      // the block's other chunk is in the partner lane (other half)
      bm[c][t] = max(bm[c][t], (uint32_t)__shfl_xor((int)bm[c][t], 32));
      am = max(am, bm[c][t]);
    }
  }
  const int sh = am >= 0x80u ? min(max((int)(am >> 7) - 127 - 14, -100), 113) : 0;
  const float down = u2f((uint32_t)(127 - sh) << 23);  // 2^-sh
  cmul = u2f((uint32_t)(127 + sh) << 23);
  uint32_t scales = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // the block's largest magnitude after the row rescale (exact: 8 significant bits)
      const uint32_t ab = f2u(u2f(bm[c][t] << 16) * down);
      const int E = (int)(ab >> 23) - 127;
      // 448 = 1.75 x 2^8: a <= 448 x 2^e  <=>  e >= E - 8 (+1 when a's significand exceeds 1.75)
      const int e = ab < 0x00800000u ? -127 : max(E - 8 + ((ab & 0x7FFFFFu) > 0x600000u), -127);
      if (t == hh) scales |= (uint32_t)(e + 127) << (8 * c);
      // q x 2^-(sh + e) in two exact power-of-two steps (sh + e spans
      // [-227, 120], beyond one float factor; a product that underflows in
      // the first step is far below E4M3's smallest subnormal either way)
      const int x = sh + e, x1 = x / 2;
      const float f1 = u2f((uint32_t)(127 - x1) << 23), f2 = u2f((uint32_t)(127 - (x - x1)) << 23);
      auto y = [&](uint32_t bits) { return (u2f(bits) * f1) * f2; };
#pragma unroll
      for (int k = 2 * t; k < 2 * t + 2; ++k)
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
          const uint32_t w0 = qw[c][k][2 * d2], w1 = qw[c][k][2 * d2 + 1];
          s16x2 o = {};
          o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, y(w0 << 16), y(w0 & 0xFFFF0000u), 1.0f, false);
          o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, y(w1 << 16), y(w1 & 0xFFFF0000u), 1.0f, true);
          q8[c][2 * k + d2] = __builtin_bit_cast(int, o);
        }
    }
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" ::"v"(q8[c]));
  return scales;
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives elements i, 16+i, 32+i, 48+i of the 64 16-bit values
// the group's lanes address (4 consecutive values per lane, in lane order).
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// One thread's share of a KV tile: 32 consecutive head_dim elements of one
// key (16 packed bytes + 2 scale bytes) for K and for V.
template <int D>
struct RawJob {
  u32x4 pk;
  // the key's whole scale row (D/16 bytes, naturally aligned); a full-width
  // load needs no zero-extension copy across the loop back-edge
  typename std::conditional<D == 128, uint2, uint32_t>::type sfrow;
};

// The dword of a key's scale row holding the two scale bytes of job part
// `part` (in its low half for even parts, its high half for odd ones).
template <int D>
__device__ __forceinline__ uint32_t scale_word(const RawJob<D>& j, int part) {
  if constexpr (D == 128) return part < 2 ? j.sfrow.x : j.sfrow.y;
  else return j.sfrow;
}

// Every job of a thread covers the same key, so one page-table lookup per
// thread and KV tile serves the K and the V job.
template <int D, int G, int W>
__device__ __forceinline__ int job_key(int tid) {
  using C = Cfg<D, G, W>;
  static_assert(C::NT % (C::BN * C::PARTS) == 0, "jobs of a thread must share their key");
  return (tid % (C::BN * C::PARTS)) / C::PARTS;
}

// Loads below are unconditional, from always-valid addresses (keys are
// clamped to the last key any row sees; ids outside the pool read page 0),
// and what is loaded is only inspected one step later: no branch or select
// forces a wait on a load that is meant to stay in flight during a tile.
//
// Where this thread's key of KV tile jt lives.  With PA (the page size
// divides the 64-key tile, so it is a power of two up to 64) the key keeps
// its page slot and in-page row in every tile: the tile's page is entry
// jt * (64 / ps) + key / ps of the request's page list, and each load address
// is one multiply-add from a per-job base.  Otherwise the page and the row
// in it come from a division of the key's position.
template <int D, int G, int W, bool PA>
struct KeyAddr {
  using C = Cfg<D, G, W>;
  const uint8_t* code0[C::JOBS_PER_THREAD];  // job j's codes in page 0 (PA: at this key's row)
  const uint8_t* sf0[C::JOBS_PER_THREAD];    // its scale row likewise
  const int32_t* ptb;                        // the request's page list
  uint32_t page_code_bytes, page_sf_bytes;   // one page of codes / scales (PA)
  int key, kend_max, tpg, kq, kmaxq;

  __device__ __forceinline__ KeyAddr(const PrefillArgs& a, int tid, int hk, int kend_max_,
                                     const int32_t* ptb_)
      : ptb(ptb_), kend_max(kend_max_) {
    key = job_key<D, G, W>(tid);
    const int ps = (int)a.ps_div.d;
    const int row0 = PA ? (key & (ps - 1)) * a.Hk + hk : hk;  // (token, head) row within page 0
#pragma unroll
    for (int j = 0; j < C::JOBS_PER_THREAD; ++j) {
      const int id = tid + C::NT * j;
      const int tensor = id / (C::BN * C::PARTS);  // 0: K, 1: V
      const int part = id % C::PARTS;
      code0[j] = (tensor ? a.vc : a.kc) + (int64_t)row0 * (D / 2) + part * 16;
      sf0[j] = (tensor ? a.vsf : a.ksf) + (int64_t)row0 * (D / 16);
    }
    tpg = kq = kmaxq = 0;
    page_code_bytes = page_sf_bytes = 0;
    if constexpr (PA) {
      tpg = C::BN / ps;
      kq = key / ps;
      kmaxq = kend_max / ps;
      page_code_bytes = (uint32_t)(ps * a.Hk * (D / 2));
      page_sf_bytes = (uint32_t)(ps * a.Hk * (D / 16));
    }
  }

  // raw page id of the key in KV tile jt (clamped to the last key any row sees)
  __device__ __forceinline__ int lookup(const PrefillArgs& a, int jt) const {
    if constexpr (PA) return ptb[min(jt * tpg + kq, kmaxq)];
    else return ptb[fastdiv((uint32_t)min(jt * C::BN + key, kend_max), a.ps_div)];
  }

  // Issue the loads of the thread's jobs of KV tile jt; returns whether the
  // key is live (at or before the last key any row sees, in a valid page) and
  // notes in page_bad a live key whose page id is outside the pool.
  __device__ __forceinline__ bool load(const PrefillArgs& a, RawJob<D>* job, int jt, int page,
                                       bool& page_bad) const {
    const int kk = jt * C::BN + key;
    const bool live = kk <= kend_max;  // later keys are masked for every row: zeros
    const bool in_pool = (uint32_t)page < (uint64_t)a.num_pages;
    page_bad |= live && !in_pool;  // reported once, after the KV loop
    const uint32_t pg = in_pool ? (uint32_t)page : 0u;
#pragma unroll
    for (int j = 0; j < C::JOBS_PER_THREAD; ++j) {
      if constexpr (PA) {
        job[j].pk = *(const u32x4*)(code0[j] + (uint64_t)pg * page_code_bytes);
        job[j].sfrow = *(const decltype(job[j].sfrow)*)(sf0[j] + (uint64_t)pg * page_sf_bytes);
      } else {
        const int ps = (int)a.ps_div.d;
        const int64_t rows = ((int64_t)pg * ps + (kk - (int)fastdiv((uint32_t)kk, a.ps_div) * ps)) * a.Hk;
        job[j].pk = *(const u32x4*)(code0[j] + rows * (D / 2));
        job[j].sfrow = *(const decltype(job[j].sfrow)*)(sf0[j] + rows * (D / 16));
      }
    }
    return live && in_pool;
  }
};

// Pin the first use of the prefetched registers at the point of the call
// (right after a barrier): otherwise the compiler hoists their unpacking into
// the previous tile's matrix phase and waits for the loads there.  The pin is
// an ordering point for memory operations, so it goes before the tile's LDS
// reads, not between them and the dequantization.
template <int D, int G, int W>
__device__ __forceinline__ void pin_jobs(RawJob<D>* job) {
#pragma unroll
  for (int j = 0; j < Cfg<D, G, W>::JOBS_PER_THREAD; ++j) asm volatile("" : "+v"(job[j].pk), "+v"(job[j].sfrow));
}


// The staging of one KV tile cut into half-words: piece p of a thread
// dequantizes 8 elements (word (p/2)%4 of job p/8, its low or high half) and
// every second piece stores the finished 16-byte chunk.  The pieces are
// interleaved with the matrix instructions of the tile before.
template <int D, int G, int W, int DQ = 0>
struct TileStager {
  using C = Cfg<D, G, W>;
  static constexpr int PIECES = 8 * C::JOBS_PER_THREAD;
  uint8_t* rowp[C::JOBS_PER_THREAD];
  uint32_t S01[C::JOBS_PER_THREAD];  // the part's two E4M3 scales as an f16 pair (exact)
  f32x2 S32[C::JOBS_PER_THREAD];     // (DQ 3) the same two scales in f32, as the bf16 decode uses them
  uint32_t sw[C::JOBS_PER_THREAD];   // the part's two raw scale bytes
  uint8_t* sfp;                      // (DQ 1) where the K part's scale bytes go
  u32x4 chunk;
  uint32_t R01;                      // (DQ 4, 5) the K part's S_b / 2^e as an f16 pair (exact)
  int kpart;                         // (DQ 4, 5) the K part
  uint2 kout;                        // (DQ 4) one requantized 16-element block
  u32x4 kout8;                       // (DQ 5) one requantized 16-element block
  __device__ __forceinline__ TileStager(const RawJob<D>* job, bool live, uint8_t* smem, int tid) {
#pragma unroll
    for (int j = 0; j < C::JOBS_PER_THREAD; ++j) {
      const int id = tid + C::NT * j;
      const int tensor = id / (C::BN * C::PARTS);
      const int rem = id - tensor * C::BN * C::PARTS;
      const int key = rem / C::PARTS, part = rem % C::PARTS;
      rowp[j] = tensor ? smem + C::K_STAGE + key * C::VROW + part * 64
                       : DQ == 1 ? smem + key * C::KRAW + part * 16
                       : DQ >= 4 ? smem + key * Mx<D, DQ>::KROW
                                 : smem + key * C::KROW + part * 64;
      if (j == 0) sfp = smem + key * C::KRAW + 64 + 2 * part;
      // both E4M3 scales of the part in one conversion (dead keys: zero scales)
      sw[j] = live ? (scale_word<D>(job[j], part) >> (16 * (part & 1))) & 0xFFFFu : 0u;
      const f32x2 S = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[j], 1.0f, false);
      S32[j] = S;
      if constexpr (DQ != 3) {
        const f16x2 Sh = {(_Float16)S[0], (_Float16)S[1]};
        S01[j] = __builtin_bit_cast(uint32_t, Sh);
      }
      if constexpr (DQ >= 4) {
        if (j == 0) {
          // The part's blocks 2p + k (k = 0, 1) pair with blocks 2(p^1) + k
          // of the neighbouring part into MX blocks (p/2, k); both parts
          // compute the pair's exponent, the even one stores it.
          kpart = part;
          const uint32_t pw = live ? (scale_word<D>(job[0], part ^ 1) >> (16 * ((part ^ 1) & 1))) & 0xFFFFu : 0u;
          const f32x2 Sp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pw, 1.0f, false);
          uint32_t xb = 0;
          f16x2 R;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float smax = __builtin_fmaxf(S[k], Sp[k]);
            const int e = smax > 0.0f ? (Mx<D, DQ>::FP8 ? mx8_exponent_of_scale(smax) : mx_exponent_of_scale(smax)) : 0;
            // S_b / 2^e, 4 significant bits: FP4 in (0, 1] and at least
            // 2^-18, FP8 in (0, 75) and at least 2^-12: exact in f16
            R[k] = (_Float16)(S[k] * u2f((uint32_t)(127 - e) << 23));
            xb |= (smax > 0.0f ? (uint32_t)(e + 127) : 0u) << (8 * k);
          }
          R01 = __builtin_bit_cast(uint32_t, R);
          if ((part & 1) == 0) {
            rowp[0][Mx<D, DQ>::CODES + part / 2] = (uint8_t)(xb & 0xFFu);
            rowp[0][Mx<D, DQ>::CODES + 4 + part / 2] = (uint8_t)(xb >> 8);
          }
        }
      }
    }
  }
  template <int P>
  __device__ __forceinline__ void piece(const RawJob<D>* job) {
    constexpr int j = P / 8, w = (P / 2) % 4, h = P % 2;
    if constexpr (DQ == 4 && j == 0) {
      // requantize 4 codes of block 2p + w/2: e2m1(code) x S_b / 2^e (an
      // exact f16 product, magnitude <= 6), rounded to nearest-even E2M1
      static_assert(C::JOBS_PER_THREAD == 2, "MX scores: 4-wave tiles");
      const _Float16 r = __builtin_bit_cast(f16x2, R01)[w / 2];
      const f16x2 rr = {r, r};
      const uint32_t x = job[0].pk[w];
      uint32_t& out = w % 2 ? kout.y : kout.x;
      if constexpr (h == 0) out = 0;
      static_for<2 * h, 2 * h + 2>([&](auto bc) {
        constexpr int sel = decltype(bc)::value;  // byte of the code word: elements 2 sel, 2 sel + 1
        const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, sel) * rr;
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(out, v, 1.0f, sel);
      });
      // the block's 8 code bytes (words 2k, 2k + 1 of the part) to their place
      if constexpr (w % 2 == 1 && h == 1) *(uint2*)(rowp[0] + Mx<D, DQ>::code_off(2 * kpart + w / 2)) = kout;
    } else if constexpr (DQ == 5 && j == 0) {
      // requantize 4 codes of block 2p + w/2: e2m1(code) x S_b / 2^e (an
      // exact f16 product, magnitude <= 448), rounded to nearest-even E4M3,
      // one byte per element in head_dim order
      static_assert(C::JOBS_PER_THREAD == 2, "MX scores: 4-wave tiles");
      const _Float16 r = __builtin_bit_cast(f16x2, R01)[w / 2];
      const f16x2 rr = {r, r};
      const uint32_t x = job[0].pk[w];
      s16x2 o = {};
      o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(o, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2 * h) * rr,
                                                   1.0f, false);
      o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(o, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2 * h + 1) * rr,
                                                   1.0f, true);
      kout8[2 * (w % 2) + h] = __builtin_bit_cast(uint32_t, o);
      // the block's 16 element bytes (words 2k, 2k + 1 of the part) to their place
      if constexpr (w % 2 == 1 && h == 1) *(u32x4*)(rowp[0] + Mx<D, DQ>::code_off(2 * kpart + w / 2)) = kout8;
    } else if constexpr (DQ == 1 && j == 0) {
      // raw K: the part's 16 code bytes and its 2 scale bytes (job 0 is K
      // for 4-wave tiles, the only ones the ablation is built for)
      static_assert(C::JOBS_PER_THREAD == 2, "in-loop decode ablation: 4-wave tiles");
      if constexpr (P == 7) {
        *(u32x4*)rowp[0] = job[0].pk;
        *(uint16_t*)sfp = (uint16_t)sw[0];
      }
    } else if constexpr (DQ == 3) {
      // bf16: the f32 scale straight into the f32 products
      if constexpr (h == 1) *(u32x4*)(rowp[j] + w * 16) = decode8_bf16(job[j].pk[w], S32[j][w < 2 ? 0 : 1]);
    } else {
      const _Float16 S = __builtin_bit_cast(f16x2, S01[j])[w < 2 ? 0 : 1];
      const f16x2 SS = {S, S};
      const uint32_t x = job[j].pk[w];
      if constexpr (DQ == 2) {
        if constexpr (h == 1) *(u32x4*)(rowp[j] + w * 16) = decode8<DQ>(x, SS);
      } else {
        chunk[2 * h] = fp4x2_times<2 * h>(x, SS);
        chunk[2 * h + 1] = fp4x2_times<2 * h + 1>(x, SS);
        if constexpr (h == 1) *(u32x4*)(rowp[j] + w * 16) = chunk;
      }
    }
  }
};

// The stand-in of a wave that stages nothing (the heavy half of a pair):
// no state, no loads, no LDS writes.
struct NoStager {
  template <class J>
  __device__ __forceinline__ NoStager(const J*, bool, uint8_t*, int) {}
  template <int P, class J>
  __device__ __forceinline__ void piece(const J*) {}
};
template <bool STAGE, int D, int G, int W, int DQ>
struct StagerOf {
  using type = typename std::conditional<STAGE, TileStager<D, G, W, DQ>, NoStager>::type;
};

// The work item of workgroup `tile`: request b, KV head hk, Q tile qt, and
// the KV tile range [jt_begin, jt_end) (the whole range unless the item is
// one chunk of a split Q tile; split: -1, or (split id << 10) | (chunk << 5)
// | chunks).
struct Item {
  int b, hk, qt, jt_begin, jt_end, split;
};

// Paired order: work item `tile` is the pair pp of (request, KV head) bh --
// its Q tile pp (the light one) and QT - 1 - pp (the heavy one), which see
// about the same number of KV tiles together whatever pp is.  The light
// tile's waves also stage every KV tile the heavy one visits.  The middle
// tile of an odd count has no partner: its light half holds no rows (qt =
// QT).  Returns this half's item; `qt_heavy` is the tile whose keys the
// staging covers.
__device__ __forceinline__ Item decode_pair(const PrefillArgs& a, uint32_t tile, bool heavy, int& qt_heavy) {
  Item it;
  it.jt_begin = 0;
  it.jt_end = 0x7FFFFFFF;
  it.split = -1;
  const uint32_t bh_n = (uint32_t)a.B * a.Hk;
  const uint32_t pp = tile / bh_n, bh = tile - pp * bh_n;
  it.b = bh / a.Hk;
  it.hk = bh - it.b * a.Hk;
  qt_heavy = a.QT - 1 - (int)pp;
  it.qt = heavy ? qt_heavy : ((int)pp < qt_heavy ? (int)pp : a.QT);
  return it;
}
__device__ __forceinline__ Item decode_item(const PrefillArgs& a, uint32_t tile) {
  Item it;
  it.jt_begin = 0;
  it.jt_end = 0x7FFFFFFF;
  it.split = -1;
  if (a.worklist) {
    const int4 e = a.worklist[tile];
    it.b = e.x;
    it.qt = e.y / a.Hk;
    it.hk = e.y - it.qt * a.Hk;
    it.jt_begin = (uint32_t)e.z >> 16;
    it.jt_end = e.z & 0xFFFF;
    it.split = e.w;
    return it;
  }
  const uint32_t bh_n = (uint32_t)a.B * a.Hk;
  uint32_t bh, qrev;
  if (a.order == kOrderHeaviest) {
    // heaviest Q tiles of every (request, head) first
    qrev = tile / bh_n;
    bh = tile - qrev * bh_n;
    // When the whole grid is resident at once, workgroup p and p + grid/2
    // share a CU: the second half walks the remaining tiles lightest first
    // so that every CU gets one heavy and one light tile.
    const uint32_t half = (a.QT + 1) / 2;
    if (a.snake && qrev >= half) qrev = a.QT - 1 - (qrev - half);
  } else if (a.order == kOrderStream) {
    // stream-major: XCD x (blockIdx % nxcd) owns a contiguous range of
    // (request, head) streams, each walked heaviest tile first
    const uint32_t nx = a.nxcd, x = tile % nx, s = tile / nx;
    const uint32_t per = a.num_tiles / nx, rem = a.num_tiles % nx;
    const uint32_t L = x * per + (x < rem ? x : rem) + s;
    bh = L / a.QT;
    qrev = L - bh * a.QT;
  } else {
    // request order: (request, head) streams in order, each one's Q tiles
    // lightest first -- no reordering at all
    bh = tile / a.QT;
    qrev = a.QT - 1 - (tile - bh * a.QT);
  }
  it.b = bh / a.Hk;
  it.hk = bh - it.b * a.Hk;
  it.qt = a.QT - 1 - qrev;
  return it;
}

// Q^T operand fragments of one query row (the lane's row; hh selects the
// half of each 16-element k-step): lane holds Q[row][16c + 8hh .. +7], in f16
// after an exact power-of-two rescale of the row: bf16 values have 8
// significant bits, and the row's largest magnitude goes to [2^14, 2^15), so
// every value within 2^-28 of it stays a normal f16.  The row's scale comes
// back in its score scale, returned (scores -> log2 domain).  DQ 3: the same
// rescale, the fragments in bf16 (exact; raw scores keep the same bound).
template <int D, int DQ>
__device__ __forceinline__ float load_q(const uint16_t* qrow, int hh, float score_scale, f16x8 (&qf)[D / 16]) {
  constexpr int NDC = D / 16;
  u32x4 qw[NDC];
  uint32_t am = 0;  // largest |bf16| bit pattern of the row
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qw[c] = *(const u32x4*)(qrow + c * 16 + hh * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) am = max(am, max(qw[c][e] & 0x7FFFu, (qw[c][e] >> 16) & 0x7FFFu));
  }
  am = max(am, (uint32_t)__shfl_xor((int)am, 32));  // the row's other half
  const int sh = am >= 0x80u ? min(max((int)(am >> 7) - 127 - 14, -100), 113) : 0;
  const float down = u2f((uint32_t)(127 - sh) << 23);  // 2^-sh
#pragma unroll
  for (int c = 0; c < NDC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = u2f(qw[c][e] << 16) * down, hi = u2f(qw[c][e] & 0xFFFF0000u) * down;
      if constexpr (DQ == 3) {  // bf16 matrix instructions: the same rescale, exact in bf16 (RNE below its normals)
        const bf16x2 h = {(__bf16)lo, (__bf16)hi};
        qw[c][e] = __builtin_bit_cast(uint32_t, h);
      } else {
        const f16x2 h = {(_Float16)lo, (_Float16)hi};
        qw[c][e] = __builtin_bit_cast(uint32_t, h);
      }
    }
#pragma unroll
  for (int c = 0; c < NDC; ++c) __builtin_memcpy(&qf[c], &qw[c], 16);
  // Consume the Q fragments here, so their load waits are placed before the
  // KV loop rather than inside it (where they would also wait for the
  // prefetch of the next tile).
#pragma unroll
  for (int c = 0; c < NDC; ++c) asm volatile("" ::"v"(qf[c]));
  return score_scale * u2f((uint32_t)(127 + sh) << 23);
}

// ---- split Q tile: all but the last chunk to arrive publish a partial
// (unnormalized O^T, reference max, sum); the last one merges them all in
// chunk order (symmetric: the result does not depend on arrival order).
// The partials move through device-coherent loads and stores and the
// counters through relaxed device-scope atomics: no cache-wide write-back
// or invalidate, which would evict the KV tiles other work-groups on the
// same L2 are reading.  Every thread of the workgroup calls this (it has
// barriers); `active` threads (the ones holding the tile's O^T; ltid in
// [0, 2 ROWS) their index in the partial's layout, 64 per 32-row block)
// move data.  Returns false when this workgroup published its partial and
// is done.
template <int D, int ROWS>
__device__ __forceinline__ bool split_merge(const PrefillArgs& a, int split, int tid, int ltid, bool active,
                                            int r, bool exact, float cscale, float& m_run, float& l_tot,
                                            f32x16 (&o)[D / 32]) {
  constexpr int NDB = D / 32, NT = 2 * ROWS;
  const int sid = split >> 10, chunk = (split >> 5) & 31, nch = split & 31;
  int* arrive = a.counters + 2 * sid;
  __shared__ int s_prior;
  if (tid == 0) s_prior = __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int prior = s_prior;
  const __amdgpu_buffer_rsrc_t parts = coherent_rsrc(
      a.partials + (int64_t)sid * a.max_chunks * a.partial_floats,
      (uint32_t)(a.max_chunks * a.partial_floats * 4));
  const int ml_base = ROWS * D;  // floats: O^T, then m per row, then l per row
  const int hh = (ltid >> 5) & 1;
  if (prior < nch - 1) {
    if (active) {
      const int cb = chunk * (int)a.partial_floats * 4;  // byte offset of this chunk
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          coherent_store4(parts, cb + ((db * 4 + i4) * NT + ltid) * 16,
                          (f32x4){o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]});
      if (hh == 0) {
        coherent_store1(parts, cb + (ml_base + r) * 4, m_run);
        coherent_store1(parts, cb + (ml_base + ROWS + r) * 4, l_tot);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial is written
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(arrive + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  // last to arrive: the other chunks have all arrived and are finishing
  // their partials; wait (bounded) until all of them are published
  if (tid == 0) {
    int spins = 0;
    while (__hip_atomic_load(arrive + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nch - 1) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == (1 << 22)) {
        atomicOr(a.err, (uint32_t)NVFP4KV_DEV_SPLIT_TIMEOUT);
        break;
      }
    }
  }
  __syncthreads();
  if (!active) return true;
  float m_all = m_run;
  for (int c = 0; c < nch; ++c)
    if (c != chunk)
      m_all = __builtin_fmaxf(m_all, coherent_load1(parts, (c * (int)a.partial_floats + ml_base + r) * 4));
  const float m_ref = m_all == -__builtin_inff() ? 0.0f : m_all;
  f32x16 acc[NDB];
  float l_acc = 0.0f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
  // Identical arithmetic for the chunk held in registers and the chunks
  // read back (explicit FMAs), so the bits do not depend on which chunk
  // arrived last.
  for (int c = 0; c < nch; ++c) {
    const int cb = c * (int)a.partial_floats * 4;
    const bool mine = c == chunk;
    const float mc = mine ? m_run : coherent_load1(parts, cb + (ml_base + r) * 4);
    const float lc = mine ? l_tot : coherent_load1(parts, cb + (ml_base + ROWS + r) * 4);
    const float f = __builtin_amdgcn_exp2f(exact ? (mc - m_ref) * cscale : mc - m_ref);
    l_acc = __builtin_fmaf(lc, f, l_acc);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v = {o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]};
        if (!mine) v = coherent_load4(parts, cb + ((db * 4 + i4) * NT + ltid) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * i4 + e] = __builtin_fmaf(v[e], f, acc[db][4 * i4 + e]);
      }
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = acc[db];
  l_tot = l_acc;
  m_run = m_all;
  return true;
}

// PAIR: two W-wave tiles in one workgroup of 2W waves (the paired order):
// waves [0, W) compute the light Q tile and stage every KV tile of the pair,
// waves [W, 2W) compute the heavy one and stage nothing, so that the tile
// on the longest path runs its matrix and softmax work with the staging on
// the other waves of its SIMDs.  Every wave passes the same barriers: one
// after the prologue and one per KV tile of the heavy tile.
template <int D, int G, int W, bool PA, int DQ, bool PAIR = false>
__global__ __launch_bounds__(64 * W * (PAIR ? 2 : 1), 8 / (W * (PAIR ? 2 : 1))) void prefill_kernel(PrefillArgs a) {
  using C = Cfg<D, G, W>;
  // Two staging buffers: tile j+1 is dequantized into one while tile j is
  // read from the other, with a single barrier per KV tile.
  constexpr int STG = C::K_STAGE + C::V_STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STG];
  const int tid_all = threadIdx.x, lane = tid_all & 63;
  const bool heavy = PAIR && tid_all >= C::NT;  // (wave-uniform)
  const int tid = PAIR ? tid_all & (C::NT - 1) : tid_all;  // thread within this half
  const int wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;

  int qt_stage = 0;
  const Item it = PAIR ? decode_pair(a, blockIdx.x, heavy, qt_stage) : decode_item(a, blockIdx.x);
  const int b = it.b, hk = it.hk, qt = it.qt, jt_begin = it.jt_begin, jt_end = it.jt_end, split = it.split;
  const uint32_t tile = blockIdx.x;
  const int q_begin = a.qo[b];
  const int Lq = a.qo[b + 1] - q_begin;
  const int Lk = a.kvl[b];
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q0 = qt * C::BQ;
  const int rows_valid = min(C::BQ, Lq - q0);
  if (!PAIR && rows_valid <= 0) return;  // (uniform batches with short requests)
  const int kend_max = off + q0 + rows_valid - 1;  // last key any row sees
  const int kend_min = off + q0;                   // last key of the first row
  // this half's KV tiles: [jt_begin, ntiles) (none for a half without rows)
  const int ntiles = rows_valid > 0 ? min(kend_max / C::BN + 1, jt_end) : jt_begin;
  // the keys the staging covers: the heavy tile's when paired
  const int kend_stage = PAIR ? off + qt_stage * C::BQ + min(C::BQ, Lq - qt_stage * C::BQ) - 1 : kend_max;
  const int nstage = PAIR ? kend_stage / C::BN + 1 : ntiles;
  const int32_t* ptb = a.pt + a.kvp[b];

  // Software pipeline: data of tile jt+1 and the page id of tile jt+2 are in
  // flight while tile jt is computed.
  RawJob<D> job[C::JOBS_PER_THREAD];
  bool page_bad = false;
  const KeyAddr<D, G, W, PA> ka(a, tid, hk, kend_stage, ptb);
  bool live = false;
  int page_next = 0;
  if (!heavy) {
    live = ka.load(a, job, jt_begin, ka.lookup(a, jt_begin), page_bad);
    page_next = ka.lookup(a, jt_begin + 1);
  }

  const int r = wave * 32 + n;  // this lane's tile row
  const int tr = r % C::BQ, g = r / C::BQ;
  const bool row_valid = tr < rows_valid;
  const int tok = q0 + tr;
  const int hq = hk * G + g;
  const int kend = off + tok;

  const float gk = *a.kscale, gv = *a.vscale;
  if (tile == 0 && tid_all == 0 && !(scale_ok(gk) && scale_ok(gv)))
    atomicOr(a.err, (uint32_t)NVFP4KV_DEV_BAD_SCALE_ATTN);
  // (rows past the tile's end read the tile's first row; a paired light half
  // without rows reads the request's first)
  const uint16_t* const qrow = a.q + ((int64_t)(q_begin + (row_valid ? tok : rows_valid > 0 ? q0 : 0)) * a.Hq + hq) * D;
  f16x8 qf[C::NDC];    // 16-bit Q^T fragments (modes 0-3)
  i32x8 q8[D / 64];    // MXFP8 Q^T fragments (modes 4, 5)
  uint32_t qsc = 0;    // their E8M0 scale bytes, one per K-step
  float cscale;
  if constexpr (DQ >= 4) {
    float cmul;
    qsc = load_q_mx<DQ, PAIR ? 1 : 0>(qrow, hh, q8, cmul);
    cscale = a.sm_scale_log2 * gk * cmul;
  } else {
    cscale = load_q<D, DQ>(qrow, hh, a.sm_scale_log2 * gk, qf);
  }

  f32x16 o[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) o[i] = (f32x16){};
  // reference max: log2 units, or raw score units on a wave whose rows need
  // the exact score form (the same on every chunk of a split tile)
  float m_run = -__builtin_inff(), l_run = 0.0f;
  const bool exact = __any(exact_scores<D, DQ>(cscale));

  // V^T operand addressing (transpose reads): lane t of each 16-lane group
  // points at 4 consecutive head_dim values of one key.
  const int t16 = lane & 15, g16 = (lane >> 4) & 1;
  const int voff = C::K_STAGE + (4 * hh + (t16 >> 2)) * C::VROW + (16 * g16 + 4 * (t16 & 3)) * 2;

  // Pipeline prologue: the first tile staged (into buffer jt_begin & 1), the
  // next tile's NVFP4 bytes and the one after's page ids in flight.
  if (!heavy) {
    pin_jobs<D, G, W>(job);
    {
      TileStager<D, G, W, DQ> st(job, live, smem + (jt_begin & 1) * STG, tid);
      static_for<0, TileStager<D, G, W, DQ>::PIECES>([&](auto pc) { st.template piece<decltype(pc)::value>(job); });
    }
    live = ka.load(a, job, jt_begin + 1, page_next, page_bad);
    page_next = ka.lookup(a, jt_begin + 2);
  }
  __syncthreads();

  // One KV tile j: S^T = K Q^T from buffer j&1; dequantize tile j+1 into the
  // other buffer (VALU work that runs beside the matrix cores); prefetch tile
  // j+2; (mask), online softmax, O^T += V^T P^T; one barrier.
  auto tile_step = [&](const int jt, auto masked, auto exact_form, auto stage_form) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr bool EXACT = decltype(exact_form)::value;
    constexpr bool STAGE = decltype(stage_form)::value;  // this wave stages tile j+1
    const uint8_t* const sK = smem + (jt & 1) * STG;
    const uint8_t* const vbase = sK + voff;
    if constexpr (STAGE) pin_jobs<D, G, W>(job);

    // ---- S^T = K Q^T for 64 keys: lane holds S^T[key 32kb + 8(i/4) + 4hh + i%4][row n].
    // The 2*NDC matrix instructions alternate the two 32-key blocks (no
    // back-to-back dependence), K fragments are read KA instructions ahead,
    // and the staging of tile j+1 into the other buffer (then the loads of
    // tile j+2) is placed piece by piece between them, so that it issues
    // while the matrix core runs.  Scheduling barriers keep that order.
    f32x16 s[2];
    s[0] = s[1] = (f32x16){};
    if constexpr (DQ >= 4) {
      // MX scores: the instruction (kb, c) = (i & 1, i >> 1) multiplies the
      // MXFP4 (MXFP8) keys of block kb by the MXFP8 queries of K-step c; the
      // lane reads its 16 (32) element bytes of each (kb, c) and one word of
      // E8M0 bytes per kb (byte c: K-step c) up front.
      using X = Mx<D, DQ>;
      constexpr int NQK = D / 32;
      i32x8 kf[NQK];
      uint32_t ksc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* row = sK + (kb * 32 + n) * X::KROW;
        ksc[kb] = *(const uint32_t*)(row + X::CODES + 4 * hh);
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
          const uint8_t* f = row + 2 * X::FRAG * c + X::FRAG * hh;
          const u32x4 v = *(const u32x4*)f;
          const u32x4 v2 = X::FP8 ? *(const u32x4*)(f + 16) : (u32x4){0u, 0u, 0u, 0u};
          kf[2 * c + kb] = (i32x8){(int)v[0], (int)v[1], (int)v[2], (int)v[3], (int)v2[0], (int)v2[1], (int)v2[2], (int)v2[3]};
        }
      }
      typename StagerOf<STAGE, D, G, W, DQ>::type stager(job, live, smem + ((jt + 1) & 1) * STG, tid);
      static_for<0, NQK>([&](auto ic) {
        constexpr int i = decltype(ic)::value, kb = i & 1, c = i >> 1;
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[i], q8[c], s[kb], X::FP8 ? 0 : 4, 0, c, ksc[kb], c, qsc);
        constexpr int HP = TileStager<D, G, W, DQ>::PIECES;
        constexpr int P0 = (i * HP + NQK - 1) / NQK, P1 = ((i + 1) * HP + NQK - 1) / NQK;
        if constexpr (STAGE) static_for<P0, P1>([&](auto pc) { stager.template piece<decltype(pc)::value>(job); });
        if constexpr (STAGE && i == NQK - 1) {
          live = ka.load(a, job, jt + 2, page_next, page_bad);
          page_next = ka.lookup(a, jt + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
    constexpr int NQK = 2 * C::NDC, KA = 3;
    f16x8 kf[KA];
    auto kread = [&](int i) {
      if constexpr (DQ == 1) {
        // decode in registers: 4 code bytes (this lane's 8 elements) and the
        // block's scale byte of the raw K row
        const uint8_t* row = sK + ((i & 1) * 32 + n) * C::KRAW;
        const uint32_t x = *(const uint32_t*)(row + (i >> 1) * 8 + hh * 4);
        const uint32_t sb = row[64 + (i >> 1)];
        const _Float16 S = (_Float16)__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, false)[0];
        const f16x2 SS = {S, S};
        return __builtin_bit_cast(f16x8, decode8<1>(x, SS));
      } else {
        f16x8 v;
        __builtin_memcpy(&v, sK + ((i & 1) * 32 + n) * C::KROW + hh * 16 + (i >> 1) * 32, 16);
        return v;
      }
    };
#pragma unroll
    for (int i = 0; i < KA; ++i) kf[i] = kread(i);
    typename StagerOf<STAGE, D, G, W, DQ>::type stager(job, live, smem + ((jt + 1) & 1) * STG, tid);
    static_for<0, NQK>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      s[i & 1] = mma16<DQ>(kf[i % KA], qf[i >> 1], s[i & 1]);
      if constexpr (i + KA < NQK) kf[i % KA] = kread(i + KA);
      // staging pieces [P0, P1) in this slot
      constexpr int HP = TileStager<D, G, W, DQ>::PIECES;
      constexpr int P0 = (i * HP + NQK - 1) / NQK, P1 = ((i + 1) * HP + NQK - 1) / NQK;
      if constexpr (STAGE) static_for<P0, P1>([&](auto pc) { stager.template piece<decltype(pc)::value>(job); });
      if constexpr (STAGE && i == NQK - 1) {
        // past the last tile this stages and loads unused (clamped) data
        live = ka.load(a, job, jt + 2, page_next, page_bad);
        page_next = ka.lookup(a, jt + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    }

    // ---- causal mask (diagonal tiles only): key > kend  <=>  offset(i) > lim
    if constexpr (MASK) {
      const int lim = kend - jt * C::BN - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i / 4) + (i % 4) > lim) s[kb][i] = -__builtin_inff();
    }
    // ---- online softmax in the log2 domain (row max on raw scores, scale > 0)
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[kb][i]);
    mx = half_max(mx);
    // Lazy rescaling: the reference max moves only when the tile's max
    // exceeds it by more than kRescaleSlack (log2 units), so p stays below
    // 2^kRescaleSlack and the O^T rescale is skipped on most tiles.
    float m_new, alpha;
    bool grow;
    if constexpr (EXACT) {
      grow = (mx - m_run) * cscale > kRescaleSlack;  // (-inf) - (-inf): NaN, no growth
      m_new = grow ? mx : m_run;
      alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * cscale) : 1.0f;
    } else {
      const float m_tile = mx * cscale;
      grow = m_tile > m_run + kRescaleSlack;
      m_new = grow ? m_tile : m_run;
      alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    }
    m_run = m_new;
    l_run *= alpha;
    if (__any(grow)) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
    }
    // (a row with no visible key yet keeps -inf: its p must be 0, not NaN)
    const float m_sub = m_new == -__builtin_inff() ? 0.0f : m_new;

    // ---- P^T operands straight from the accumulators, one 16-key chunk kc
    // at a time (elements 8(kc&1)..+7 of s[kc/2]), rounded to f16; the row
    // sum adds the rounded values (the weights the products use).
    // O^T += V^T P^T with V^T fragments by transpose reads of the [key][d]
    // stage: keys 4hh..4hh+3 and 8+4hh..8+4hh+3 of each chunk (the P^T
    // order).  Chunk 0's exponentials come first; those of chunk kc+1 are
    // placed between the NDB matrix instructions of chunk kc, V fragments are
    // read VA instructions ahead.
    constexpr int NPV = 4 * C::NDB, VA = 3;
    uint32_t pw[4][4];
    auto pexp = [&](float x) {
      return __builtin_amdgcn_exp2f(EXACT ? (x - m_sub) * cscale : __builtin_fmaf(x, cscale, -m_sub));
    };
    auto exps = [&](int kc, int j) {  // pair j of chunk kc
      const float p0 = pexp(s[kc >> 1][8 * (kc & 1) + 2 * j]);
      const float p1 = pexp(s[kc >> 1][8 * (kc & 1) + 2 * j + 1]);
      if constexpr (DQ == 3) {
        const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnesBf16x2, l_run, false);
        pw[kc][j] = __builtin_bit_cast(uint32_t, pp);
      } else {
        const f16x2 pp = {(_Float16)p0, (_Float16)p1};
        l_run = __builtin_amdgcn_fdot2(pp, kOnesF16x2, l_run, false);
        pw[kc][j] = __builtin_bit_cast(uint32_t, pp);
      }
    };
    auto vread = [&](int i) {  // MFMA i: chunk i / NDB, head_dim block i % NDB
      const uint8_t* vp = vbase + (i / C::NDB) * 16 * C::VROW + (i % C::NDB) * 64;
      const s16x4 lo = lds_read_tr16(vp);
      const s16x4 hi = lds_read_tr16(vp + 8 * C::VROW);
      f16x8 vf;
      __builtin_memcpy(&vf, &lo, 8);
      __builtin_memcpy((char*)&vf + 8, &hi, 8);
      return vf;
    };
    f16x8 vf[VA];
#pragma unroll
    for (int i = 0; i < VA; ++i) vf[i] = vread(i);
#pragma unroll
    for (int j = 0; j < 4; ++j) exps(0, j);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NPV>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int kc = i / C::NDB, db = i % C::NDB;
      f16x8 pf;
      __builtin_memcpy(&pf, pw[kc], 16);
      o[db] = mma16<DQ>(vf[i % VA], pf, o[db]);
      if constexpr (i + VA < NPV) vf[i % VA] = vread(i + VA);
      if constexpr (kc + 1 < 4) {
        // pairs [J0, J1) of chunk kc+1 in this slot
        constexpr int J0 = db * 4 / C::NDB, J1 = (db + 1) * 4 / C::NDB;
        static_for<J0, J1>([&](auto jc) { exps(kc + 1, decltype(jc)::value); });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    __syncthreads();  // tile j+1 staged; buffer j&1 free
  };
  // KV tiles entirely at or below the first row's last key need no mask.
  const int n_full = min(ntiles, (kend_min + 1) / C::BN);
  auto kv_loop = [&](auto exact_form, auto stage_form) {
    int jt = jt_begin;
    for (; jt < n_full; ++jt) tile_step(jt, std::false_type{}, exact_form, stage_form);
    for (; jt < ntiles; ++jt) tile_step(jt, std::true_type{}, exact_form, stage_form);
  };
  if (heavy) {
    if (exact)
      kv_loop(std::true_type{}, std::false_type{});
    else
      kv_loop(std::false_type{}, std::false_type{});
  } else {
    if (exact)
      kv_loop(std::true_type{}, std::true_type{});
    else
      kv_loop(std::false_type{}, std::true_type{});
  }
  if (!PAIR && page_bad) atomicOr(a.err, (uint32_t)NVFP4KV_DEV_PAGE_OOB);

  float l_tot = l_run + __shfl_xor(l_run, 32);
  if (split >= 0 && !split_merge<D, 32 * W>(a, split, tid, tid, true, r, exact, cscale, m_run, l_tot, o)) return;

  // ---- epilogue: O / l * g_v -> bf16; lane holds O^T[d][row n]
  const float inv = gv / l_tot;
  if (row_valid) {
    uint16_t* orow = a.out + ((int64_t)(q_begin + tok) * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * hh;
        __bf16 v0 = (__bf16)(o[db][4 * i4 + 0] * inv), v1 = (__bf16)(o[db][4 * i4 + 1] * inv);
        __bf16 v2 = (__bf16)(o[db][4 * i4 + 2] * inv), v3 = (__bf16)(o[db][4 * i4 + 3] * inv);
        uint16_t u0, u1, u2, u3;
        __builtin_memcpy(&u0, &v0, 2);
        __builtin_memcpy(&u1, &v1, 2);
        __builtin_memcpy(&u2, &v2, 2);
        __builtin_memcpy(&u3, &v3, 2);
        *(uint2*)(orow + d) = make_uint2(u0 | ((uint32_t)u1 << 16), u2 | ((uint32_t)u3 << 16));
      }
  }
  if constexpr (PAIR) {
    // the light half, its own tiles done, stages the rest of the heavy
    // tile's KV tiles (one barrier each, as the heavy half's tile steps)
    if (!heavy) {
      for (int jt = ntiles; jt < nstage; ++jt) {
        pin_jobs<D, G, W>(job);
        TileStager<D, G, W, DQ> st(job, live, smem + ((jt + 1) & 1) * STG, tid);
        static_for<0, TileStager<D, G, W, DQ>::PIECES>([&](auto pc) { st.template piece<decltype(pc)::value>(job); });
        live = ka.load(a, job, jt + 2, page_next, page_bad);
        page_next = ka.lookup(a, jt + 3);
        __syncthreads();
      }
      if (page_bad) atomicOr(a.err, (uint32_t)NVFP4KV_DEV_PAGE_OOB);
    }
  }
}

#if NVFP4KV_PREFILL_SHARD == 0
// ---- device-built work list (ragged or split batches), heaviest item first.
// One workgroup: histogram of item costs (KV tiles an item visits), an
// exclusive scan in descending cost order, then each (request, Q tile) pair,
// one per thread, places its items (x KV heads) at the next free positions of
// their cost buckets.  An item is a Q tile, or, when split_len > 0, one of
// the balanced chunks of its KV range.  Batches whose KV does not fit in L2
// (PR #3575 page, section 3) use the stream order below instead.
constexpr int kCostBuckets = 4096;

__device__ __forceinline__ int tile_cost(int lq, int off, int t, int BQ) {
  return (off + min((t + 1) * BQ, lq) - 1) / kBlockN + 1;
}

// Exclusive scan of `sum` (this thread's share) across the 1024 threads:
// returns the sum of the shares of threads 0 .. tid-1.
__device__ __forceinline__ int block_exclusive_scan(int sum, int* warp_tot) {
  const int tid = threadIdx.x;
  int incl = sum;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += y;
  }
  if ((tid & 63) == 63) warp_tot[tid >> 6] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < (tid >> 6); ++w) wbase += warp_tot[w];
  __syncthreads();
  return wbase + incl - sum;
}

// Stream order (large batches whose KV does not fit in L2, nothing split):
// requests sorted by total cost, heaviest first; the Q tiles of one (request,
// KV head) stream consecutive and heaviest first, all on one XCD (workgroup p
// runs on XCD p % 8, and the stream of head h goes to XCD h % 8), so that a
// stream's KV tiles are fetched once into that XCD's L2 and reused by its Q
// tiles while they are resident.  Needs Hk % 8 == 0 (every XCD then gets the
// same number of items) and B <= kStreamOrderMaxReq.

__device__ void worklist_stream_order(const int32_t* __restrict__ qo, const int32_t* __restrict__ kvl,
                                      int B, int Hk, int BQ, int QT, int4* __restrict__ list,
                                      int* hist, int* warp_tot) {
  __shared__ int rank_req[kStreamOrderMaxReq];  // request of each rank
  __shared__ int rank_off[kStreamOrderMaxReq];  // tiles of the rank, then their exclusive scan
  const int tid = threadIdx.x;
  auto ntiles_of = [&](int rq) { return (qo[rq + 1] - qo[rq] + BQ - 1) / BQ; };
  auto total_of = [&](int rq) {
    const int lq = qo[rq + 1] - qo[rq], off = kvl[rq] - lq;
    int tot = 0;
    for (int t = 0; t * BQ < lq; ++t) tot += tile_cost(lq, off, t, BQ);
    return tot;
  };
  for (int rq = tid; rq < B; rq += 1024) atomicAdd(&hist[min(total_of(rq), kCostBuckets - 1)], 1);
  __syncthreads();
  // bucket starts in descending total cost
  constexpr int per = kCostBuckets / 1024;
  int vals[per], sum = 0;
  for (int i = 0; i < per; ++i) {
    vals[i] = hist[kCostBuckets - 1 - (tid * per + i)];
    sum += vals[i];
  }
  int run = block_exclusive_scan(sum, warp_tot);
  for (int i = 0; i < per; ++i) {
    hist[kCostBuckets - 1 - (tid * per + i)] = run;
    run += vals[i];
  }
  __syncthreads();
  for (int rq = tid; rq < B; rq += 1024) {
    const int rank = atomicAdd(&hist[min(total_of(rq), kCostBuckets - 1)], 1);
    rank_req[rank] = rq;
    rank_off[rank] = ntiles_of(rq);
  }
  __syncthreads();
  // exclusive scan of the tile counts in rank order
  constexpr int rper = kStreamOrderMaxReq / 1024;
  int rv[rper], rsum = 0;
  for (int i = 0; i < rper; ++i) {
    const int rank = tid * rper + i;
    rv[i] = rank < B ? rank_off[rank] : 0;
    rsum += rv[i];
  }
  int rrun = block_exclusive_scan(rsum, warp_tot);
  for (int i = 0; i < rper; ++i) {
    const int rank = tid * rper + i;
    if (rank < B) rank_off[rank] = rrun;
    rrun += rv[i];
  }
  __syncthreads();
  // XCD x holds heads h = x, x + 8, ...: per rank, Hk/8 streams of nt tiles
  const int hpx = Hk / kXcds;
  for (int rank = tid; rank < B; rank += 1024) {
    const int rq = rank_req[rank];
    const int lq = qo[rq + 1] - qo[rq], off = kvl[rq] - lq;
    const int nt = ntiles_of(rq);
    for (int h = 0; h < Hk; ++h) {
      const int x = h % kXcds, hi = h / kXcds;
      for (int tp = 0; tp < nt; ++tp) {
        const int t = nt - 1 - tp;  // heaviest tile first
        const int local = rank_off[rank] * hpx + hi * nt + tp;
        list[(int64_t)local * kXcds + x] = make_int4(rq, t * Hk + h, tile_cost(lq, off, t, BQ), -1);
      }
    }
  }
}

// Request order: items in (request, Q tile ascending, chunk, KV head) order,
// the positions from a scan of the item counts over the (request, Q tile)
// pairs.
__device__ void worklist_request_order(const int32_t* __restrict__ qo, const int32_t* __restrict__ kvl,
                                       int B, int Hk, int BQ, int QT, int split_len,
                                       int4* __restrict__ list, int* n_split, int* warp_tot) {
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)B * QT, per = (n + 1023) / 1024;
  const int64_t i0 = min(n, tid * per), i1 = min(n, i0 + per);
  auto chunks_of = [&](int64_t i, int& rq, int& t, int& lq, int& off, int& c) {
    rq = (int)(i / QT);
    t = (int)(i - (int64_t)rq * QT);
    lq = qo[rq + 1] - qo[rq];
    off = kvl[rq] - lq;
    if (t * BQ >= lq) return 0;
    c = tile_cost(lq, off, t, BQ);
    return split_len > 0 ? (c + split_len - 1) / split_len : 1;
  };
  int cnt = 0, rq, t, lq, off, c;
  for (int64_t i = i0; i < i1; ++i) cnt += chunks_of(i, rq, t, lq, off, c);
  int pos = block_exclusive_scan(cnt, warp_tot);
  for (int64_t i = i0; i < i1; ++i) {
    const int nch = chunks_of(i, rq, t, lq, off, c);
    if (nch == 0) continue;
    const int sid = nch > 1 ? atomicAdd(n_split, Hk) : -1;
    for (int k = 0; k < nch; ++k, ++pos) {
      const int beg = k * c / nch, end = (k + 1) * c / nch;
      for (int h = 0; h < Hk; ++h)
        list[(int64_t)pos * Hk + h] = make_int4(rq, t * Hk + h, (beg << 16) | end,
                                                nch > 1 ? ((sid + h) << 10) | (k << 5) | nch : -1);
    }
  }
}

// The work list of one call, in the given issue order.  It also zeroes the
// split tiles' arrival counters, so that every call starts from zero whatever
// an earlier call (or the workspace's first contents) left there.
__global__ __launch_bounds__(1024) void worklist_kernel(const int32_t* __restrict__ qo,
                                                        const int32_t* __restrict__ kvl, int B,
                                                        int Hk, int BQ, int QT, int split_len,
                                                        int order, int4* __restrict__ list,
                                                        int* __restrict__ counters,
                                                        int64_t num_counters) {
  __shared__ int hist[kCostBuckets];
  __shared__ int warp_tot[16];
  __shared__ int n_split;
  const int tid = threadIdx.x;
  for (int64_t i = tid; i < num_counters; i += 1024) counters[i] = 0;
  for (int i = tid; i < kCostBuckets; i += 1024) hist[i] = 0;
  if (tid == 0) n_split = 0;
  __syncthreads();
  if (order == kOrderStream) {
    worklist_stream_order(qo, kvl, B, Hk, BQ, QT, list, hist, warp_tot);
    return;
  }
  if (order == kOrderRequest) {
    worklist_request_order(qo, kvl, B, Hk, BQ, QT, split_len, list, &n_split, warp_tot);
    return;
  }
  for (int64_t i = tid; i < (int64_t)B * QT; i += 1024) {
    const int rq = (int)(i / QT), t = (int)(i - (int64_t)rq * QT);
    const int lq = qo[rq + 1] - qo[rq], off = kvl[rq] - lq;
    if (t * BQ >= lq) continue;
    {
      const int c = tile_cost(lq, off, t, BQ);
      const int nch = split_len > 0 ? (c + split_len - 1) / split_len : 1;
      for (int k = 0; k < nch; ++k) {
        const int w = (k + 1) * c / nch - k * c / nch;
        atomicAdd(&hist[min(w, kCostBuckets - 1)], Hk);
      }
    }
  }
  __syncthreads();
  // exclusive scan over buckets in descending cost: pos[c] = sum_{c' > c} hist[c']
  // each thread owns 4 consecutive descending buckets
  const int per = kCostBuckets / 1024;
  int vals[per];
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    vals[i] = hist[kCostBuckets - 1 - (tid * per + i)];
    sum += vals[i];
  }
  // inclusive scan of `sum` across the 1024 threads (wave64 shuffles + LDS)
  int incl = sum;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += y;
  }
  if ((tid & 63) == 63) warp_tot[tid >> 6] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < (tid >> 6); ++w) wbase += warp_tot[w];
  int run = wbase + incl - sum;
  __syncthreads();
  for (int i = 0; i < per; ++i) {
    hist[kCostBuckets - 1 - (tid * per + i)] = run;
    run += vals[i];
  }
  __syncthreads();
  for (int64_t i = tid; i < (int64_t)B * QT; i += 1024) {
    const int rq = (int)(i / QT), t = (int)(i - (int64_t)rq * QT);
    const int lq = qo[rq + 1] - qo[rq], off = kvl[rq] - lq;
    if (t * BQ >= lq) continue;
    {
      const int c = tile_cost(lq, off, t, BQ);
      const int nch = split_len > 0 ? (c + split_len - 1) / split_len : 1;
      const int sid = nch > 1 ? atomicAdd(&n_split, Hk) : -1;
      for (int k = 0; k < nch; ++k) {
        const int beg = k * c / nch, end = (k + 1) * c / nch;
        const int p = atomicAdd(&hist[min(end - beg, kCostBuckets - 1)], Hk);
        for (int h = 0; h < Hk; ++h)
          list[p + h] = make_int4(rq, t * Hk + h, (beg << 16) | end,
                                  nch > 1 ? ((sid + h) << 10) | (k << 5) | nch : -1);
      }
    }
  }
}

#endif  // NVFP4KV_PREFILL_SHARD == 0

// One launch: a.num_items workgroups of one W-wave tile, or (PAIR, 4-wave
// tiles) of two.
template <int D, int G, int W, bool PA, int DQ, bool PAIR>
void launch_one(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, G, W, PA, DQ, PAIR>), dim3(a.num_items), dim3(64 * W * (PAIR ? 2 : 1)),
                     0, s, a);
}
template <int D, int G, int W, int DQ, bool PAIR>
void launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (kBlockN % a.ps_div.d == 0)
    launch_one<D, G, W, true, DQ, PAIR>(a, s);
  else
    launch_one<D, G, W, false, DQ, PAIR>(a, s);
}

// The kernels of one shape held by this shard: launches and returns true,
// or returns false when another shard holds them.
template <int D, int G, int W, int DQ>
bool launch_shape(const PrefillArgs& a, bool paired, hipStream_t s) {
  if (paired) {
    if constexpr (W == 4 && prefill_shard_of(D, true) == NVFP4KV_PREFILL_SHARD) {
      launch_prefill<D, G, W, DQ, true>(a, s);
      return true;
    }
    return false;
  }
  if constexpr (prefill_shard_of(D, false) == NVFP4KV_PREFILL_SHARD) {
    launch_prefill<D, G, W, DQ, false>(a, s);
    return true;
  }
  return false;
}
// The ablation and MX score modes (head_dim 128, group 4, 4-wave tiles, page
// sizes dividing the KV tile).
template <int DQ>
bool launch_mode(const PrefillArgs& a, bool paired, hipStream_t s) {
  if (paired) {
    if constexpr (prefill_shard_of(128, true) == NVFP4KV_PREFILL_SHARD) {
      launch_one<128, 4, 4, true, DQ, true>(a, s);
      return true;
    }
    return false;
  }
  if constexpr (prefill_shard_of(128, false) == NVFP4KV_PREFILL_SHARD) {
    launch_one<128, 4, 4, true, DQ, false>(a, s);
    return true;
  }
  return false;
}

}  // namespace

#define NVFP4KV_CAT2(x, y) x##y
#define NVFP4KV_CAT(x, y) NVFP4KV_CAT2(x, y)
bool NVFP4KV_CAT(launch_prefill_shard, NVFP4KV_PREFILL_SHARD)(const PrefillArgs& a, int D, int G, int W,
                                                             int dq, bool paired, hipStream_t s) {
  switch (dq) {
    case 1: return launch_mode<1>(a, paired, s);
    case 2: return launch_mode<2>(a, paired, s);
    case 4: return launch_mode<4>(a, paired, s);
    case 5: return launch_mode<5>(a, paired, s);
    default: break;
  }
#define NVFP4KV_CASE(DD, GG, WW)                                                       \
  if (D == DD && G == GG && W == WW)                                                   \
    return dq == 3 ? launch_shape<DD, GG, WW, 3>(a, paired, s)                         \
                   : dq == 0 ? launch_shape<DD, GG, WW, 0>(a, paired, s) : false;
  NVFP4KV_CASE(128, 1, 4) NVFP4KV_CASE(128, 2, 4) NVFP4KV_CASE(128, 4, 4) NVFP4KV_CASE(128, 8, 4)
  NVFP4KV_CASE(128, 1, 8) NVFP4KV_CASE(128, 2, 8) NVFP4KV_CASE(128, 4, 8) NVFP4KV_CASE(128, 8, 8)
  NVFP4KV_CASE(64, 1, 4) NVFP4KV_CASE(64, 2, 4) NVFP4KV_CASE(64, 4, 4) NVFP4KV_CASE(64, 8, 4)
#undef NVFP4KV_CASE
  return false;
}

}  // namespace nvfp4kv

#if NVFP4KV_PREFILL_SHARD == 0
using namespace nvfp4kv;

extern "C" int paged_prefill_causal(const void* q, const int32_t* qo_indptr,
                                    const int32_t* kv_indptr, const int32_t* page_table,
                                    const int32_t* kv_lens, const nvfp4kv_cache* caches, void* out,
                                    float sm_scale, const nvfp4kv_prefill_plan* plan,
                                    void* workspace, int64_t workspace_bytes, uint32_t* dev_error,
                                    void* stream) {
  if (!plan || !caches || !(sm_scale > 0.0f) || !(sm_scale <= 3.402823466e38f)) return NVFP4KV_EINVAL;
  const nvfp4kv_prefill_plan& p = *plan;
  const nvfp4kv_cache& c = *caches;
  if (p.num_kv_heads != c.num_kv_heads || p.head_dim != c.head_dim ||
      p.page_size != c.page_size || p.num_q_heads % p.num_kv_heads != 0)
    return NVFP4KV_EINVAL;
  if (p.num_tiles == 0) return NVFP4KV_OK;
  if (!q || !qo_indptr || !kv_indptr || !page_table || !kv_lens || !out || !dev_error ||
      !c.k_cache || !c.v_cache || !c.k_sf || !c.v_sf || !c.k_scale || !c.v_scale)
    return NVFP4KV_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 8) || !aligned(c.k_cache, 16) || !aligned(c.v_cache, 16) ||
      !aligned(c.k_sf, 8) || !aligned(c.v_sf, 8))
    return NVFP4KV_EINVAL;
  if (p.num_items >= (1ll << 31) || p.batch <= 0) return NVFP4KV_EUNSUPPORTED;
  if (p.workspace_bytes > 0 && (!workspace || workspace_bytes < p.workspace_bytes ||
                                !aligned(workspace, 256)))
    return NVFP4KV_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.qo = qo_indptr;
  a.kvp = kv_indptr;
  a.pt = page_table;
  a.kvl = kv_lens;
  a.kc = c.k_cache;
  a.vc = c.v_cache;
  a.ksf = c.k_sf;
  a.vsf = c.v_sf;
  a.kscale = c.k_scale;
  a.vscale = c.v_scale;
  a.out = (uint16_t*)out;
  a.err = dev_error;
  a.num_pages = c.num_pages;
  a.ps_div = make_fastdiv((uint32_t)c.page_size);
  a.Hq = p.num_q_heads;
  a.Hk = p.num_kv_heads;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.B = p.batch;
  a.QT = p.q_tiles_per_head;
  if (p.schedule == kOrderStream ? !stream_order_available(p)
      : p.schedule == kOrderPaired ? !paired_order_available(p)
                                   : p.schedule != kOrderHeaviest && p.schedule != kOrderRequest)
    return NVFP4KV_EUNSUPPORTED;
  const bool paired = p.schedule == kOrderPaired;
  a.order = p.schedule;
  a.nxcd = p.num_xcd > 0 ? p.num_xcd : 1;
  a.num_tiles = (uint32_t)p.num_tiles;
  // paired: one workgroup per (request, KV head) and pair of Q tiles
  a.num_items = paired ? (uint32_t)((int64_t)p.batch * p.num_kv_heads * ((p.q_tiles_per_head + 1) / 2))
                       : (uint32_t)p.num_items;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int D = p.head_dim;
  const int W = p.block_q * G / 32;  // waves per tile chosen by the plan
  // every kernel this call could launch exists, or nothing is launched
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  const bool shape_ok = g_ok && ((D == 128 && (W == 4 || W == 8)) || (D == 64 && W == 4));
  // bf16 staging (mode 3) for every kernel shape; the other modes of the
  // dequant-placement ablation and the MX score modes for head_dim 128, GQA
  // group 4, 4-wave tiles and page sizes dividing the KV tile
  const bool mode_ok = p.dequant_mode == 0 || p.dequant_mode == 3 ||
                       (p.dequant_mode >= 1 && p.dequant_mode <= 5 && D == 128 && G == 4 && W == 4 &&
                        kBlockN % c.page_size == 0);
  if (!shape_ok || !mode_ok) return NVFP4KV_EUNSUPPORTED;
  const WorkspaceLayout wl = workspace_layout(p);
  // the heavy/light pairing assumes two co-resident workgroups per CU
  a.snake = p.block_q * (p.num_q_heads / p.num_kv_heads) == 128 &&
            p.num_tiles <= 2 * (int64_t)p.cu_count;
  if (!p.uniform_q || p.split_len > 0) {
    a.worklist = (const int4*)workspace;
    a.counters = (int*)((uint8_t*)workspace + wl.counters);
    a.partials = (float*)((uint8_t*)workspace + wl.partials);
    a.partial_floats = wl.partial_bytes / 4;
    a.max_chunks = p.max_chunks;
    hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, s, qo_indptr, kv_lens, p.batch,
                       p.num_kv_heads, p.block_q, p.q_tiles_per_head, p.split_len, p.schedule,
                       (int4*)workspace, a.counters, 2 * p.num_split_tiles);
  }
  // (shape_ok and mode_ok above: exactly one shard holds the kernel)
  const bool launched = launch_prefill_shard0(a, D, G, W, p.dequant_mode, paired, s) ||
                        launch_prefill_shard1(a, D, G, W, p.dequant_mode, paired, s) ||
                        launch_prefill_shard2(a, D, G, W, p.dequant_mode, paired, s);
  if (!launched) return NVFP4KV_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP;
}

// ---- paged_prefill_causal_noalloc: the same launch with the workspace taken
// from a library-owned device array instead of the caller.  Each GPU holds its
// own copy of the array (in the code object's device memory) until the
// process ends; the host reaches it through the address that
// hipGetSymbolAddress returns on that device, never through the array's name
// (a host-side stand-in).
namespace nvfp4kv {
namespace {
constexpr int64_t kNoallocScratchBytes = NVFP4KV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

// The array's device address on the current device: looked up once per
// device (with that device current), then reused.  Null if the lookup fails.
void* scratch_device_ptr() {
  static std::mutex mu;
  static std::vector<void*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}
}  // namespace
}  // namespace nvfp4kv

extern "C" int paged_prefill_causal_noalloc(const void* q, const int32_t* qo_indptr,
                                            const int32_t* kv_indptr, const int32_t* page_table,
                                            const int32_t* kv_lens, const nvfp4kv_cache* caches,
                                            void* out, float sm_scale,
                                            const nvfp4kv_prefill_plan* plan, uint32_t* dev_error,
                                            void* stream) {
  if (!plan) return NVFP4KV_EINVAL;
  if (plan->workspace_bytes > kNoallocScratchBytes) return NVFP4KV_EWORKSPACE;
  void* ws = nullptr;
  if (plan->workspace_bytes > 0) {
    ws = scratch_device_ptr();
    if (!ws) return NVFP4KV_EHIP;
  }
  return paged_prefill_causal(q, qo_indptr, kv_indptr, page_table, kv_lens, caches, out, sm_scale,
                              plan, ws, ws ? kNoallocScratchBytes : 0, dev_error, stream);
}
#endif  // NVFP4KV_PREFILL_SHARD == 0
