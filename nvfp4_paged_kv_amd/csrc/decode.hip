// decode.hip -- one decode step of attention over the NVFP4 paged cache
// (gfx950, wave64, f16 MFMA).
//
// The step that follows the prefill in serving, on the same cache, codecs and
// page table: every request has one new query token, already appended, that
// attends to all of its kv_len keys (the Lq = 1 case of the prefill's
// bottom-right causal definition).  The KV range of a request is cut into
// chunks; the chunks' partial results are combined in chunk order by a
// second kernel, so the result does not depend on scheduling.
//
// One wave per (request, chunk, group of HP adjacent KV heads), eight
// independent waves per workgroup.  A token's code row stores the KV heads
// one after another, so HP heads whose slices fill one 128-byte line (HP = 2
// for head_dim 128, 4 for head_dim 64, when the head count allows) give every
// line of the code rows a single reader, which fetches it once.  Tiles of 32
// keys when a lane takes 64 elements of the row, else 64 keys:
//  * S^T = K Q^T with v_mfma_f32_16x16x32_f16: A = 16 keys x 32 contraction
//    elements, B = Q^T with the HP x G query heads of the wave as its columns
//    (columns >= HP x G are zero).  The contraction runs over the HP heads'
//    elements concatenated, in a lane-shaped order: lane (key k, quarter q)
//    supplies, in MFMA c, elements q*E + 8c .. +7 of the concatenated row
//    (E = HP x head_dim / 4), and the Q^T operand uses the same order, with
//    zeros where the element belongs to another head than the column's.  So
//    each lane dequantizes one contiguous quarter of the key's row straight
//    into registers.  K needs no LDS: each K element feeds one wave only.
//  * Online softmax per query head in the log2 domain with the prefill's lazy
//    rescaling; the four lanes of a column (one per quarter) share its max.
//  * O^T += V^T P^T with v_mfma_f32_16x16x32_f16, one 16-row head_dim block
//    at a time: V is dequantized into the wave's own LDS rows [key][HP x d]
//    and read back with transpose reads in the key order in which the S^T
//    accumulators hold P^T; the P^T operand of a block keeps only the
//    columns of the block's head.
// E2M1 x E4M3 is exact in f16 (and one packed f16 multiply applies a block
// scale to two elements); the bf16 queries enter as f16 after an exact
// per-head power-of-two rescale, P as f16.  g_k folds into the softmax scale
// and g_v into the output.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr f16x2 kOnes = {(_Float16)1.0f, (_Float16)1.0f};
constexpr float kRescaleSlack = 8.0f;  // log2 units, as in the prefill

// As in the prefill: rows whose scores can reach 2^24 in log2 units (c times
// the largest raw score, head_dim x 2^15 x 2688) form p = exp2((s - m) c) with
// the reference m in raw score units; others p = exp2(fma(s, c, -m)) with m
// in log2 units.  The choice is per query head, the same on every chunk.
template <int D>
__device__ __forceinline__ bool exact_scores(float c) {
  constexpr float kMaxRaw = (float)D * 32768.0f * 2688.0f;
  return c * kMaxRaw >= 16777216.0f;
}
constexpr int kWaves = 8;              // independent waves per workgroup

template <int D, int HP>
struct DCfg {
  static constexpr int E = HP * D / 4;          // elements of a lane quarter of the wave's row
  static constexpr int NC = E / 8;              // QK MFMAs per 16-key block (8 elements each)
  static constexpr int NB = E >= 64 ? 2 : 4;    // 16-key blocks per tile
  static constexpr int TK = 16 * NB;            // keys per tile
  static constexpr int NDB = HP * D / 16;       // 16-row head_dim blocks of O^T
  static constexpr int NSC = E / 16;            // block scales of a lane quarter (1, 2 or 4)
  static constexpr int VROW = 2 * HP * D + 32;  // padded f16 V row in LDS (bytes)
  static constexpr int LDS_WAVE = TK * VROW;
};

struct DecodeArgs {
  const uint16_t* q;
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
  float* partials;  // [batch][Hq][max_chunks][D + 4]: O, max, sum
  uint32_t* err;
  int64_t num_pages;
  int64_t num_items;
  FastDiv ps_div;
  int Hq, Hk, B;
  int chunk_len, max_chunks;
  float sm_scale_log2;
};


// One lane's quarter rows of a tile: for each 16-key block kb, the E/2 code
// bytes of K and of V and the dword holding their E/16 scale bytes.
template <int D, int HP>
struct Raw {
  uint32_t k[DCfg<D, HP>::NB][DCfg<D, HP>::NC], v[DCfg<D, HP>::NB][DCfg<D, HP>::NC];
  uint32_t ksf[DCfg<D, HP>::NB], vsf[DCfg<D, HP>::NB];
};

// 8 codes (one dword) times the E4M3 scale S, as 8 f16 values: two codes
// per conversion, one packed multiply per pair (the products have at most 5
// significant bits and lie in 2^-10 .. 2688: exact in f16).
__device__ __forceinline__ f16x8 dequant8(uint32_t x, float S) {
  const _Float16 s = (_Float16)S;  // exact (an E4M3 value)
  const f16x2 ss = {s, s};
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * ss;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * ss;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * ss;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * ss;
  const u32x4 w = {__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                   __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
  return __builtin_bit_cast(f16x8, w);
}

template <int D, int G, int HP>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs a) {
  using C = DCfg<D, HP>;
  constexpr int NB = C::NB, NC = C::NC, TK = C::TK;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * C::LDS_WAVE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  if (item >= a.num_items) return;
  // item = ((request * max_chunks) + chunk) * (Hk / HP) + head group
  const int ngr = a.Hk / HP;
  const int hk0 = (int)(item % ngr) * HP;
  const int64_t bc = item / ngr;
  const int chunk = (int)(bc % a.max_chunks), b = (int)(bc / a.max_chunks);
  const int Lk = a.kvl[b];
  const int k0 = chunk * a.chunk_len;
  if (k0 >= Lk) return;  // (ragged batches: past this request's last chunk)
  const int k1 = min(Lk, k0 + a.chunk_len);
  const int ntiles = (k1 - k0 + TK - 1) / TK;
  const int nchunks = (Lk + a.chunk_len - 1) / a.chunk_len;
  const int k16 = lane & 15, qq = lane >> 4;  // key within a 16-key block / quarter
  const int col = lane & 15;                  // query head column of the B and D operands
  const int lh = qq * C::E / D;               // the head (of the wave's HP) of this lane's quarter
  const int ldo = qq * C::E % D;              // its first head_dim element
  const bool col_live = col < HP * G;
  const int ch = col / G;                     // the head (of the HP) of this lane's column
  uint8_t* const vst = smem + wave * C::LDS_WAVE;
  const int32_t* const ptb = a.pt + a.kvp[b];

  const float gk = *a.kscale, gv = *a.vscale;
  if (item == 0 && lane == 0 && !(scale_ok(gk) && scale_ok(gv)))
    atomicOr(a.err, (uint32_t)NVFP4KV_DEV_BAD_SCALE_ATTN);
  // ---- Q^T operand: lane (col, qq) holds, for MFMA c, elements ldo + 8c .. +7
  // of query head hk0*G + col when the quarter's head is the column's, else
  // zeros; in f16 after an exact power-of-two rescale of the query head's
  // row (its largest magnitude to [2^14, 2^15)), folded back into its score
  // scale
  f16x8 qf[NC];
  float cscale;
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + hk0 * G + min(col, HP * G - 1)) * D + ldo;
    const bool mine = col_live && ch == lh;
    u32x4 qw[NC];
    uint32_t am = 0;  // largest |bf16| bit pattern of the row
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qw[c] = *(const u32x4*)(qrow + 8 * c);
      if (!mine) qw[c] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) am = max(am, max(qw[c][e] & 0x7FFFu, (qw[c][e] >> 16) & 0x7FFFu));
    }
    am = max(am, (uint32_t)__shfl_xor((int)am, 16));  // the row's other quarters
    am = max(am, (uint32_t)__shfl_xor((int)am, 32));
    const int sh = am >= 0x80u ? min(max((int)(am >> 7) - 127 - 14, -100), 113) : 0;
    const float down = u2f((uint32_t)(127 - sh) << 23);  // 2^-sh
    cscale = a.sm_scale_log2 * gk * u2f((uint32_t)(127 + sh) << 23);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 h = {(_Float16)(u2f(qw[c][e] << 16) * down), (_Float16)(u2f(qw[c][e] & 0xFFFF0000u) * down)};
        qw[c][e] = __builtin_bit_cast(uint32_t, h);
      }
      qf[c] = __builtin_bit_cast(f16x8, qw[c]);
    }
  }

  // ---- loads: page ids two tiles ahead, NVFP4 bytes one tile ahead.  Keys
  // past the chunk end are clamped to its last key (valid addresses; masked).
  bool page_bad = false;
  // the lane's scale bytes: E/16 of them at byte qq*E/16 of the wave's scale
  // row, read as the aligned dword that holds them
  constexpr int kScaleBytes = C::NSC;
  const int sfo = qq * kScaleBytes;
  auto lookup = [&](int t, int (&pg)[NB]) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const int key = min(k0 + TK * t + 16 * kb + k16, k1 - 1);
      pg[kb] = ptb[fastdiv((uint32_t)key, a.ps_div)];
    }
  };
  auto load = [&](int t, const int (&pg)[NB], Raw<D, HP>& r) {
    const int ps = (int)a.ps_div.d;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const int key = min(k0 + TK * t + 16 * kb + k16, k1 - 1);
      const bool in_pool = (uint32_t)pg[kb] < (uint64_t)a.num_pages;
      page_bad |= !in_pool;
      const int64_t rowi =
          ((int64_t)(in_pool ? pg[kb] : 0) * ps + (key - (int)fastdiv((uint32_t)key, a.ps_div) * ps)) *
              a.Hk + hk0;
      const int64_t co = rowi * (D / 2) + qq * (C::E / 2);
      if constexpr (NC >= 4) {
#pragma unroll
        for (int h = 0; h < NC / 4; ++h) {
          const u32x4 kw = *(const u32x4*)(a.kc + co + 16 * h), vw = *(const u32x4*)(a.vc + co + 16 * h);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            r.k[kb][4 * h + c] = kw[c];
            r.v[kb][4 * h + c] = vw[c];
          }
        }
      } else {
        const uint2 kw = *(const uint2*)(a.kc + co), vw = *(const uint2*)(a.vc + co);
        r.k[kb][0] = kw.x;
        r.k[kb][1] = kw.y;
        r.v[kb][0] = vw.x;
        r.v[kb][1] = vw.y;
      }
      const int64_t so = rowi * (D / 16) + (sfo & ~3);
      r.ksf[kb] = *(const uint32_t*)(a.ksf + so) >> (8 * (sfo & 3));
      r.vsf[kb] = *(const uint32_t*)(a.vsf + so) >> (8 * (sfo & 3));
    }
  };
  // the lane's block scales: scale j applies to elements 16j .. 16j + 15 of
  // its quarter, so MFMA c (elements 8c .. 8c + 7) takes scale c / 2
  auto scales = [&](uint32_t sfw, float (&S)[C::NSC]) {
    const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sfw, 1.0f, false);
    S[0] = lo[0];
    if constexpr (C::NSC >= 2) S[1] = lo[1];
    if constexpr (C::NSC == 4) {
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sfw, 1.0f, true);
      S[2] = hi[0];
      S[3] = hi[1];
    }
  };

  f32x4 o[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // reference max: log2 units, or raw score units on a wave whose query heads
  // need the exact score form
  float m_run = -__builtin_inff(), l_run = 0.0f;
  const bool exact = __any(col_live && exact_scores<D>(cscale));

  // V^T transpose-read addressing: lane t of each 16-lane group (quarter qq)
  // points at 4 consecutive head_dim values of key 4qq + t/4 (+16, +32m).
  const int voff = (4 * qq + (k16 >> 2)) * C::VROW + 4 * (k16 & 3) * 2;

  Raw<D, HP> raw;
  int pg[NB], pg_next[NB];
  lookup(0, pg);
  load(0, pg, raw);
  lookup(1, pg_next);

  // the KV loop, in one copy per score form (the choice is fixed per wave)
  auto kv_loop = [&](auto exact_form) {
  constexpr bool EXACT = decltype(exact_form)::value;
  for (int t = 0; t < ntiles; ++t) {
    Raw<D, HP> nraw;
    load(t + 1, pg_next, nraw);  // past the last tile: clamped, unused
    lookup(t + 2, pg_next);

    // ---- S^T = K Q^T: s[kb] holds S^T[key 16kb + 4qq + r][column]
    f32x4 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      float S[C::NSC];
      scales(raw.ksf[kb], S);
      s[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const f16x8 kf = dequant8(raw.k[kb][c], S[c / 2]);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }
    // ---- stage V (this lane's quarter rows) into the wave's LDS rows
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      float S[C::NSC];
      scales(raw.vsf[kb], S);
      uint8_t* vrow = vst + (16 * kb + k16) * C::VROW + qq * C::E * 2;
#pragma unroll
      for (int c = 0; c < NC; ++c) *(f16x8*)(vrow + 16 * c) = dequant8(raw.v[kb][c], S[c / 2]);
    }
    // ---- keys past the request's end (last tile only)
    const int kbase = k0 + TK * t;
    if (kbase + TK > Lk) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kbase + 16 * kb + 4 * qq + r >= Lk) s[kb][r] = -__builtin_inff();
    }
    // ---- online softmax: the column's max over its 4 quarter lanes
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
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
    // P^T for the 32 keys of half m: keys 32m + 4qq + r (block 2m), then
    // 32m + 16 + 4qq + r (block 2m+1); rounded to f16, the row sum adds the
    // rounded values
#pragma unroll
    for (int m = 0; m < NB / 2; ++m) {
      uint32_t pw[4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const float x0 = s[2 * m + h][2 * r2], x1 = s[2 * m + h][2 * r2 + 1];
          const float p0 = __builtin_amdgcn_exp2f(EXACT ? (x0 - m_new) * cscale : __builtin_fmaf(x0, cscale, -m_new));
          const float p1 = __builtin_amdgcn_exp2f(EXACT ? (x1 - m_new) * cscale : __builtin_fmaf(x1, cscale, -m_new));
          const f16x2 pp = {(_Float16)p0, (_Float16)p1};
          l_run = __builtin_amdgcn_fdot2(pp, kOnes, l_run, false);
          pw[2 * h + r2] = __builtin_bit_cast(uint32_t, pp);
        }
      // ---- O^T += V^T P^T, each head_dim block with its head's columns
#pragma unroll
      for (int hh = 0; hh < HP; ++hh) {
        f16x8 pf;
        {
          const bool keep = HP == 1 || ch == hh;
          const u32x4 pk = {keep ? pw[0] : 0u, keep ? pw[1] : 0u, keep ? pw[2] : 0u, keep ? pw[3] : 0u};
          pf = __builtin_bit_cast(f16x8, pk);
        }
#pragma unroll
        for (int db = hh * (D / 16); db < (hh + 1) * (D / 16); ++db) {
          const uint8_t* vp = vst + voff + 32 * m * C::VROW + 16 * db * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 16 * C::VROW));
          f16x8 vf;
          __builtin_memcpy(&vf, &lo, 8);
          __builtin_memcpy((char*)&vf + 8, &hi, 8);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }
    raw = nraw;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) pg[kb] = pg_next[kb];
  }
  };
  if (exact)
    kv_loop(std::true_type{});
  else
    kv_loop(std::false_type{});
  if (page_bad) atomicOr(a.err, (uint32_t)NVFP4KV_DEV_PAGE_OOB);

  // ---- the column's sum over its 4 quarter lanes; then output or partial
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!col_live) return;
  const int hq = hk0 * G + col;
  // this lane's head_dim blocks: those of its column's head
  constexpr int DB = D / 16;
  if (nchunks == 1) {
    const float inv = gv / l_tot;
    uint16_t* orow = a.out + ((int64_t)b * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      if (db / DB != ch) continue;
      const bf16x2 v01 = {(__bf16)(o[db][0] * inv), (__bf16)(o[db][1] * inv)};
      const bf16x2 v23 = {(__bf16)(o[db][2] * inv), (__bf16)(o[db][3] * inv)};
      *(uint2*)(orow + 16 * (db % DB) + 4 * qq) =
          make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
    }
  } else {
    float* part = a.partials + (((int64_t)b * a.Hq + hq) * a.max_chunks + chunk) * decode_partial_floats(D);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
      if (db / DB == ch) *(f32x4*)(part + 16 * (db % DB) + 4 * qq) = o[db];
    if (qq == 0) {
      part[D] = m_run;
      part[D + 1] = l_tot;
      part[D + 2] = exact ? cscale : 0.0f;  // how the merge compares references
    }
  }
}

// Combine the chunks of every request with more than one, in chunk order:
// one wave per (request, query head), D/64 head_dim elements per lane.
template <int D>
__global__ __launch_bounds__(64 * kWaves) void decode_merge_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (item >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(item / a.Hq);
  const int n = (a.kvl[b] + a.chunk_len - 1) / a.chunk_len;
  if (n <= 1) return;
  constexpr int64_t PF = decode_partial_floats(D);
  constexpr int U = 8;  // chunks whose loads are issued together
  constexpr int E = D / 64;
  const float* base = a.partials + item * a.max_chunks * PF;
  // Online over blocks of U chunks (one round of loads per block; requests
  // with at most U chunks need one): the block's max raises the reference,
  // the running sums are rescaled to it, then the block's chunks are added
  // in chunk order, so the sums do not depend on the loads' timing.
  float M = -__builtin_inff();
  float acc[E] = {};
  float L = 0.0f;
  // references in raw score units (times the row's scale c) or in log2 units
  const float c = base[D + 2];
  auto ratio = [&](float from, float to) {
    return __builtin_amdgcn_exp2f(c > 0.0f ? (from - to) * c : from - to);
  };
  for (int c0 = 0; c0 < n; c0 += U) {
    float mc[U], lc[U], oc[U][E];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int c = min(c0 + i, n - 1);  // past the end: a valid chunk, weight 0
      mc[i] = c0 + i < n ? base[c * PF + D] : -__builtin_inff();
      lc[i] = base[c * PF + D + 1];
#pragma unroll
      for (int e = 0; e < E; ++e) oc[i][e] = base[c * PF + lane * E + e];
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < U; ++i) Mb = __builtin_fmaxf(Mb, mc[i]);
    if (c0 > 0 && Mb > M) {  // the reference moves: rescale what is summed
      const float r = ratio(M, Mb);
      L *= r;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= r;
    }
    M = Mb;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (c0 + i >= n) break;
      const float f = ratio(mc[i], M);
      L = __builtin_fmaf(lc[i], f, L);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(oc[i][e], f, acc[e]);
    }
  }
  const float inv = *a.vscale / L;
  uint16_t* orow = a.out + item * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const __bf16 v = (__bf16)(acc[e] * inv);
    orow[e] = __builtin_bit_cast(uint16_t, v);
  }
}

template <int D, int G, int HP>
void launch_hp(const DecodeArgs& a, hipStream_t s) {
  const uint32_t grid = (uint32_t)((a.num_items + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((decode_kernel<D, G, HP>), dim3(grid), dim3(64 * kWaves), 0, s, a);
}

// hp is decode_heads_per_wave(D, G, Hk): 1, 2 or 4, at most HPMAX
template <int D, int G>
void launch_decode(const DecodeArgs& a, int hp, hipStream_t s) {
  constexpr int HPMAX = decode_heads_per_wave(D, G, 16);
  if (hp == 1) {
    launch_hp<D, G, 1>(a, s);
  } else if constexpr (HPMAX >= 2) {
    if (hp == 2) {
      launch_hp<D, G, 2>(a, s);
    } else if constexpr (HPMAX >= 4) {
      launch_hp<D, G, 4>(a, s);
    }
  }
}

}  // namespace
}  // namespace nvfp4kv

using namespace nvfp4kv;

extern "C" int paged_decode(const void* q, const int32_t* kv_indptr, const int32_t* page_table,
                            const int32_t* kv_lens, const nvfp4kv_cache* caches, void* out,
                            float sm_scale, const nvfp4kv_decode_plan* plan, void* workspace,
                            int64_t workspace_bytes, uint32_t* dev_error, void* stream) {
  if (!plan || !caches || !(sm_scale > 0.0f) || !(sm_scale <= 3.402823466e38f)) return NVFP4KV_EINVAL;
  const nvfp4kv_decode_plan& p = *plan;
  const nvfp4kv_cache& c = *caches;
  if (p.num_kv_heads != c.num_kv_heads || p.head_dim != c.head_dim || p.page_size != c.page_size ||
      p.num_q_heads % p.num_kv_heads != 0)
    return NVFP4KV_EINVAL;
  if (p.num_items == 0) return NVFP4KV_OK;
  if (!q || !kv_indptr || !page_table || !kv_lens || !out || !dev_error || !c.k_cache ||
      !c.v_cache || !c.k_sf || !c.v_sf || !c.k_scale || !c.v_scale)
    return NVFP4KV_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 8) || !aligned(c.k_cache, 16) || !aligned(c.v_cache, 16) ||
      !aligned(c.k_sf, 8) || !aligned(c.v_sf, 8))
    return NVFP4KV_EINVAL;
  if (p.chunk_len <= 0 || p.chunk_len % kBlockN != 0 || p.max_chunks <= 0) return NVFP4KV_EINVAL;
  // the plan's wave count must be the one its shape gives (the kernel maps
  // every item below num_items to a request, chunk and head group)
  const int hp = decode_heads_per_wave(p.head_dim, p.num_q_heads / p.num_kv_heads, p.num_kv_heads);
  if (p.heads_per_wave != hp || p.num_items != (int64_t)p.batch * (p.num_kv_heads / hp) * p.max_chunks)
    return NVFP4KV_EINVAL;
  if (p.workspace_bytes > 0 &&
      (!workspace || workspace_bytes < p.workspace_bytes || !aligned(workspace, 16)))
    return NVFP4KV_EWORKSPACE;
  DecodeArgs a{};
  a.q = (const uint16_t*)q;
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
  a.partials = (float*)workspace;
  a.err = dev_error;
  a.num_pages = c.num_pages;
  a.num_items = p.num_items;
  a.ps_div = make_fastdiv((uint32_t)c.page_size);
  a.Hq = p.num_q_heads;
  a.Hk = p.num_kv_heads;
  a.B = p.batch;
  a.chunk_len = p.chunk_len;
  a.max_chunks = p.max_chunks;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  const int G = p.num_q_heads / p.num_kv_heads;
#define NVFP4KV_DCASE(D_, G_) \
  if (p.head_dim == D_ && G == G_) launch_decode<D_, G_>(a, hp, s); else
  NVFP4KV_DCASE(128, 1) NVFP4KV_DCASE(128, 2) NVFP4KV_DCASE(128, 4) NVFP4KV_DCASE(128, 8)
  NVFP4KV_DCASE(64, 1) NVFP4KV_DCASE(64, 2) NVFP4KV_DCASE(64, 4) NVFP4KV_DCASE(64, 8)
  return NVFP4KV_EUNSUPPORTED;
#undef NVFP4KV_DCASE
  if (p.max_chunks > 1) {
    const uint32_t grid = (uint32_t)(((int64_t)p.batch * p.num_q_heads + kWaves - 1) / kWaves);
    if (p.head_dim == 128)
      hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(grid), dim3(64 * kWaves), 0, s, a);
    else
      hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(grid), dim3(64 * kWaves), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP;
}
