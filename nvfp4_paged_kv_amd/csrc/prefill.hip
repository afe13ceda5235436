// prefill.hip -- batched causal prefill attention over the NVFP4 paged KV
// cache (gfx950, wave64, bf16 MFMA).
//
// Design points taken from the pages, re-made for CDNA4:
//  * FlashInfer PR #4769 page (NVFP4 KV tile repack; code analysis and "why"
//    sections): decoding NVFP4 inside the matrix-multiply loop made the
//    kernel instruction-bound; each KV tile is instead dequantized ONCE into a
//    16-bit staging tile that the matrix cores then read natively.  Here: the
//    whole workgroup decodes the tile (E2M1 x E4M3 is exact in bf16) into LDS,
//    K and V both staged [key][d]; K feeds v_mfma_f32_32x32x16_bf16 with
//    16-byte LDS reads, V with gfx950 LDS transpose reads.  The raw NVFP4
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

#include <type_traits>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
  const int2* worklist;  // ragged batches; null when uniform
  uint32_t* err;
  int64_t num_pages;
  FastDiv ps_div;
  int Hq, Hk;
  float sm_scale_log2;  // sm_scale * log2(e)
  int B, QT, head_first, nxcd;
  int snake;  // every tile is resident at once: pair heavy with light tiles
  uint32_t num_tiles;
};

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
  static constexpr int V_STAGE = BN * VROW;
  static constexpr int NDC = D / 16;        // MFMA k-steps over head_dim
  static constexpr int NDB = D / 32;        // 32-wide head_dim blocks of O^T
  static constexpr int PARTS = D / 32;      // 32-element dequant jobs per key row
  static constexpr int JOBS_PER_THREAD = 2 * BN * PARTS / NT;  // K and V
};

// Online-softmax reference max slack (log2 domain): probabilities are formed
// against a max that may lag the true running max by up to this much.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  // lo, hi are exactly representable in bf16: keep their upper halves.
  return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

template <int D>
__device__ __forceinline__ uint32_t scale_pair(const RawJob<D>& j, int part) {
  if constexpr (D == 128) return ((part < 2 ? j.sfrow.x : j.sfrow.y) >> (16 * (part & 1))) & 0xFFFFu;
  else return (j.sfrow >> (16 * (part & 1))) & 0xFFFFu;
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

// Raw page id of this thread's key in KV tile jt.
template <int D, int G, int W>
__device__ __forceinline__ int lookup_page(const PrefillArgs& a, int tid, int jt, int kend_max,
                                           const int32_t* ptb) {
  const int kk = min(jt * Cfg<D, G, W>::BN + job_key<D, G, W>(tid), kend_max);
  return ptb[fastdiv((uint32_t)kk, a.ps_div)];
}

// Issue the loads of this thread's jobs of KV tile jt; returns whether the
// key is live (at or before the last key any row sees, in a valid page).
template <int D, int G, int W>
__device__ __forceinline__ bool load_jobs(const PrefillArgs& a, RawJob<D> (&job)[Cfg<D, G, W>::JOBS_PER_THREAD],
                                          int tid, int jt, int page, int kend_max, int hk) {
  using C = Cfg<D, G, W>;
  const int kk = jt * C::BN + job_key<D, G, W>(tid);
  const bool live = kk <= kend_max;  // later keys are masked for every row: zeros
  const bool in_pool = (uint32_t)page < (uint64_t)a.num_pages;
  if (live && !in_pool) atomicOr(a.err, (uint32_t)NVFP4KV_DEV_PAGE_OOB);
  const int ps = (int)a.ps_div.d;
  const int64_t row =
      ((int64_t)(in_pool ? page : 0) * ps + (kk - (int)fastdiv((uint32_t)kk, a.ps_div) * ps)) * a.Hk + hk;
#pragma unroll
  for (int j = 0; j < C::JOBS_PER_THREAD; ++j) {
    const int id = tid + C::NT * j;
    const int tensor = id / (C::BN * C::PARTS);  // 0: K, 1: V
    const int part = id % C::PARTS;
    const uint8_t* cb = tensor ? a.vc : a.kc;
    const uint8_t* sb = tensor ? a.vsf : a.ksf;
    job[j].pk = *(const u32x4*)(cb + row * (D / 2) + part * 16);
    job[j].sfrow = *(const decltype(job[j].sfrow)*)(sb + row * (D / 16));
  }
  return live && in_pool;
}

// Dequantize a job (e2m1 x E4M3 is exact in bf16) into its staged row;
// dead keys stage zeros.  The empty asm pins the first use of the prefetched
// registers here (after the barrier): otherwise the compiler hoists their
// unpacking into the previous tile's matrix phase and waits for the loads
// there.
template <int D, int G, int W>
__device__ __forceinline__ void stage_jobs(RawJob<D>* job, bool live, uint8_t* smem, int tid) {
  using C = Cfg<D, G, W>;
#pragma unroll
  for (int j = 0; j < C::JOBS_PER_THREAD; ++j) asm volatile("" : "+v"(job[j].pk), "+v"(job[j].sfrow));
#pragma unroll
  for (int j = 0; j < C::JOBS_PER_THREAD; ++j) {
    const int id = tid + C::NT * j;
    const int tensor = id / (C::BN * C::PARTS);
    const int rem = id - tensor * C::BN * C::PARTS;
    const int key = rem / C::PARTS, part = rem % C::PARTS;
    uint8_t* rowp = tensor ? smem + C::K_STAGE + key * C::VROW : smem + key * C::KROW;
    const uint32_t sf = live ? scale_pair<D>(job[j], part) : 0u;
    const float S0 = e4m3_decode(sf & 0xFFu), S1 = e4m3_decode((sf >> 8) & 0xFFu);
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // 8 elements per packed dword
      const float S = w < 2 ? S0 : S1;
      const uint32_t x = job[j].pk[w];
      f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 0);
      f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 1);
      f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 2);
      f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 3);
      const u32x4 o = {bf16_pair(f0[0] * S, f0[1] * S), bf16_pair(f1[0] * S, f1[1] * S),
                       bf16_pair(f2[0] * S, f2[1] * S), bf16_pair(f3[0] * S, f3[1] * S)};
      *(u32x4*)(rowp + (part * 4 + w) * 16) = o;
    }
  }
}

template <int D, int G, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void prefill_kernel(PrefillArgs a) {
  using C = Cfg<D, G, W>;
  // Two staging buffers: tile j+1 is dequantized into one while tile j is
  // read from the other, with a single barrier per KV tile.
  constexpr int STG = C::K_STAGE + C::V_STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;

  // ---- which (request, KV head, Q tile) this workgroup computes
  int b, hk, qt;
  const uint32_t tile = blockIdx.x;
  if (a.worklist) {
    const int2 e = a.worklist[tile];
    b = e.x;
    qt = e.y / a.Hk;
    hk = e.y - qt * a.Hk;
  } else {
    const uint32_t bh_n = (uint32_t)a.B * a.Hk;
    uint32_t bh, qrev;
    if (a.head_first) {
      // heaviest Q tiles of every (request, head) first
      qrev = tile / bh_n;
      bh = tile - qrev * bh_n;
      // When the whole grid is resident at once, workgroup p and p + grid/2
      // share a CU: the second half walks the remaining tiles lightest first
      // so that every CU gets one heavy and one light tile.
      const uint32_t half = (a.QT + 1) / 2;
      if (a.snake && qrev >= half) qrev = a.QT - 1 - (qrev - half);
    } else {
      // stream-major: XCD x (blockIdx % nxcd) owns a contiguous range of
      // (request, head) streams, each walked heaviest tile first
      const uint32_t nx = a.nxcd, x = tile % nx, s = tile / nx;
      const uint32_t per = a.num_tiles / nx, rem = a.num_tiles % nx;
      const uint32_t L = x * per + (x < rem ? x : rem) + s;
      bh = L / a.QT;
      qrev = L - bh * a.QT;
    }
    b = bh / a.Hk;
    hk = bh - b * a.Hk;
    qt = a.QT - 1 - qrev;
  }

  const int q_begin = a.qo[b];
  const int Lq = a.qo[b + 1] - q_begin;
  const int Lk = a.kvl[b];
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q0 = qt * C::BQ;
  const int rows_valid = min(C::BQ, Lq - q0);
  if (rows_valid <= 0) return;  // (uniform batches with short requests)
  const int kend_max = off + q0 + rows_valid - 1;  // last key any row sees
  const int kend_min = off + q0;                   // last key of the first row
  const int ntiles = kend_max / C::BN + 1;
  const int32_t* ptb = a.pt + a.kvp[b];

  // Software pipeline: data of tile jt+1 and the page id of tile jt+2 are in
  // flight while tile jt is computed.
  RawJob<D> job[C::JOBS_PER_THREAD];
  bool live = load_jobs<D, G, W>(a, job, tid, 0, lookup_page<D, G, W>(a, tid, 0, kend_max, ptb), kend_max, hk);
  int page_next = lookup_page<D, G, W>(a, tid, 1, kend_max, ptb);

  const int r = wave * 32 + n;  // this lane's tile row
  const int tr = r % C::BQ, g = r / C::BQ;
  const bool row_valid = tr < rows_valid;
  const int tok = q0 + tr;
  const int hq = hk * G + g;
  const int kend = off + tok;

  const float gk = *a.kscale, gv = *a.vscale;
  if (tile == 0 && tid == 0 && !(scale_ok(gk) && scale_ok(gv)))
    atomicOr(a.err, (uint32_t)NVFP4KV_DEV_BAD_SCALE_ATTN);
  const float cscale = a.sm_scale_log2 * gk;  // scores -> log2 domain

  // ---- Q^T operand fragments: lane holds Q[row][16c + 8hh .. +7]
  bf16x8 qf[C::NDC];
  {
    const uint16_t* qrow = a.q + ((int64_t)(q_begin + (row_valid ? tok : q0)) * a.Hq + hq) * D;
#pragma unroll
    for (int c = 0; c < C::NDC; ++c) {
      u32x4 w = *(const u32x4*)(qrow + c * 16 + hh * 8);
      __builtin_memcpy(&qf[c], &w, 16);
    }
    // Consume the Q fragments here, so their load waits are placed before the
    // KV loop rather than inside it (where they would also wait for the
    // prefetch of the next tile).
#pragma unroll
    for (int c = 0; c < C::NDC; ++c) asm volatile("" ::"v"(qf[c]));
  }

  f32x16 o[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) o[i] = (f32x16){};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  // V^T operand addressing (transpose reads): lane t of each 16-lane group
  // points at 4 consecutive head_dim values of one key.
  const int t16 = lane & 15, g16 = (lane >> 4) & 1;
  const int voff = C::K_STAGE + (4 * hh + (t16 >> 2)) * C::VROW + (16 * g16 + 4 * (t16 & 3)) * 2;

  // Pipeline prologue: tile 0 staged, tile 1's NVFP4 bytes and tile 2's page
  // ids in flight.
  stage_jobs<D, G, W>(job, live, smem, tid);
  live = load_jobs<D, G, W>(a, job, tid, 1, page_next, kend_max, hk);
  page_next = lookup_page<D, G, W>(a, tid, 2, kend_max, ptb);
  __syncthreads();

  // One KV tile j: S^T = K Q^T from buffer j&1; dequantize tile j+1 into the
  // other buffer (VALU work that runs beside the matrix cores); prefetch tile
  // j+2; (mask), online softmax, O^T += V^T P^T; one barrier.
  auto tile_step = [&](const int jt, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const uint8_t* const sK = smem + (jt & 1) * STG;
    const uint8_t* const vbase = sK + voff;

    // ---- S^T = K Q^T for 64 keys: lane holds S^T[key 32kb + 8(i/4) + 4hh + i%4][row n]
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
      const uint8_t* krow = sK + (kb * 32 + n) * C::KROW + hh * 16;
#pragma unroll
      for (int c = 0; c < C::NDC; ++c) {
        bf16x8 kf;
        __builtin_memcpy(&kf, krow + c * 32, 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }

    // ---- stage tile j+1 (the other buffer was released by the last barrier;
    // past the last tile this stages unused data), then prefetch tile j+2
    stage_jobs<D, G, W>(job, live, smem + ((jt + 1) & 1) * STG, tid);
    live = load_jobs<D, G, W>(a, job, tid, jt + 2, page_next, kend_max, hk);
    page_next = lookup_page<D, G, W>(a, tid, jt + 3, kend_max, ptb);

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
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the reference max moves only when the tile's max
    // exceeds it by more than kRescaleSlack (log2 units), so p stays below
    // 2^kRescaleSlack and the O^T rescale is skipped on most tiles.
    const float m_tile = mx * cscale;
    const bool grow = m_tile > m_run + kRescaleSlack;
    const float m_new = grow ? m_tile : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], cscale, -m_new));
        s[kb][i] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
    if (__any(grow)) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
    }

    // ---- P^T operands straight from the accumulators (16-key chunks)
    bf16x8 pf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[kc][j] = (__bf16)s[kc >> 1][8 * (kc & 1) + j];

    // ---- O^T += V^T P^T; V^T fragments by transpose reads of the [key][d] stage:
    // keys 4hh..4hh+3 and 8+4hh..8+4hh+3 of each 16-key chunk (the P^T order)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint8_t* vp = vbase + kc * 16 * C::VROW + db * 64;
        const s16x4 lo = lds_read_tr16(vp);
        const s16x4 hi = lds_read_tr16(vp + 8 * C::VROW);
        bf16x8 vf;
        __builtin_memcpy(&vf, &lo, 8);
        __builtin_memcpy((char*)&vf + 8, &hi, 8);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kc], o[db], 0, 0, 0);
      }
    }
    __syncthreads();  // tile j+1 staged; buffer j&1 free
  };
  // KV tiles entirely at or below the first row's last key need no mask.
  const int n_full = min(ntiles, (kend_min + 1) / C::BN);
  int jt = 0;
  for (; jt < n_full; ++jt) tile_step(jt, std::false_type{});
  for (; jt < ntiles; ++jt) tile_step(jt, std::true_type{});

  // ---- epilogue: O / l * g_v -> bf16; lane holds O^T[d][row n]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
}

// ---- ragged batches: device-built work list, heaviest tile first.
// One workgroup: histogram of tile costs (KV tiles a Q tile visits), an
// exclusive scan in descending cost order, then each request places its
// tiles (x KV heads) at the next free positions of its cost buckets.
constexpr int kCostBuckets = 4096;

__global__ __launch_bounds__(1024) void worklist_kernel(const int32_t* __restrict__ qo,
                                                        const int32_t* __restrict__ kvl, int B,
                                                        int Hk, int BQ, int2* __restrict__ list) {
  __shared__ int hist[kCostBuckets];
  __shared__ int warp_tot[16];
  const int tid = threadIdx.x;
  for (int i = tid; i < kCostBuckets; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int rq = tid; rq < B; rq += 1024) {
    const int lq = qo[rq + 1] - qo[rq], off = kvl[rq] - lq;
    for (int t = 0; t * BQ < lq; ++t) {
      const int last = off + min((t + 1) * BQ, lq) - 1;
      const int c = min(last / kBlockN + 1, kCostBuckets - 1);
      atomicAdd(&hist[c], Hk);
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
  for (int rq = tid; rq < B; rq += 1024) {
    const int lq = qo[rq + 1] - qo[rq], off = kvl[rq] - lq;
    for (int t = 0; t * BQ < lq; ++t) {
      const int last = off + min((t + 1) * BQ, lq) - 1;
      const int c = min(last / kBlockN + 1, kCostBuckets - 1);
      const int p = atomicAdd(&hist[c], Hk);
      for (int h = 0; h < Hk; ++h) list[p + h] = make_int2(rq, t * Hk + h);
    }
  }
}

template <int D, int G, int W>
void launch_prefill(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, G, W>), dim3(a.num_tiles), dim3(64 * W), 0, s, a);
}

}  // namespace
}  // namespace nvfp4kv

using namespace nvfp4kv;

extern "C" int paged_prefill_causal(const void* q, const int32_t* qo_indptr,
                                    const int32_t* kv_indptr, const int32_t* page_table,
                                    const int32_t* kv_lens, const nvfp4kv_cache* caches, void* out,
                                    float sm_scale, const nvfp4kv_prefill_plan* plan,
                                    void* workspace, int64_t workspace_bytes, uint32_t* dev_error,
                                    void* stream) {
  if (!plan || !caches) return NVFP4KV_EINVAL;
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
  if (p.num_tiles >= (1ll << 31) || p.batch <= 0) return NVFP4KV_EUNSUPPORTED;
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
  a.head_first = p.head_first;
  a.nxcd = p.num_xcd > 0 ? p.num_xcd : 1;
  a.num_tiles = (uint32_t)p.num_tiles;
  // the heavy/light pairing assumes two co-resident workgroups per CU
  a.snake = p.block_q * (p.num_q_heads / p.num_kv_heads) == 128 &&
            p.num_tiles <= 2 * (int64_t)device_props().cu_count;
  if (!p.uniform_q) {
    a.worklist = (const int2*)workspace;
    hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, s, qo_indptr, kv_lens, p.batch,
                       p.num_kv_heads, p.block_q, (int2*)workspace);
  }
  const int G = p.num_q_heads / p.num_kv_heads;
  const int D = p.head_dim;
  const int W = p.block_q * G / 32;  // waves per tile chosen by the plan
#define NVFP4KV_CASE(DD, GG, WW) \
  if (D == DD && G == GG && W == WW) launch_prefill<DD, GG, WW>(a, s); else
  NVFP4KV_CASE(128, 1, 4) NVFP4KV_CASE(128, 2, 4) NVFP4KV_CASE(128, 4, 4) NVFP4KV_CASE(128, 8, 4)
  NVFP4KV_CASE(128, 1, 8) NVFP4KV_CASE(128, 2, 8) NVFP4KV_CASE(128, 4, 8) NVFP4KV_CASE(128, 8, 8)
  NVFP4KV_CASE(64, 1, 4) NVFP4KV_CASE(64, 2, 4) NVFP4KV_CASE(64, 4, 4) NVFP4KV_CASE(64, 8, 4)
  return NVFP4KV_EUNSUPPORTED;
#undef NVFP4KV_CASE
  return hipGetLastError() == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP;
}
