/*
 * nvfp4kv.h -- C ABI of the MI355X (gfx950) NVFP4 paged-KV library:
 * NVFP4 quantize + append into a paged KV cache through a slot mapping, and
 * batched causal prefill attention that reads those NVFP4 pages.
 *
 * Sources: the FlashInfer pull-request analysis pages
 *   [PR #6204] "NVFP4 KV cache append: removing the host sync" (append API,
 *              device global scales checked in the kernel, no host sync),
 *   [PR #4769] "NVFP4 KV tile repack" (prefill over NVFP4 KV, dequantize each
 *              KV tile once into a 16-bit staging tile),
 *   [PR #3575] "FP8 causal attention: O(1) tile decode and global scheduling"
 *              (uniform-length flag, heaviest-first Q tiles, L2 gate),
 *   [PR #5043] "plan(): Python max() to Tensor.max()" (plan-step max lengths
 *              from vectorised reductions, lengths cast to int32).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the name ends in `_host`.  All
 *     buffers belong to the caller; the library allocates nothing and keeps no
 *     state besides a per-device property cache and, for
 *     paged_prefill_causal_noalloc, one static device array per GPU.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns: none synchronizes the host, except
 *     nvfp4kv_read_device_error, which exists to do exactly that.
 *   - Problems the host can see without reading device memory return a
 *     negative status before anything is enqueued.  Problems only the device
 *     can see (bad device scales, out-of-range slots or page ids) set bits in
 *     the caller's 32-bit device error word `dev_error` (atomic OR).
 *   - Element types: bf16 = IEEE bfloat16 bit patterns (2 bytes).
 *
 * NVFP4 cache format (readings of the pages, which do not fix a layout):
 *   - a block is 16 consecutive head_dim elements of one (token, head);
 *     element value = e2m1(code) * E4M3(sf) * g, g the tensor's global
 *     decode scale (k_scale or v_scale);
 *   - E2M1 codes are 4 bits (bit 3 = sign), two per byte, the even element in
 *     the low nibble; scale factors are OCP E4M3FN bytes (unsigned use);
 *   - NHD pages: cache   uint8 [num_pages][page_size][num_kv_heads][head_dim/2]
 *                scales  uint8 [num_pages][page_size][num_kv_heads][head_dim/16]
 *   - slot s names cache row s: page s / page_size, offset s % page_size.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
enum {
  NVFP4KV_OK = 0,
  NVFP4KV_EINVAL = -1,        /* null pointer, bad size, misaligned pointer */
  NVFP4KV_EUNSUPPORTED = -2,  /* shape this build has no kernel for */
  NVFP4KV_ERANGE = -3,        /* host-visible length inconsistency (q_len > kv_len, ...) */
  NVFP4KV_EHIP = -4,          /* the HIP runtime reported an error */
  NVFP4KV_EWORKSPACE = -5     /* workspace missing or smaller than plan->workspace_bytes */
};

/* Bits of the device error word. */
enum {
  NVFP4KV_DEV_BAD_K_SCALE = 1u, /* k_scale not positive finite: the append wrote nothing */
  NVFP4KV_DEV_BAD_V_SCALE = 2u, /* v_scale not positive finite: the append wrote nothing */
  NVFP4KV_DEV_SLOT_OOB = 4u,    /* a slot >= num_pages * page_size: that row was skipped */
  NVFP4KV_DEV_PAGE_OOB = 8u,    /* a page id outside [0, num_pages): read as zeros */
  NVFP4KV_DEV_BAD_SCALE_ATTN = 16u, /* the prefill saw a non positive-finite k/v scale */
  NVFP4KV_DEV_SPLIT_TIMEOUT = 32u   /* a split Q tile's merge gave up waiting (never expected) */
};

/*
 * nvfp4_append_paged_kv -- quantize new K/V rows to NVFP4 and write them into
 * the paged cache at the slots slot_mapping names.  [PR #6204] introduction
 * and append-function section; the scale contract is its docstring section.
 *
 *   k, v          bf16 [num_tokens][num_kv_heads][head_dim], contiguous,
 *                 16-byte aligned.
 *   slot_mapping  int64 [num_tokens]; slot < 0 = padding row (skipped);
 *                 slot >= num_pages*page_size sets NVFP4KV_DEV_SLOT_OOB and
 *                 the row is skipped.  Two tokens with one slot: unspecified
 *                 which one wins.
 *   k_scale, v_scale  device fp32 scalars: global decode scales.  Checked by
 *                 the kernel, never read by the host.  If either is not
 *                 positive finite the kernel sets NVFP4KV_DEV_BAD_K_SCALE /
 *                 _BAD_V_SCALE and writes nothing at all.
 *   k_cache, v_cache, k_sf, v_sf  the NHD cache and scale pages (see above);
 *                 k_cache/v_cache 4-byte aligned.  Only the addressed rows
 *                 are written.
 *   dev_error     device uint32 error word (required).
 * Block quantizer (fp32, fixed order): a = max|x_i| (NaN ignored);
 * s = a / (6 g); sf = E4M3 round-to-nearest-even of s, saturating at 448;
 * r = sf ? 1/(E4M3(sf) g) : 0; code_i = sign(x_i) | E2M1 round-to-nearest-
 * even of x_i r, saturating at 6 (NaN -> magnitude 0).
 * num_tokens == 0: returns NVFP4KV_OK, enqueues nothing and checks nothing
 * (the scales included).
 */
int nvfp4_append_paged_kv(const void* k, const void* v, const int64_t* slot_mapping,
                          int64_t num_tokens, const float* k_scale, const float* v_scale,
                          uint8_t* k_cache, uint8_t* v_cache, uint8_t* k_sf, uint8_t* v_sf,
                          int64_t num_pages, int32_t page_size, int32_t num_kv_heads,
                          int32_t head_dim, uint32_t* dev_error, void* stream);

/* One NVFP4 paged cache: K and V share the geometry. */
typedef struct {
  const uint8_t* k_cache; /* [num_pages][page_size][num_kv_heads][head_dim/2] */
  const uint8_t* v_cache;
  const uint8_t* k_sf;    /* [num_pages][page_size][num_kv_heads][head_dim/16], 8-byte aligned */
  const uint8_t* v_sf;
  const float* k_scale;   /* device fp32 scalar */
  const float* v_scale;   /* device fp32 scalar */
  int64_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
} nvfp4kv_cache;

/* Host-side launch plan of one prefill batch (filled by nvfp4_prefill_plan). */
typedef struct {
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size;
  int32_t max_q_len, max_kv_len;   /* [PR #5043] prefill plan() max lengths */
  int64_t total_q, total_kv;
  int32_t uniform_q;   /* [PR #3575] review: total_q == batch * max_q_len */
  int32_t uniform_kv;  /* total_kv == batch * max_kv_len (informational) */
  int32_t head_first;  /* [PR #3575] L2 gate: all KV streams fit in L2 (informational;
                          `schedule` is what runs) */
  int32_t block_q;     /* query tokens per tile (tile = block_q tokens x G heads) */
  int32_t block_n;     /* keys per KV tile */
  int32_t q_tiles_per_head; /* uniform: ceil(max_q_len / block_q) */
  int32_t max_tile_cost;    /* KV tiles visited by the heaviest Q tile */
  int32_t num_xcd;          /* XCDs the tile order is spread over */
  int64_t num_tiles;        /* Q tiles over all requests and KV heads */
  int64_t kv_bytes;         /* NVFP4 K+V bytes the batch reads */
  int64_t l2_bytes;         /* L2 capacity used by the gate (all XCDs) */
  int64_t workspace_bytes;  /* device workspace paged_prefill_causal needs */
  int32_t split_len;        /* KV tiles per chunk of a split Q tile (0: no split) */
  int32_t max_chunks;       /* chunks of the most split Q tile */
  int64_t num_items;        /* work items: Q tiles, or their KV chunks (one
                               workgroup each; under schedule 4 two Q tiles
                               share one workgroup) */
  int64_t num_split_tiles;  /* Q tiles (x KV heads) whose KV range is split */
  /* Staging form and dequant-placement ablation (the PR #4769 page's
     before/after comparison); the plan sets 3 and a caller may change it
     before paged_prefill_causal:
       3  each NVFP4 KV tile decoded once per workgroup into a bf16 LDS tile
          (every E2M1 x E4M3 product is exact in bf16), bf16 queries and
          probabilities, bf16 matrix instructions -- the kernel's own design
          and the plan's choice; every kernel shape;
       0  the same with an f16 staging tile (exact as well), f16 queries
          after an exact power-of-two rescale per row and f16 probabilities
          (three more significant bits), f16 matrix instructions; every
          kernel shape (the f16 form the ablation modes 1 and 2 vary);
       1  as 0 with K codes and scales staged raw in LDS, every wave
          decoding its K operand fragments in registers inside the matrix
          loop (V as 0);
       2  as 0, decoding the codes with a byte table (v_perm) instead of the
          hardware conversion;
       4  native low-precision scores ([PR #4769] code analysis: the branch
          for matrix cores that take E2M1 operands): K requantized while
          staged from NVFP4 (E4M3 scale per 16) to MXFP4 (E8M0 scale per
          32, the format gfx950's scaled matrix instruction takes), queries
          in MXFP8, S = Q K^T on the scaled FP4 x FP8 instruction; V and P
          as 0.  Both requantizations round, so mode 4 has its own accuracy
          contract: |o - o_ref| <= 0.75 (1 + |o_ref|) per element and
          rms(o - o_ref) <= 0.2 rms(o_ref) per batch on N(0,1) data (its
          typical per-row relative error is about 12%);
       5  as 4 with K requantized to MXFP8 (E4M3 elements): twice the
          staged K bytes, the same instruction rate, contract 0.3 and 0.05
          (typical per-row relative error about 3%).
     1, 2, 4 and 5 exist for head_dim 128, GQA group 4, 4-wave tiles
     (block_q 32) and page sizes dividing 64; other shapes, and other mode
     values, return NVFP4KV_EUNSUPPORTED before anything is launched.
     0 to 3 give results within the same tolerance of the oracle (0, 1 and
     2 bit-identical). */
  int32_t dequant_mode;
  int32_t cu_count;         /* CUs the tile width and the KV split were sized for */
  /* Order in which the Q tiles (or their KV chunks) are issued.  The plan
     fills in its own choice; a caller may change it before
     paged_prefill_causal (results are bitwise the same in every order):
       1  heaviest first over every request and head ([PR #3575] sections 1
          and 2: global reverse order; head-first when the KV fits in L2);
       2  stream order: the Q tiles of one (request, KV head) consecutive,
          heaviest first, all on one XCD (the plan's choice when the KV does
          not fit in L2, [PR #3575] section 3); not with split Q tiles, and
          for ragged batches only with num_kv_heads % 8 == 0 and batch <= 8192;
       3  request order: requests in order, each one's Q tiles lightest first
          (no reordering; the baseline the others are measured against);
       4  paired order: Q tiles t and q_tiles_per_head - 1 - t of one
          (request, KV head) -- together about the same number of KV tiles
          for every t ([PR #3575] section 2 balances causal tiles by issuing
          the heavy ones first; here each heavy tile is matched with a light
          one) -- share one workgroup of twice the tile's waves: the light
          tile's waves stage every KV tile of the pair (the heavy tile's
          range) and compute their own, the heavy tile's waves only
          compute.  The plan's choice for uniform batches of 4-wave tiles
          that fill every workgroup slot without a split and whose KV fits
          in L2; available for uniform batches (uniform_q) of 4-wave tiles
          (block_q x G == 128) with nothing split (split_len 0).
     Other values, or 2 or 4 where it is not available, return
     NVFP4KV_EUNSUPPORTED. */
  int32_t schedule;
} nvfp4kv_prefill_plan;

/*
 * nvfp4_prefill_plan -- host-only plan step ([PR #5043] prefill plan();
 * [PR #3575] uniform check and L2 gate).  Reads two host arrays with single
 * vectorisable passes (no per-request work beyond one loop), touches no
 * device memory.
 *   qo_indptr_host  int32 [batch+1]: query rows of request r are
 *                   [qo_indptr[r], qo_indptr[r+1]); qo_indptr[0] == 0.
 *   kv_lens_host    int32 [batch]: cached keys of request r.  Lengths held
 *                   as uint32 must be converted to int32 first.
 *   kv_indptr_host  int32 [batch+1] or NULL: if given, each request must own
 *                   exactly ceil(kv_len / page_size) page-table entries.
 *   l2_bytes        L2 capacity of the whole device for the gate; 0 = query
 *                   the current HIP device.
 *   cu_count        compute units to size the tile width and the KV split
 *                   for; 0 = query the current HIP device.
 *   split_len       KV tiles per chunk when heavy Q tiles are split: 0 =
 *                   automatic (only for batches whose Q tiles cannot fill
 *                   every workgroup slot of the GPU), > 0 = split every Q
 *                   tile longer than this, < 0 = never.
 *   tile_waves      waves per attention workgroup (32 query rows each): 0 =
 *                   automatic (8 for head_dim 128 when the batch has at least
 *                   4 such tiles per CU, else 4), or 4, or 8 (head_dim 128).
 * Returns NVFP4KV_ERANGE if some q_len > kv_len, a length is negative, or a
 * page count does not match; NVFP4KV_EUNSUPPORTED if head_dim is not 64 or
 * 128, or num_q_heads / num_kv_heads is not 1, 2, 4 or 8; NVFP4KV_EINVAL for
 * a tile_waves other than 0, 4 or 8 (8 with head_dim 64), or a negative
 * l2_bytes or cu_count.
 * The reductions are single passes over the two int32 arrays in compiled
 * code (the work of a whole-tensor reduction, without a per-element
 * interpreted loop); only batches small enough to have their KV ranges split
 * take a second pass over their Q tiles.
 */
int nvfp4_prefill_plan(const int32_t* qo_indptr_host, const int32_t* kv_lens_host,
                       const int32_t* kv_indptr_host, int32_t batch, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                       int64_t l2_bytes, int32_t cu_count, int32_t split_len,
                       int32_t tile_waves, nvfp4kv_prefill_plan* plan);

/*
 * paged_prefill_causal -- batched causal prefill attention over the NVFP4
 * paged cache ([PR #4769]: each KV tile is dequantized once into a 16-bit LDS
 * staging tile outside the matrix-core loop -- bf16 by default (plan->
 * dequant_mode 3), since every E2M1 x E4M3 product is exact in bf16, with
 * bf16 queries and probabilities on bf16 matrix instructions; the f16 form
 * is dequant_mode 0; [PR #3575]: O(1) tile decode for uniform batches,
 * heaviest-first Q tiles, L2-gated order).
 *   q          bf16 [total_q][num_q_heads][head_dim], contiguous, 16-byte aligned.
 *   qo_indptr  int32 [batch+1] (device copy of the plan's host array).
 *   kv_indptr  int32 [batch+1]: request r's pages are
 *              page_table[kv_indptr[r] .. kv_indptr[r+1]).
 *   page_table int32 page ids; key j of request r is row
 *              (page_table[kv_indptr[r] + j/page_size], j % page_size).
 *   kv_lens    int32 [batch] (device copy of the plan's host array).
 *   caches     host pointer to the cache descriptor (its pointers are device
 *              pointers); geometry must match the plan.
 *   out        bf16 [total_q][num_q_heads][head_dim].
 *   sm_scale   softmax scale applied to q.k; must be positive and finite
 *              (NVFP4KV_EINVAL otherwise).
 *   plan       host pointer, from nvfp4_prefill_plan for these lengths.
 *   workspace  device buffer of at least plan->workspace_bytes (may be NULL
 *              when that is 0), 256-byte aligned, with no required contents:
 *              it holds the device work list and, for split Q tiles, the
 *              chunks' partial results and arrival counters, all of which
 *              the call itself initialises (the counters are zeroed by the
 *              work-list kernel that runs first).  Calls that share a
 *              workspace must not overlap.
 * Split Q tiles (plan->split_len > 0, batches too small to fill the GPU): the
 * KV range of a heavy Q tile is cut into chunks computed by separate
 * workgroups; the last chunk to finish merges the others' partial
 * (unnormalized O, running max, sum) in chunk order, so results do not depend
 * on which chunk finishes last.
 * Semantics: query row i of request r (q_len = Lq, kv_len = Lk) sits at
 * position Lk - Lq + i and attends to keys 0 .. Lk - Lq + i (bottom-right
 * causal alignment); query head h reads KV head h / (num_q_heads /
 * num_kv_heads); o = softmax(sm_scale * q . k_hat) . v_hat with k_hat, v_hat
 * the dequantized cache values.  Output rounded to bf16 (nearest-even).
 * Page ids outside [0, num_pages) set NVFP4KV_DEV_PAGE_OOB and read as 0.
 */
int paged_prefill_causal(const void* q, const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* page_table, const int32_t* kv_lens,
                         const nvfp4kv_cache* caches, void* out, float sm_scale,
                         const nvfp4kv_prefill_plan* plan, void* workspace,
                         int64_t workspace_bytes, uint32_t* dev_error, void* stream);

/*
 * paged_prefill_causal_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): paged_prefill_causal without the workspace argument.
 * The work list, split counters and partials go to a library-owned device
 * array of NVFP4KV_NOALLOC_SCRATCH_BYTES on each GPU (held from the first
 * use of the library on that GPU until the process ends); the call itself
 * allocates nothing.  A plan whose workspace_bytes exceed that size returns
 * NVFP4KV_EWORKSPACE before anything is enqueued.  The array keeps the last
 * call's contents; each call initialises what it reads (work list, zeroed
 * counters).  All calls on one GPU share the array: calls that overlap in
 * time on one GPU (different streams, or different host threads) race and
 * must not be issued.  Other arguments, errors and results are those of
 * paged_prefill_causal.
 */
#define NVFP4KV_NOALLOC_SCRATCH_BYTES (64ll << 20)
int paged_prefill_causal_noalloc(const void* q, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                 const int32_t* page_table, const int32_t* kv_lens,
                                 const nvfp4kv_cache* caches, void* out, float sm_scale,
                                 const nvfp4kv_prefill_plan* plan, uint32_t* dev_error,
                                 void* stream);

/* Host-side launch plan of one decode batch (filled by nvfp4_decode_plan). */
typedef struct {
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size;
  int32_t max_kv_len;       /* decode plan max_kv_len */
  int64_t total_kv;
  int32_t chunk_len;        /* keys per KV chunk (a multiple of 64) */
  int32_t max_chunks;       /* chunks of the longest request */
  int64_t num_items;        /* waves launched: batch x (num_kv_heads / heads_per_wave) x max_chunks */
  int64_t workspace_bytes;  /* chunk partials (0 when no request has two chunks) */
  int32_t heads_per_wave;   /* adjacent KV heads per wave: 2 (head_dim 128) or 4
                               (head_dim 64) when num_kv_heads allows and their
                               query heads number at most 16, else fewer */
} nvfp4kv_decode_plan;

/*
 * nvfp4_decode_plan -- host-only plan of a decode step: every request has one
 * new query token (already appended to the cache) that attends to all of its
 * kv_len keys.  The KV range of a request is cut into chunks of chunk_len
 * keys, one wave per (request, chunk, group of heads_per_wave adjacent KV
 * heads: their slices of a token's code row fill one 128-byte line, so each
 * line has one reader), so that short batches still fill the GPU; the
 * chunks' partial results are merged in chunk order.
 *   kv_lens_host  int32 [batch], each >= 1.
 *   chunk_len     keys per chunk: 0 = automatic (at least 256, enough chunks
 *                 for about 8 waves per CU), else a positive multiple of 64.
 * Returns NVFP4KV_ERANGE for a kv_len < 1, NVFP4KV_EINVAL for a bad
 * chunk_len, NVFP4KV_EUNSUPPORTED for shapes paged_prefill_causal does not
 * support either (head_dim 64 or 128, GQA group 1, 2, 4 or 8).
 */
int nvfp4_decode_plan(const int32_t* kv_lens_host, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t chunk_len, nvfp4kv_decode_plan* plan);

/*
 * paged_decode -- one decode step of attention over the NVFP4 paged cache:
 * the next step after the prefill, on the same cache, codecs and page table.
 *   q          bf16 [batch][num_q_heads][head_dim], contiguous, 16-byte aligned.
 *   kv_indptr, page_table, kv_lens, caches  as for paged_prefill_causal.
 *   out        bf16 [batch][num_q_heads][head_dim], 8-byte aligned.
 *   plan       host pointer, from nvfp4_decode_plan for these lengths.
 *   workspace  device buffer of at least plan->workspace_bytes, 16-byte
 *              aligned (may be NULL when that is 0); no initial contents are
 *              needed.  Calls that share a workspace must not overlap.
 * Semantics: those of paged_prefill_causal with one query row per request
 * (the row at position kv_len - 1 sees keys 0 .. kv_len - 1).  When a request
 * has more than one chunk, a second kernel combines the chunks' (unnormalized
 * O, max, sum) in chunk order.
 */
int paged_decode(const void* q, const int32_t* kv_indptr, const int32_t* page_table,
                 const int32_t* kv_lens, const nvfp4kv_cache* caches, void* out, float sm_scale,
                 const nvfp4kv_decode_plan* plan, void* workspace, int64_t workspace_bytes,
                 uint32_t* dev_error, void* stream);

/*
 * nvfp4kv_read_device_error -- the one synchronizing call: waits for `stream`,
 * copies the device error word to *bits_host and, if clear != 0, resets it to
 * 0.  Not for use under graph capture.
 */
int nvfp4kv_read_device_error(uint32_t* dev_error, void* stream, uint32_t* bits_host, int clear);

/* Human-readable name of a status code (static storage). */
const char* nvfp4kv_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int nvfp4kv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4KV_H */
