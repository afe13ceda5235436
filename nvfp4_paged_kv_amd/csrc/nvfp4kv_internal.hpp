// nvfp4kv_internal.hpp -- host-side helpers shared by the library's
// translation units (not part of the C ABI).
#pragma once
#include <stdint.h>

#include "../../include/nvfp4kv.h"

namespace nvfp4kv {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Per-device properties the plan and the launchers use (cached once per
// device; querying them never synchronizes).
struct DeviceProps {
  int cu_count;
  int num_xcd;
  int64_t l2_bytes_per_xcd;
};
const DeviceProps& device_props();

// Keys of one KV tile.  An attention tile has W waves of 32 query rows: 4
// (two workgroups per CU) or, for head_dim 128 batches with at least
// kWideTilesPerCu tiles per CU, 8 (one workgroup per CU; every dequantized KV
// tile then feeds twice the matrix work).
constexpr int kBlockN = 64;
constexpr int kWideTilesPerCu = 4;
// Split Q tiles: chunks of at least kMinSplit KV tiles, at most kMaxChunks.
constexpr int kMinSplit = 8;
constexpr int kMaxChunks = 16;

// Issue orders of the prefill's Q tiles (nvfp4kv_prefill_plan.schedule).
// Stream order on ragged batches keeps each KV head's streams on one of the
// kXcds XCDs (needs num_kv_heads % kXcds == 0) and ranks at most
// kStreamOrderMaxReq requests in one workgroup's LDS.
constexpr int kOrderHeaviest = 1;
constexpr int kOrderStream = 2;
constexpr int kOrderRequest = 3;
constexpr int kOrderPaired = 4;
constexpr int kXcds = 8;
constexpr int kStreamOrderMaxReq = 8192;
inline bool stream_order_available(const nvfp4kv_prefill_plan& p) {
  const bool list = !p.uniform_q || p.split_len > 0;
  return p.split_len == 0 &&
         (!list || (p.num_kv_heads % kXcds == 0 && p.batch <= kStreamOrderMaxReq));
}

// Paired order: uniform batches of 4-wave tiles with nothing split (no work
// list): Q tiles pp and q_tiles_per_head - 1 - pp of one (request, KV head)
// share one 8-wave workgroup.
inline bool paired_order_available(const nvfp4kv_prefill_plan& p) {
  return p.uniform_q && p.split_len == 0 && p.block_q * (p.num_q_heads / p.num_kv_heads) == 128;
}

// Workspace layout of one prefill call (shared by the plan and the launcher):
// [work list: 16 B per item][arrival counters: 2 x int32 per split tile]
// [partials: per split tile, max_chunks x (rows x head_dim fp32 + 2 x rows fp32)].
inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
struct WorkspaceLayout {
  int64_t list, counters, partials, total, partial_bytes;
};
inline WorkspaceLayout workspace_layout(const nvfp4kv_prefill_plan& p) {
  WorkspaceLayout w{};
  const bool need_list = !p.uniform_q || p.split_len > 0;
  const int64_t rows = (int64_t)p.block_q * (p.num_q_heads / p.num_kv_heads);
  w.partial_bytes = rows * p.head_dim * 4 + rows * 8;
  w.list = 0;
  w.counters = align256(need_list ? p.num_items * 16 : 0);
  w.partials = align256(w.counters + p.num_split_tiles * 8);
  w.total = p.num_split_tiles > 0 ? w.partials + p.num_split_tiles * p.max_chunks * w.partial_bytes
                                  : (need_list ? w.counters : 0);
  return w;
}

// Decode: chunks of at least kDecodeMinChunk keys, at most kDecodeMaxChunks
// per request, sized for about kDecodeWavesPerCu waves per CU (one round of
// the decode kernel's 8-wave workgroups, one per CU).  Workspace:
// one partial of head_dim + 4 fp32 (O, then max and sum; 16-byte rows) per
// (request, query head, chunk) when some request has two chunks.
constexpr int kDecodeMinChunk = 256;
constexpr int kDecodeMaxChunks = 4096;
constexpr int kDecodeWavesPerCu = 8;
constexpr int64_t decode_partial_floats(int head_dim) { return head_dim + 4; }
// KV heads per decode wave: as many adjacent heads as fill one 128-byte line
// of a token's code row (head_dim / 2 bytes each), while their query heads
// fit the 16 columns of the score MFMA and the head count divides evenly.
constexpr int decode_heads_per_wave(int head_dim, int group, int num_kv_heads) {
  int hp = 256 / head_dim;
  while (hp > 1 && (hp * group > 16 || num_kv_heads % hp != 0)) hp /= 2;
  return hp;
}
inline int64_t decode_workspace_bytes(const nvfp4kv_decode_plan& p) {
  return p.max_chunks > 1 ? (int64_t)p.batch * p.num_q_heads * p.max_chunks *
                                decode_partial_floats(p.head_dim) * 4
                          : 0;
}

}  // namespace nvfp4kv
