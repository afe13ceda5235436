// host.cpp -- host side of the C ABI: the prefill plan, status strings, the
// synchronizing device-error read and the device property cache.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {

const DeviceProps& device_props() {
  static std::mutex mu;
  static std::vector<DeviceProps> cache;
  static std::vector<bool> have;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) {
    cache.resize(dev + 1);
    have.resize(dev + 1, false);
  }
  if (!have[dev]) {
    DeviceProps p{256, 8, 4 << 20};
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      p.cu_count = v;
    // gfx950 groups 32 CUs per XCD; each XCD has its own L2.
    p.num_xcd = p.cu_count >= 32 ? p.cu_count / 32 : 1;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeL2CacheSize, dev) == hipSuccess && v > 0)
      p.l2_bytes_per_xcd = v;
    cache[dev] = p;
    have[dev] = true;
  }
  return cache[dev];
}

}  // namespace nvfp4kv

using namespace nvfp4kv;

extern "C" int nvfp4_prefill_plan(const int32_t* qo_indptr_host, const int32_t* kv_lens_host,
                                  const int32_t* kv_indptr_host, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t page_size, int64_t l2_bytes, int32_t cu_count,
                                  int32_t split_len, int32_t tile_waves,
                                  nvfp4kv_prefill_plan* plan) {
  if (!plan || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || page_size <= 0 ||
      head_dim <= 0 || l2_bytes < 0 || cu_count < 0 ||
      (batch > 0 && (!qo_indptr_host || !kv_lens_host)))
    return NVFP4KV_EINVAL;
  if (!(tile_waves == 0 || tile_waves == 4 || (tile_waves == 8 && head_dim == 128)))
    return NVFP4KV_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return NVFP4KV_EUNSUPPORTED;
  const int G = num_q_heads / num_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return NVFP4KV_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return NVFP4KV_EUNSUPPORTED;
  if (batch > 0 && qo_indptr_host[0] != 0) return NVFP4KV_ERANGE;

  nvfp4kv_prefill_plan p{};
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.page_size = page_size;
  // CUs the tile-width and split decisions size the batch against (0 = those
  // of the current device)
  const int cus = cu_count > 0 ? cu_count : device_props().cu_count;
  p.cu_count = cus;
  // bf16 staging tile, bf16 queries and probabilities, bf16 matrix
  // instructions (dequant mode 3)
  p.dequant_mode = 3;
  p.block_n = kBlockN;
  // One pass of reductions over the host arrays ([PR #5043]: max lengths from
  // a vectorised reduction, not a per-request Python loop).
  int32_t max_q = 0, max_kv = 0;
  int64_t tot_q = 0, tot_kv = 0, qtiles4 = 0, qtiles8 = 0;
  const int bq4 = 128 / G, bq8 = 256 / G;
  int32_t max_cost = 0;
  bool bad = false;
  for (int32_t r = 0; r < batch; ++r) {
    const int32_t lq = qo_indptr_host[r + 1] - qo_indptr_host[r];
    const int32_t lk = kv_lens_host[r];
    bad |= (lq < 0) | (lk < 0) | (lq > lk);
    if (kv_indptr_host)
      bad |= (kv_indptr_host[r + 1] - kv_indptr_host[r]) != (lk + page_size - 1) / page_size;
    max_q = lq > max_q ? lq : max_q;
    max_kv = lk > max_kv ? lk : max_kv;
    tot_q += lq;
    tot_kv += lk;
    qtiles4 += (lq + bq4 - 1) / bq4;
    qtiles8 += (lq + bq8 - 1) / bq8;
    // heaviest tile of this request: its last one, whose last row sees keys 0..lk-1
    const int32_t cost = lq > 0 ? (lk - 1) / kBlockN + 1 : 0;
    max_cost = cost > max_cost ? cost : max_cost;
  }
  if (bad) return NVFP4KV_ERANGE;
  if (kv_indptr_host && batch > 0 && kv_indptr_host[0] != 0) return NVFP4KV_ERANGE;
  p.max_q_len = max_q;
  p.max_kv_len = max_kv;
  p.total_q = tot_q;
  p.total_kv = tot_kv;
  p.uniform_q = tot_q == (int64_t)batch * max_q;  // [PR #3575] review: O(1) uniform check
  p.uniform_kv = tot_kv == (int64_t)batch * max_kv;
  // 8-wave tiles (256 rows, one workgroup per CU) halve the dequantization
  // per row but need many tiles to balance; 4-wave tiles (two per CU) for
  // head_dim 64 and for batches with fewer than kWideTilesPerCu 8-wave tiles
  // per CU.
  const bool wide = tile_waves == 8 ||
                    (tile_waves == 0 && head_dim == 128 &&
                     qtiles8 * num_kv_heads >= (int64_t)kWideTilesPerCu * cus);
  p.block_q = wide ? bq8 : bq4;
  p.q_tiles_per_head = (max_q + p.block_q - 1) / p.block_q;
  p.max_tile_cost = max_cost;
  p.num_tiles = (wide ? qtiles8 : qtiles4) * num_kv_heads;
  if (max_cost >= 65536) return NVFP4KV_EUNSUPPORTED;  // KV tile index packs into 16 bits
  // Batches whose Q tiles cannot fill every workgroup slot (one 8-wave or two
  // 4-wave workgroups per CU) split the KV range of their heaviest Q tiles so
  // that every slot gets about the same number of KV tiles: chunk length =
  // total KV tiles / slots.
  const int64_t slots = (int64_t)cus * (wide ? 1 : 2);
  p.num_items = p.num_tiles;
  if (split_len >= 0 && (split_len > 0 || p.num_tiles < slots)) {
    int64_t total_cost = 0;
    for (int32_t r = 0; r < batch; ++r) {
      const int32_t lq = qo_indptr_host[r + 1] - qo_indptr_host[r];
      const int32_t off = kv_lens_host[r] - lq;
      for (int32_t t = 0; t * p.block_q < lq; ++t)
        total_cost += (off + std::min((t + 1) * p.block_q, lq) - 1) / kBlockN + 1;
    }
    total_cost *= num_kv_heads;
    int32_t len = split_len > 0 ? split_len
                                : std::max((int32_t)((total_cost + slots - 1) / slots), kMinSplit);
    len = std::max(len, (max_cost + kMaxChunks - 1) / kMaxChunks);
    if (max_cost > len) {
      p.split_len = len;
      p.max_chunks = (max_cost + len - 1) / len;
      int64_t items = 0, split = 0;
      for (int32_t r = 0; r < batch; ++r) {
        const int32_t lq = qo_indptr_host[r + 1] - qo_indptr_host[r];
        const int32_t off = kv_lens_host[r] - lq;
        for (int32_t t = 0; t * p.block_q < lq; ++t) {
          const int32_t c = (off + std::min((t + 1) * p.block_q, lq) - 1) / kBlockN + 1;
          const int32_t nch = (c + len - 1) / len;
          items += nch;
          split += nch > 1;
        }
      }
      p.num_items = items * num_kv_heads;
      p.num_split_tiles = split * num_kv_heads;
    }
  }
  // [PR #3575] L2 gate: KV bytes = tokens x heads x bytes per token-head (K and
  // V, NVFP4: head_dim/2 code bytes + head_dim/16 scale bytes each); the
  // head-first (global reverse) order only when twice that fits in L2.
  p.kv_bytes = tot_kv * num_kv_heads * (int64_t)(head_dim / 2 + head_dim / 16) * 2;
  if (l2_bytes > 0) {
    p.l2_bytes = l2_bytes;
    p.num_xcd = cus >= 32 ? cus / 32 : 1;  // gfx950: 32 CUs per XCD
  } else {
    const DeviceProps& d = device_props();
    p.l2_bytes = d.l2_bytes_per_xcd * d.num_xcd;
    p.num_xcd = d.num_xcd;
  }
  p.head_first = 2 * p.kv_bytes <= p.l2_bytes;
  // Issue order: heaviest first over everything when the KV fits in L2;
  // otherwise stream order (each stream's KV fetched once into one XCD's L2)
  // where it is available, else heaviest first.
  p.schedule = !p.head_first && stream_order_available(p) ? kOrderStream : kOrderHeaviest;
  // Paired order instead of heaviest first for uniform batches of 4-wave
  // tiles that fill every workgroup slot without a split: the heavy causal
  // tiles, which set the batch's length, run with their staging done by the
  // waves of their light partners.
  if (p.schedule == kOrderHeaviest && paired_order_available(p) && p.num_tiles >= slots)
    p.schedule = kOrderPaired;
  // Ragged or split batches need a device work list (and, when split, the
  // chunks' partials and arrival counters).
  p.workspace_bytes = workspace_layout(p).total;
  *plan = p;
  return NVFP4KV_OK;
}

extern "C" int nvfp4_decode_plan(const int32_t* kv_lens_host, int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                 int32_t chunk_len, nvfp4kv_decode_plan* plan) {
  if (!plan || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || page_size <= 0 ||
      head_dim <= 0 || (batch > 0 && !kv_lens_host) || chunk_len < 0 || chunk_len % kBlockN != 0)
    return NVFP4KV_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return NVFP4KV_EUNSUPPORTED;
  const int G = num_q_heads / num_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return NVFP4KV_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return NVFP4KV_EUNSUPPORTED;
  nvfp4kv_decode_plan p{};
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.page_size = page_size;
  int32_t max_kv = 0;
  int64_t tot_kv = 0;
  bool bad = false;
  for (int32_t r = 0; r < batch; ++r) {
    const int32_t lk = kv_lens_host[r];
    bad |= lk < 1;
    max_kv = lk > max_kv ? lk : max_kv;
    tot_kv += lk;
  }
  if (bad) return NVFP4KV_ERANGE;
  p.max_kv_len = max_kv;
  p.total_kv = tot_kv;
  // One wave per (request, chunk, group of heads_per_wave KV heads).
  // Chunks: at least kDecodeMinChunk keys (the merge costs one partial per
  // chunk), and enough of them for about kDecodeWavesPerCu waves per CU.
  p.heads_per_wave = decode_heads_per_wave(head_dim, G, num_kv_heads);
  const int64_t groups = num_kv_heads / p.heads_per_wave;
  int64_t len = chunk_len;
  if (len == 0) {
    const int64_t target = (int64_t)kDecodeWavesPerCu * device_props().cu_count;
    len = (tot_kv * groups + target - 1) / std::max<int64_t>(target, 1);
    len = std::max<int64_t>((len + kBlockN - 1) / kBlockN * kBlockN, kDecodeMinChunk);
  }
  len = std::max<int64_t>(len, ((int64_t)max_kv + kDecodeMaxChunks - 1) / kDecodeMaxChunks);
  len = (len + kBlockN - 1) / kBlockN * kBlockN;
  p.chunk_len = (int32_t)std::min<int64_t>(len, 1 << 30);
  p.max_chunks = batch > 0 ? (int32_t)((max_kv + p.chunk_len - 1) / p.chunk_len) : 0;
  p.num_items = (int64_t)batch * groups * p.max_chunks;
  p.workspace_bytes = decode_workspace_bytes(p);
  *plan = p;
  return NVFP4KV_OK;
}

extern "C" int nvfp4kv_read_device_error(uint32_t* dev_error, void* stream, uint32_t* bits_host,
                                         int clear) {
  if (!dev_error || !bits_host) return NVFP4KV_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(bits_host, dev_error, 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return NVFP4KV_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return NVFP4KV_EHIP;
  if (clear) {
    if (hipMemsetAsync(dev_error, 0, 4, s) != hipSuccess) return NVFP4KV_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return NVFP4KV_EHIP;
  }
  return NVFP4KV_OK;
}

extern "C" const char* nvfp4kv_status_string(int status) {
  switch (status) {
    case NVFP4KV_OK: return "ok";
    case NVFP4KV_EINVAL: return "invalid argument (null pointer, size or alignment)";
    case NVFP4KV_EUNSUPPORTED: return "unsupported shape (head_dim or GQA group size)";
    case NVFP4KV_ERANGE: return "inconsistent lengths (q_len > kv_len, negative length or page count)";
    case NVFP4KV_EHIP: return "HIP runtime error";
    case NVFP4KV_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

extern "C" int nvfp4kv_abi_version(void) { return 105; }
