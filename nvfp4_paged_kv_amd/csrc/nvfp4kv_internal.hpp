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

}  // namespace nvfp4kv
