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

// Rows of one attention tile and keys of one KV tile.
constexpr int kTileRows = 128;
constexpr int kBlockN = 64;

}  // namespace nvfp4kv
