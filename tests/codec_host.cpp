// codec_host.cpp -- host (CPU) build of the HIP path's codec helpers
// (nvfp4_paged_kv_amd/csrc/nvfp4kv_codec.hpp), so the software encoders and
// the fast divider the kernels use can be compared with the oracle on the CPU.
#include <stdint.h>
#include "../nvfp4_paged_kv_amd/csrc/nvfp4kv_codec.hpp"

extern "C" {
void host_e2m1_sw(const uint32_t* pats, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (uint8_t)(((pats[i] >> 28) & 8u) | nvfp4kv::e2m1_mag_from_abs_bits(pats[i] & 0x7FFFFFFFu));
}
void host_e4m3(const float* s, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nvfp4kv::e4m3_encode(s[i]);
}
void host_e4m3_decode(uint8_t* codes, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = nvfp4kv::e4m3_decode(codes[i]);
}
void host_fastdiv(const uint32_t* n, int64_t cnt, uint32_t d, uint32_t* q) {
  nvfp4kv::FastDiv f = nvfp4kv::make_fastdiv(d);
  for (int64_t i = 0; i < cnt; ++i) q[i] = nvfp4kv::fastdiv(n[i], f);
}
int host_scale_ok(float g) { return nvfp4kv::scale_ok(g); }
}
