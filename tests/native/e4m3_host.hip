// Host build of the library's device E4M3FN encoder (e4m3fn_from_f32 in the kernels' common
// header), for the CPU test that checks it on every binary32 bit pattern against the oracle.
// Test infrastructure: nothing in the library links this file.
#include "../../paged_kv_cache_176_amd/csrc/common.hpp"

extern "C" void e4m3fn_encode_patterns(uint32_t first, uint32_t count, uint8_t* out) {
  for (uint32_t i = 0; i < count; ++i) {
    const uint32_t u = first + i;
    out[i] = (uint8_t)pa::e4m3fn_from_f32(__builtin_bit_cast(float, u));
  }
}
