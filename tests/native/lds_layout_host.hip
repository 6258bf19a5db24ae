// Host build of the LDS ring swizzles the kernels use (paged_kv_cache_176_amd/csrc/lds_layout.hpp),
// for the layout test: the test computes the kernels' lane address patterns with these functions.
#include "../../paged_kv_cache_176_amd/csrc/lds_layout.hpp"

extern "C" int host_row_chunk_swz(int key) { return pa::row_chunk_swz(key); }
extern "C" int host_fp8_chunk_swz(int key) { return pa::fp8_chunk_swz(key); }
extern "C" int host_prefill_k_swz(int key) { return pa::prefill_k_swz(key); }
extern "C" int host_prefill_v_swz(int key) { return pa::prefill_v_swz(key); }
