// Cache write: new tokens' K and V into their paged slots.
//
// V is addressed with its own head stride and written with its own width at its
// own column offset (vLLM PR #64064, "Details": the symmetric kernel reused K's
// head stride and element count for V).  bf16 caches receive the bits unchanged;
// fp8 caches receive E4M3FN(fp32(x) / fp32(scale)), round to nearest even,
// saturating at +-448 (reading of the pages' "fp8 E4M3 cache, per-tensor and
// per-head scales").
//
// One thread moves one 8-element vector (16 B of bf16 in; 16 B bf16 or 8 B fp8
// out).  The thread -> (token, head, vector) mapping is token-major so that a
// wave covers whole rows and its loads and stores are contiguous.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

// IDX: the flat item index type, 32-bit whenever the launch's item count fits (the divisions
// by the per-token and per-head counts are then 32-bit, a fraction of the 64-bit sequence)
template <bool FP8, bool VEC, typename IDX>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  const int nk = VEC ? a.c.dk / 8 : a.c.dk;          // vectors (or elements) per head for K
  const int nv = a.value ? (VEC ? a.c.dv / 8 : a.c.dv) : 0;
  const int per_head = nk + nv;
  const int per_tok = per_head * a.c.num_kv_heads;
  const IDX total = (IDX)per_tok * (IDX)a.num_tokens;
  for (IDX item = (IDX)blockIdx.x * blockDim.x + threadIdx.x; item < total; item += (IDX)gridDim.x * blockDim.x) {
    const int t = (int)(item / (IDX)per_tok);
    const int r = (int)(item - (IDX)t * (IDX)per_tok);
    const int h = r / per_head;
    const int c = r - h * per_head;
    const bool isk = c < nk;
    const int e0 = VEC ? (isk ? c : c - nk) * 8 : (isk ? c : c - nk);      // element in K or V
    const uint16_t* src = isk ? a.key + (int64_t)t * a.k_st + (int64_t)h * a.k_sh + e0
                              : a.value + (int64_t)t * a.v_st + (int64_t)h * a.v_sh + e0;
    // the source (and the fp8 scale) do not depend on the slot: their loads go out
    // together with the slot's, one memory round trip instead of two
    u32x4 xv = {0, 0, 0, 0};
    uint16_t xs = 0;
    if constexpr (VEC) xv = *reinterpret_cast<const u32x4*>(src);
    else xs = *src;
    float scale = 1.0f;
    if constexpr (FP8) {
      const float* sp = isk ? a.c.k_scale : a.c.v_scale;
      scale = a.c.scale_mode == 2 ? sp[h] : sp[0];
    }
    const int64_t slot = a.slots[t];
    if (slot < 0) continue;                          // padding token
    const int bs = a.c.block_size;
    int64_t blk, pos;
    if ((bs & (bs - 1)) == 0) {                      // power-of-two block size: shifts
      blk = slot >> __builtin_ctz(bs);
      pos = slot & (bs - 1);
    } else {
      blk = slot / bs;
      pos = slot - blk * bs;
    }
    const int64_t row = blk * a.c.sb + pos * a.c.ss + (int64_t)h * a.c.sh;   // elements
    const int64_t dst_el = row + (isk ? 0 : a.c.v_off) + e0;
    if constexpr (!FP8) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.c.data) + dst_el;
      if constexpr (VEC) *reinterpret_cast<u32x4*>(dst) = xv;
      else *dst = xs;
    } else {
      uint8_t* dst = a.c.data + dst_el;
      if constexpr (VEC) {
        *reinterpret_cast<u32x2*>(dst) = bf16x8_to_e4m3fn(xv, scale);
      } else {
        *dst = (uint8_t)e4m3fn_from_f32(bf16_bits_to_f32(xs) / scale);
      }
    }
  }
}

bool launch_cache_write(const CacheWriteArgs& a, hipStream_t s) {
  const bool fp8 = a.c.esize == 1;
  // 8-element vectors need 16-byte aligned sources and 16 B (bf16) / 8 B (fp8)
  // aligned destinations for every (token, head, vector).
  auto al = [](const void* p, int n) { return ((uintptr_t)p % n) == 0; };
  const int dst_align = fp8 ? 8 : 16;
  bool vec = a.c.dk % 8 == 0 && al(a.key, 16) && a.k_st % 8 == 0 && a.k_sh % 8 == 0 &&
             al(a.c.data, dst_align) && a.c.sb % 8 == 0 && a.c.ss % 8 == 0 && a.c.sh % 8 == 0;
  if (a.value) vec = vec && a.c.dv % 8 == 0 && a.c.v_off % 8 == 0 && al(a.value, 16) && a.v_st % 8 == 0 &&
                     a.v_sh % 8 == 0;
  const int per = vec ? (a.c.dk + (a.value ? a.c.dv : 0)) / 8 : (a.c.dk + (a.value ? a.c.dv : 0));
  const int64_t total = (int64_t)per * a.c.num_kv_heads * a.num_tokens;
  if (total == 0) return true;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  dim3 grid((unsigned)blocks), block(256);
  // 32-bit item indices while the last item plus one grid stride stays below 2^31
  const bool narrow = total + (int64_t)blocks * 256 < ((int64_t)1 << 31);
  auto go = [&](auto fp8_tag, auto vec_tag) {
    constexpr bool F = decltype(fp8_tag)::value, V = decltype(vec_tag)::value;
    if (narrow) hipLaunchKernelGGL((cache_write_kernel<F, V, uint32_t>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((cache_write_kernel<F, V, int64_t>), grid, block, 0, s, a);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (fp8) {
    if (vec) go(T{}, T{});
    else go(T{}, F{});
  } else {
    if (vec) go(F{}, T{});
    else go(F{}, F{});
  }
  return true;
}

}  // namespace pa
