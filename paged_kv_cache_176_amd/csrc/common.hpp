// Shared device-side types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four 16-lane groups (rows) that hold the same MFMA output
// column.  v_permlane32_swap / v_permlane16_swap exchange rows in the VALU (no LDS
// round trip): with both operands v, each lane ends up with the pair {its value, the
// value 32 (then 16) lanes away}, in the same order on both lanes of the pair.  Inline
// asm: given two equal operands the compiler assumes the swap returns them unchanged
// and drops one of the pair.
__device__ __forceinline__ void swap_rows32(float& x, float& y) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap_rows16(float& x, float& y) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ float max_over_groups(float v) {
  float x = v, y = v;
  swap_rows32(x, y);
  v = fmaxf(x, y);
  x = v;
  y = v;
  swap_rows16(x, y);
  return fmaxf(x, y);
}
__device__ __forceinline__ float sum_over_groups(float v) {
  float x = v, y = v;
  swap_rows32(x, y);
  v = x + y;
  x = v;
  y = v;
  swap_rows16(x, y);
  return x + y;
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Four E4M3FN bytes (one dword) -> four bf16 in two dwords.  Exact: every E4M3FN
// value is a bf16 value (3 mantissa bits into 7, exponents 2^-9..2^8 in range).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// binary32 -> E4M3FN byte: nearest, ties to even, saturating, NaN -> 0x7F.  Also built
// for the host, where it is checked against the reference encoder on all 2^32 inputs.
__host__ __device__ __forceinline__ uint32_t e4m3fn_from_f32(float q) {
  uint32_t u = __builtin_bit_cast(uint32_t, q);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                 // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // |q| >= 448 or inf: saturate
  if (a >= 0x3C800000u) {                            // |q| >= 2^-6: normal E4M3FN
    // keep 3 of the 23 mantissa bits, ties to even on the 20 dropped bits;
    // a carry out of the mantissa bumps the exponent, as it should
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));         // rebias 127 -> 7
  }
  // subnormal range: multiples of 2^-9; |q| * 512 is exact, rint is ties-to-even
  float m = __builtin_rintf(__builtin_fabsf(q) * 512.0f);
  return sign | (uint32_t)m;                          // m = 8 is 0x08 = 2^-6, correct
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Eight bf16 (one 16-byte vector) -> eight E4M3FN bytes of fp32(x) / scale, in order.
__device__ __forceinline__ u32x2 bf16x8_to_e4m3fn(u32x4 x, float scale) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = x[i];
    const uint32_t b0 = e4m3fn_from_f32(bf16_bits_to_f32(w & 0xFFFFu) / scale);
    const uint32_t b1 = e4m3fn_from_f32(bf16_bits_to_f32(w >> 16) / scale);
    const uint32_t pair = b0 | (b1 << 8);
    if (i < 2) lo |= pair << (16 * i);
    else hi |= pair << (16 * (i - 2));
  }
  return u32x2{lo, hi};
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Split-KV partials (fp32, written once by a partial kernel, read once by the merge).
// WT: write-through stores (sc0 sc1 -- the line goes to memory at once instead of staying
// dirty in the XCD's L2 for the end of the kernel to write back).  Measured: it pays where a
// workgroup leaves large partials (MLA: 12 rows x 512 floats, 24.6 KB; the 32-row verify
// kernels) and costs a little where they are small (the DiffKV decode's 8 rows x 128), so the
// kernels choose.  Plain nontemporal stores measured slower everywhere.  The MLA verify token
// kernel (4 tokens' partials, 96 KB per workgroup) measured ~0.5-1% faster with plain stores.
template <bool WT>
__device__ __forceinline__ void store_partial4(float* p, f32x4 v) {
  if constexpr (WT) asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
  else *reinterpret_cast<f32x4*>(p) = v;
}
template <bool WT>
__device__ __forceinline__ void store_partial1(float* p, float v) {
  if constexpr (WT) asm volatile("global_store_dword %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
  else *p = v;
}
// The merge reads each partial once: nontemporal loads.
__device__ __forceinline__ f32x4 load_partial4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ float load_partial1(const float* p) { return __builtin_nontemporal_load(p); }

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4 with the
// nontemporal hint): lane i's bytes land at lds_base + 16*i, lds_base wave-uniform.
// Inline asm on purpose: the compiler's wait-count pass does not know which LDS reads
// these writes feed and answers with vmcnt(0) before some of them, which would empty
// a load ring on every tile.  Callers wait with explicit vmcnt counts instead.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// Same copy without the nontemporal hint (lines stay in L2 for a neighbour that
// reads the other part of them).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// Scalar-base forms: address = sbase (wave-uniform, SGPRs) + voff (per lane, 32-bit),
// which spares the 64-bit per-lane address arithmetic.
__device__ __forceinline__ void dma16_nt_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// Wait until at most N vector-memory ops of this wave are in flight (explicit count
// for the LDS-DMA rings above, which the compiler does not track).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Read-only int at a wave-uniform address, through the scalar data cache
// (s_load_dword).  Waited on by lgkmcnt, so it never has to drain the vector
// memory counter that tracks the K/V prefetch.  Every lane must pass the same p.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}
__device__ __forceinline__ int64_t load_uniform64(const int64_t* p) {
  return *(const __attribute__((address_space(4))) int64_t*)p;
}

// Zeros in device memory: the target of a kernel's prologue loads whose pointer argument
// is NULL, so that every per-sequence scalar can be loaded unconditionally (one memory
// round trip for all of them instead of a dependent chain through branches).
static __device__ const int64_t kZeroScalars[2] = {0, 0};

}  // namespace pa
