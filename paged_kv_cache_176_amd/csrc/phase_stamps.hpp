// Phase stamps of the split-KV partial kernels: an instrumented build only (sources compiled
// with -DPA_PHASE_STAMPS into libpagedattn_stamps.so; the library the entry points ship in has
// none of this).  Every wave keeps up to 64 s_memrealtime readings (100 MHz) in one register,
// lane k holding stamp k, and stores them at its end to the kernel's stamp array at
// [(workgroup * waves per workgroup + wave) * 64 + k], workgroup = (z * gridDim.y + y) *
// gridDim.x + x (waves past kStampWaves are not kept):
//   0 entry, 1 ring prologue issued, 2 Q landed (the kernels that issue the ring first wait
//   for Q and the prologue's tiles together, so there 2 follows 1; the kernels that load Q
//   first issue the ring after Q's wait, so there 1 follows 2), 3 + 2i / 4 + 2i the
//   wave's i-th tile after its wait / after its compute (i < 27; later tiles overwrite the
//   27th), 58 tiles consumed, 59 XCC id, 60 loop end, 61 first epilogue barrier passed,
//   62 end, 63 HW_ID.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#ifdef PA_PHASE_STAMPS
namespace pa {
constexpr int kStampWaves = 1 << 14;
}
#define PA_STAMP_DECL uint32_t st_ = 0; int it_ = 0;
#define PA_STAMP(k)                                                            \
  {                                                                            \
    const uint32_t t_ = (uint32_t)__builtin_amdgcn_s_memrealtime();            \
    st_ = lane == (k) ? t_ : st_;                                              \
  }
#define PA_STAMP_TILE_WAITED PA_STAMP(3 + 2 * it_)
#define PA_STAMP_TILE_DONE                                                     \
  {                                                                            \
    PA_STAMP(4 + 2 * it_);                                                     \
    it_ = it_ < 27 ? it_ + 1 : it_;                                            \
  }
#define PA_STAMP_FLUSH(ARR, NWAVES)                                            \
  {                                                                            \
    PA_STAMP(62);                                                              \
    const uint32_t hw_ = __builtin_amdgcn_s_getreg((31 << 11) | 4);           \
    const uint32_t xcc_ = __builtin_amdgcn_s_getreg((31 << 11) | 20);         \
    st_ = lane == 63 ? hw_ : lane == 59 ? xcc_ : lane == 58 ? (uint32_t)it_ : st_; \
    const int64_t wg_ = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x; \
    const int64_t w_ = wg_ * (NWAVES) + wave;                                  \
    if (w_ < kStampWaves) ARR[w_ * 64 + lane] = st_;                           \
  }
#else
#define PA_STAMP_DECL
#define PA_STAMP(k)
#define PA_STAMP_TILE_WAITED
#define PA_STAMP_TILE_DONE
#define PA_STAMP_FLUSH(ARR, NWAVES)
#endif
