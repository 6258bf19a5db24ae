// Matrix-core issue probe: a measurement tool beside the library, not part of the attention
// path (built into its own libmfma_probe.so; nothing here is shared with the kernels).
//
// Each configuration launches 256 workgroups whose waves run a fixed loop of
// v_mfma_f32_32x32x16_bf16 (one or more independent accumulation chains), optionally with
// FMAs and exp2 instructions interleaved, and time their own loop with the shader cycle
// counter (s_memtime).  The figures it returns -- cycles per MFMA per SIMD, and for a wave
// that only runs VALU beside an MFMA wave its cycles per instruction -- are the issue rules
// the prefill kernel's schedule is measured against: a 32x32x16 bf16 MFMA occupies the
// matrix core for 32 cycles, a dependent chain issues slower than independent ones, and
// VALU work competes with the MFMAs of its own wave (less so with the accumulator in AGPRs)
// but little with those of the other wave of its SIMD.
//
// Waves w and w + 4 of a workgroup share a SIMD (checked with HW_ID on this GPU), so the
// split configurations give them different roles through (wave >> 2) & 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

namespace mp {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kIters = 2000;
constexpr int kBlocks = 256;

// CH independent MFMA chains; NV FMAs and NE exp2 after each MFMA; MODE 0: every wave runs
// MFMAs and VALU, MODE 1: waves 0-3 run only the MFMAs, waves 4-7 only the VALU work;
// AG: accumulators pinned to AGPRs (inline-asm MFMA) instead of the compiler's VGPR form.
template <int CH, int NV, int NE, int MODE, bool AG>
__global__ __launch_bounds__(512, 1) void probe_kernel(float* out, long long* cyc, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (i - lane));
  }
  f32x16 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.5f + 0.01f * (lane + i);
  const bool vrole = MODE == 1 && ((wave >> 2) & 1);
  const bool do_m = !vrole;
  const bool do_v = MODE == 0 || vrole;
  __syncthreads();
  auto mfma = [&](int c) {
    if constexpr (AG)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(a), "v"(b));
    else
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  };
  auto valu = [&]() {
#pragma unroll
    for (int k = 0; k < NV; ++k)
      asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(v[k & 7]) : "v"(v[(k + 1) & 7]), "v"(0.25f));
#pragma unroll
    for (int k = 0; k < NE; ++k) asm volatile("v_exp_f32 %0, %0" : "+v"(v[k & 7]));
  };
  // one loop per role, so that no branch sits between the instructions being timed
  const long long t0 = clock64();
  if (do_m && do_v) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        mfma(c);
        valu();
        __builtin_amdgcn_sched_barrier(0);
      }
  } else if (do_m) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        mfma(c);
        __builtin_amdgcn_sched_barrier(0);
      }
  } else {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        valu();
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  const long long t1 = clock64();
  if constexpr (AG) {
    // the inline-asm MFMAs are invisible to the compiler's hazard checks: let the last
    // one finish before the accumulators are read
#pragma unroll
    for (int c = 0; c < CH; ++c) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[c]));
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * (blockDim.x / 64) + wave] = t1 - t0;
}

struct Config {
  const char* label;
  int ch, nv, ne, mode, ag, wps;
  void (*kernel)(float*, long long*, int);
};

#define MP_CFG(label, CH, NV, NE, MODE, AG, WPS) \
  Config{label, CH, NV, NE, MODE, AG, WPS, probe_kernel<CH, NV, NE, MODE, AG>}

const Config kConfigs[] = {
    MP_CFG("1 wave/SIMD: 1 dependent chain", 1, 0, 0, 0, false, 1),
    MP_CFG("1 wave/SIMD: 2 independent chains", 2, 0, 0, 0, false, 1),
    MP_CFG("1 wave/SIMD: 4 independent chains", 4, 0, 0, 0, false, 1),
    MP_CFG("2 waves/SIMD: 1 dependent chain each", 1, 0, 0, 0, false, 2),
    MP_CFG("1 wave/SIMD: 4 chains + 4 FMA per MFMA, VGPR acc", 4, 4, 0, 0, false, 1),
    MP_CFG("1 wave/SIMD: 4 chains + 4 FMA per MFMA, AGPR acc", 4, 4, 0, 0, true, 1),
    MP_CFG("1 wave/SIMD: 4 chains + 8 FMA per MFMA, VGPR acc", 4, 8, 0, 0, false, 1),
    MP_CFG("1 wave/SIMD: 4 chains + 8 FMA per MFMA, AGPR acc", 4, 8, 0, 0, true, 1),
    MP_CFG("1 wave/SIMD: 4 chains + 4 exp2 per MFMA, AGPR acc", 4, 0, 4, 0, true, 1),
    MP_CFG("2 waves/SIMD: 4 chains + 8 FMA per MFMA each, VGPR acc", 4, 8, 0, 0, false, 2),
    MP_CFG("2 waves/SIMD: 4 chains + 8 FMA per MFMA each, AGPR acc", 4, 8, 0, 0, true, 2),
    MP_CFG("2 waves/SIMD: 4 chains + 3 FMA + 1 exp2 per MFMA each", 4, 3, 1, 0, false, 2),
    MP_CFG("MFMA-only wave beside a wave of 6 FMA + 2 exp2 per MFMA", 4, 6, 2, 1, false, 2),
    MP_CFG("MFMA-only wave beside a wave of 4 exp2 per MFMA", 4, 0, 4, 1, false, 2),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
}  // namespace mp

extern "C" {

int mfma_probe_count() { return mp::kNumConfigs; }

const char* mfma_probe_label(int i) { return (i >= 0 && i < mp::kNumConfigs) ? mp::kConfigs[i].label : nullptr; }

// Runs configuration i (a warm-up launch, then the timed one) on the current device.
// res[0]: cycles per MFMA per SIMD (the slowest MFMA-issuing wave's loop cycles over the
// MFMAs its SIMD issued); res[1]: cycles per VALU instruction of the VALU-only wave in the
// split configurations (-1 otherwise); res[2]: the configuration's waves per SIMD.
// Returns 0, -1 for a bad index, or the HIP error code.
int mfma_probe_run(int i, double* res) {
  using namespace mp;
  if (i < 0 || i >= kNumConfigs || res == nullptr) return -1;
  const Config& c = kConfigs[i];
  const int threads = 256 * c.wps;
  const int nwaves = kBlocks * threads / 64;
  float* out = nullptr;
  long long* cyc = nullptr;
  hipError_t e = hipMalloc(&out, sizeof(float) * kBlocks * threads);
  if (e == hipSuccess) e = hipMalloc(&cyc, sizeof(long long) * nwaves);
  std::vector<long long> h(nwaves);
  for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
    hipLaunchKernelGGL(c.kernel, dim3(kBlocks), dim3(threads), 0, 0, out, cyc, kIters);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h.data(), cyc, sizeof(long long) * nwaves, hipMemcpyDeviceToHost);
  if (out) (void)hipFree(out);
  if (cyc) (void)hipFree(cyc);
  if (e != hipSuccess) return (int)e;
  const int wpb = threads / 64;
  double mx_m = 0.0, mx_v = 0.0;
  for (int w = 0; w < nwaves; ++w) {
    const bool vrole = c.mode == 1 && (((w % wpb) >> 2) & 1);
    if (vrole)
      mx_v = std::max(mx_v, (double)h[w]);
    else
      mx_m = std::max(mx_m, (double)h[w]);
  }
  const int mfma_waves_per_simd = c.mode == 0 ? c.wps : 1;
  res[0] = mx_m / ((double)mfma_waves_per_simd * kIters * c.ch);
  res[1] = c.mode == 1 ? mx_v / ((double)kIters * c.ch * (c.nv + c.ne)) : -1.0;
  res[2] = c.wps;
  return 0;
}

}  // extern "C"
