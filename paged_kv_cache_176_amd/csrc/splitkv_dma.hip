// Split-KV partial kernel with K/V streamed through LDS by direct global->LDS loads.
//
// Same contract as splitkv_partial_kernel (per (partition, KV head, sequence) one
// workgroup writes normalised partial outputs and log-sum-exp of every query row of
// the KV head) for bf16 rows: the packed K192/V128 DiffKV row and the shared 576-wide
// MLA latent row whose first 512 columns are V (vLLM PR #50371, "Purpose").
//
// Why LDS: a K operand loaded straight into MFMA lanes puts 4 lanes (64 bytes) on a
// row per load instruction, so a 128-byte line is split over two instructions; with
// the nontemporal hint that line is fetched twice, and without it the cached path
// tops out near 6 TB/s.  Here each global_load_lds_dwordx4 (16 B per lane, landing at
// LDS base + 16*lane) covers whole 128-byte lines of consecutive rows, issued with the
// nontemporal hint: the same streaming pattern measured near 6.9 TB/s.
//
// Each of the 4 waves streams its own 16-key tiles (wave w takes tiles w, w+4, ...)
// into a private LDS ring of NST stages.  Completion is tracked with explicit vmcnt
// waits (the compiler does not track LDS-DMA writes); the ring is wave-private, so no
// barrier is needed.  The loop issues no other vector-memory op: a tile's block id
// comes in by a scalar load, because any vector load waited on behind the DMA would
// drain the ring.
//   QK^T  S^T[16 keys x 16 rows] = K Q^T, v_mfma_f32_16x16x32_bf16, K operand from LDS
//         (ds_read_b128, XOR-swizzled chunks), Q in VGPRs.
//   PV    O^T[16 dims x 16 rows] += V^T P^T, v_mfma_f32_16x16x16_bf16; V^T from the SAME
//         tile by ds_read_b64_tr_b16.
// The waves' (m, l, acc) merge through LDS in a fixed order at the end.
#include "common.hpp"
#include "kernels.hpp"

namespace pa {
namespace sd {
constexpr int NW = 4;
constexpr int TT = 16;                 // keys per tile
}  // namespace sd

// chunk swizzle, as in the prefill kernel: conflict-free 16-byte reads for 8- and
// 16-lane LDS passes; depends on key bits 0-3 only
__device__ __forceinline__ int sd_swz(int key) { return ((key >> 1) ^ (key << 2)) & 7; }

// wait until at most N vector-memory ops of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DK, int DV, int VOFF, int NR, int NST, int MINW>
__global__ __launch_bounds__(sd::NW * 64, MINW) void splitkv_dma_kernel(SplitArgs a) {
  using namespace sd;
  constexpr int ROWB = (VOFF >= DK ? DK + DV : DK) * 2;   // bytes of a row that are read
  constexpr int CH = ROWB / 16;                           // 16-byte chunks per row
  constexpr int NINS = TT * CH / 64;                      // DMA instructions per tile
  constexpr int TILE_BYTES = TT * CH * 16;
  constexpr int KS = DK / 32;
  constexpr int DB = DV / 16;
  constexpr int ROWS = NR * 16;
  constexpr int MERGE_PITCH = DV + 4;
  constexpr int RING = NW * NST * TILE_BYTES;
  constexpr int MERGE = NW * ROWS * 2 * 4 + ROWS * MERGE_PITCH * 4;
  constexpr int LDS_BYTES = RING > MERGE ? RING : MERGE;
  static_assert(CH % 8 == 0 && (TT * CH) % 64 == 0, "row must be whole 128-byte groups");
  static_assert(VOFF % 8 == 0 && (VOFF >= DK || VOFF + DV <= DK), "V must be whole chunks of the row");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int P = a.num_partitions;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int S = a.seq_lens[b];
  const int q0 = a.qsl ? a.qsl[b] : b;
  const int L = a.qsl ? a.qsl[b + 1] - q0 : 1;
  const int chunk = ceil_div(ceil_div(S, P), TT) * TT;
  const int start = min(part * chunk, S);
  const int end = min(start + chunk, S);
  const int nt = ceil_div(end - start, TT);
  const int bs_shift = __builtin_ctz(a.c.block_size);
  const int bs_mask = a.c.block_size - 1;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;

  // ---- Q rows (B operand), visibility limits ----
  bf16x8 qreg[NR][KS];
  int hi[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const int r = rg * 16 + n;
    const int qi = r / G, hh = r - qi * G;
    const bool live = qi < L && qi < a.max_q;
    hi[rg] = live ? min(S - L + qi, end - 1) : -1;
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? qi : 0)) * a.q_st + (int64_t)(kvh * G + hh) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0, 0, 0, 0};
      if (live) w = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
      qreg[rg][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float sl2 = a.scale * kLog2e;

  // lane byte offsets inside a tile: K operand chunk 4ks+g of key n (per ks parity; the
  // rest of ks is an immediate) and the transposed V source (per 16-dim block, mod 4)
  const int sw = sd_swz(n);
  int koff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) koff[par] = (n * CH + ((4 * par + g) ^ sw)) * 16;
  int voff[4];
  {
    const int vkey = 4 * g + (n >> 2);
    const int vsw = sd_swz(vkey);
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
      const int ch = VOFF / 8 + 2 * d4 + ((n & 3) >> 1);   // chunk of dims 16*d4 + 4*(n&3)
      voff[d4] = (vkey * CH + ((ch & ~7) | ((ch & 7) ^ vsw))) * 16 + (n & 1) * 8;
    }
  }

  f32x4 acc[NR][DB];
  float m[NR], l[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    m[rg] = kNegInf;
    l[rg] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  char* ring = smem + wave * NST * TILE_BYTES;
  const uint8_t* head_base = a.c.data + (int64_t)kvh * a.c.sh * 2;
  // Q is complete in registers before the first DMA: the explicit vmcnt waits below
  // count DMA instructions only
  __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)

  auto issue = [&](int ti, int stage) {
    char* buf = ring + stage * TILE_BYTES;
    // block_size is a multiple of 16: the tile sits in one block, whose id is
    // wave-uniform and comes in by a scalar load (lgkmcnt, not the DMA's vmcnt)
    const int t0 = __builtin_amdgcn_readfirstlane(start + ti * TT);
    const int64_t blk = load_uniform(btrow + (t0 >> bs_shift));
    const uint8_t* tile = head_base + (blk * a.c.sb + (int64_t)(t0 & bs_mask) * a.c.ss) * 2;
    const int kmax = end - 1 - t0;                // keys past the partition re-read its last key
#pragma unroll
    for (int u = 0; u < NINS; ++u) {
      const int slot = u * 64 + lane;
      const int key = slot / CH;
      const int c = (slot - key * CH) ^ sd_swz(key);
      const uint8_t* src = tile + (int64_t)min(key, kmax) * a.c.ss * 2 + c * 16;
      dma16_nt(src, lds_addr(buf + u * 1024));
    }
  };

  auto compute = [&](int ti, int stage) {
    const char* buf = ring + stage * TILE_BYTES;
    const int j0 = start + ti * TT;
    f32x4 s[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) s[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(buf + koff[ks & 1] + (ks >> 1) * 128);
#pragma unroll
      for (int rg = 0; rg < NR; ++rg) s[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[rg][ks], s[rg], 0, 0, 0);
    }
    s16x4 pb[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      float x[4];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * g + i;
        x[i] = (j <= hi[rg]) ? s[rg][i] * sl2 : kNegInf;
        mx = fmaxf(mx, x[i]);
      }
      mx = max_over_groups(mx);
      const float mn = fmaxf(m[rg], mx);
      const float base = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[rg] - base);
      float p[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(x[i] - base);
        ps += p[i];
      }
      l[rg] = l[rg] * alpha + ps;
      m[rg] = mn;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rg][db] *= alpha;
      }
      u32x2 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      pb[rg] = __builtin_bit_cast(s16x4, pk);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const s16x4 vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(buf + voff[db & 3] + (db >> 2) * 128));
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        acc[rg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pb[rg], acc[rg][db], 0, 0, 0);
    }
  };

  // ---- this wave's tiles wave, wave+NW, ...: one consumed while up to NST-1 fly ----
  {
#pragma unroll
    for (int k = 0; k < NST - 1; ++k)
      if (wave + k * NW < nt) issue(wave + k * NW, k);
    int stage = 0;
    for (int ti = wave; ti < nt; ti += NW) {
      const int tn = ti + (NST - 1) * NW;        // tile to start now, into the slot freed last step
      if (tn < nt) issue(tn, (stage + NST - 1) % NST);
      // tiles issued after ti: min(NST-1, remaining) -> wait until only those are in flight
      const int later = min(NST - 1, (nt - 1 - ti) / NW);
      static_assert(NST <= 4, "waits below cover up to 3 tiles in flight");
      if (NST > 3 && later >= 3) wait_vm<(NST > 3 ? 3 : 0) * NINS>();
      else if (NST > 2 && later >= 2) wait_vm<(NST > 2 ? 2 : 0) * NINS>();
      else if (later >= 1) wait_vm<NINS>();
      else wait_vm<0>();
      compute(ti, stage);
      stage = (stage + 1) % NST;
    }
  }

  // ---- merge the NW waves through LDS in a fixed order, write the partials ----
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) l[rg] = sum_over_groups(l[rg]);
  __syncthreads();                                // rings are dead from here on
  float* mw = reinterpret_cast<float*>(smem);
  float* lw = mw + NW * ROWS;
  float* buf = lw + NW * ROWS;
  if (g == 0) {
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      mw[wave * ROWS + rg * 16 + n] = m[rg];
      lw[wave * ROWS + rg * 16 + n] = l[rg];
    }
  }
  __syncthreads();
  float f[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const int r = rg * 16 + n;
    float M = kNegInf;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * ROWS + r]);
    float Ls = 0.f;
    if (M != kNegInf)
      for (int w = 0; w < NW; ++w) Ls += lw[w * ROWS + r] * fast_exp2(mw[w * ROWS + r] - M);
    f[rg] = (M == kNegInf || Ls == 0.f) ? 0.f : fast_exp2(m[rg] - M) / Ls;
  }
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          f32x4* dst = reinterpret_cast<f32x4*>(buf + (rg * 16 + n) * MERGE_PITCH + db * 16 + 4 * g);
          const f32x4 v = acc[rg][db] * f[rg];
          if (w == 0) *dst = v;
          else *dst = *dst + v;
        }
    }
    __syncthreads();
  }
  const int64_t Hq = a.num_q_heads;
  for (int idx = threadIdx.x; idx < ROWS * (DV / 4); idx += NW * 64) {
    const int r = idx / (DV / 4), c4 = idx - r * (DV / 4);
    const int qi = r / G, hh = r - qi * G;
    if (qi >= L || qi >= a.max_q) continue;
    const int64_t tok = q0 + qi, head = kvh * G + hh;
    *reinterpret_cast<f32x4*>(a.part_out + ((tok * Hq + head) * P + part) * DV + c4 * 4) =
        *reinterpret_cast<const f32x4*>(buf + r * MERGE_PITCH + c4 * 4);
  }
  if (threadIdx.x < ROWS) {
    const int r = threadIdx.x;
    const int qi = r / G, hh = r - qi * G;
    if (qi < L && qi < a.max_q) {
      float M = kNegInf, Ls = 0.f;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * ROWS + r]);
      if (M != kNegInf)
        for (int w = 0; w < NW; ++w) Ls += lw[w * ROWS + r] * fast_exp2(mw[w * ROWS + r] - M);
      const int64_t tok = q0 + qi, head = kvh * G + hh;
      a.part_lse[(tok * Hq + head) * P + part] =
          (M == kNegInf || Ls == 0.f) ? kNegInf : (M + __builtin_log2f(Ls)) * kLn2;
    }
  }
}

// Eligible shapes: bf16 DiffKV rows (up to 32 rows per KV head) and bf16 MLA rows (one
// row group), with a power-of-two block size of at least 16.
static bool dma_is_diffkv(const SplitArgs& a) { return a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192; }
static bool dma_is_mla(const SplitArgs& a) { return a.c.dk == 576 && a.c.dv == 512 && a.c.v_off == 0; }

bool splitkv_dma_eligible(const SplitArgs& a) {
  const int bs = a.c.block_size;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int rows = a.max_q * G;
  if (a.c.esize != 2 || (bs & (bs - 1)) != 0 || bs < sd::TT) return false;
  return (dma_is_diffkv(a) && rows <= 32) || (dma_is_mla(a) && rows <= 16);
}

void launch_splitkv_dma(const SplitArgs& a, hipStream_t s) {
  dim3 grid(a.num_partitions, a.c.num_kv_heads, a.num_seqs), block(sd::NW * 64);
  const int rows = a.max_q * (a.num_q_heads / a.c.num_kv_heads);
  if (dma_is_mla(a))
    hipLaunchKernelGGL((splitkv_dma_kernel<576, 512, 0, 1, 2, 1>), grid, block, 0, s, a);
  else if (rows <= 16)
    hipLaunchKernelGGL((splitkv_dma_kernel<192, 128, 192, 1, 2, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((splitkv_dma_kernel<192, 128, 192, 2, 2, 2>), grid, block, 0, s, a);
}

}  // namespace pa
