// Split-KV partial kernel for 17..32 query rows per KV head over fp8 (E4M3FN)
// DiffKV rows: the multi-token verify shape, where the L tokens x G heads of a KV
// head share every K/V read (diffbot MiMo-V2.6-Flash model card, "What the kernels
// do": one program per whole verify; "Benchmarks": 4 tokens x 8 heads = 32 rows).
//
// Same contract as the other split-KV partial kernels: per (partition, KV head,
// sequence) one workgroup writes the normalised partial output and log-sum-exp of
// every query row of the KV head over the partition's keys (partitions are cut at
// 16-key granularity, as everywhere).
//
// With 32 rows the whole row set is one 32x32 MFMA operand, so each wave works on
// 32-key tiles:
//   QK^T  S^T[32 keys x 32 rows] += K[32 keys x 16 dims] Q^T, v_mfma_f32_32x32x16_bf16,
//         12 k-steps.  The A-operand row m reads key pi(m), a permutation chosen so
//         that each lane's 16 scores are two runs of 8 consecutive keys.
//   softmax each lane holds 16 of its row's 32 keys; the other 16 sit 32 lanes away
//         (one v_permlane32_swap for the max).  Lazy rescaling as in the other kernels.
//   PV    O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] P^T, 8 MFMAs per tile.  The
//         V^T operand is one ds_read_b64_tr_b8 per lane (8 consecutive keys of one
//         dim, straight from the fp8 tile) converted to bf16 in registers.
// fp8 -> bf16 conversion is exact; the K scale multiplies the scores, the V scale
// the output.  K/V tiles (32 rows x 320 B) stream into a per-wave LDS ring by
// nontemporal global_load_lds_dwordx4 covering whole 128-byte lines; a 4-chunk XOR
// swizzle by key keeps the 8-lane K reads and the 16-lane transposing reads
// conflict-free on the 20-chunk row pitch.
#include "common.hpp"
#include "kernels.hpp"
#include "phase_stamps.hpp"

namespace pa {
#ifdef PA_PHASE_STAMPS
__device__ uint32_t g_phase_stamps_wide[kStampWaves * 64];   // this kernel's stamps (phase_stamps.hpp)
#endif
namespace sw {
constexpr int TT = 32;       // keys per tile
constexpr int DK = 192, DV = 128;
constexpr int CH = 20;       // 16-byte chunks per 320-byte row (K 0..11, V 12..19)
constexpr int TILE_BYTES = TT * CH * 16;
constexpr int NINS = TILE_BYTES / 1024;   // DMA instructions per tile (10: 5 per 16-key half)
constexpr int KS = DK / 16;  // 32x32x16 k-steps
constexpr int DBW = DV / 32; // 32-dim output blocks
}  // namespace sw

__device__ __forceinline__ int sw_swz(int key) { return ((key >> 2) ^ (key >> 1)) & 3; }
__device__ __forceinline__ int sw_pos(int chunk, int key) { return (chunk & ~3) | ((chunk & 3) ^ sw_swz(key)); }
// A-operand row m of the QK^T MFMA holds key pi(m)
__device__ __forceinline__ int sw_pi(int m) {
  const int q = m >> 3, gp = (m >> 2) & 1, r = m & 3;
  return 16 * (q >> 1) + 8 * gp + 4 * (q & 1) + r;
}

// 8 fp8 bytes (two dwords) -> bf16x8
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const u32x2 a = fp8x4_to_bf16x4(lo), b = fp8x4_to_bf16x4(hi);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// NW waves per workgroup, interleaved over 32-key tiles; NST-stage ring per wave
template <int NW, int NST, int MINW>
__global__ __launch_bounds__(NW * 64, MINW) void splitkv_wide_fp8_kernel(SplitArgs a) {
  using namespace sw;
  constexpr int ROWS = 32;
  constexpr int MERGE_PITCH = DV + 4;
  constexpr int RING = NW * NST * TILE_BYTES;
  constexpr int MERGE = NW * ROWS * 2 * 4 + NW * ROWS * MERGE_PITCH * 4;
  constexpr int LDS_BYTES = RING > MERGE ? RING : MERGE;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;        // MFMA column (query row) and k-group
  const int P = a.num_partitions;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  PA_STAMP_DECL
  PA_STAMP(0)
  // the per-sequence scalars in one round trip (a NULL qsl reads zeros)
  const int32_t* qslp = a.qsl ? a.qsl + b : reinterpret_cast<const int32_t*>(kZeroScalars);
  const int S = load_uniform(a.seq_lens + b);
  const int qs0 = load_uniform(qslp), qs1 = load_uniform(qslp + 1);
  const int q0 = a.qsl ? qs0 : b;
  const int L = a.qsl ? qs1 - qs0 : 1;
  const int chunk = ceil_div(ceil_div(S, active_splits(a.pol, S, P)), 16) * 16;
  const int start = min(part * chunk, S);
  const int end = min(start + chunk, S);
  const int nt = ceil_div(end - start, TT);
  const int bs_shift = __builtin_ctz(a.c.block_size);
  const int bs_mask = a.c.block_size - 1;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;
  if (nt == 0) {                                 // an empty key range: empty partials at once
    write_empty_partials<true>(a, q0, 0, min(min(L, a.max_q), ROWS / G), G, kvh, part, DV, NW * 64);
    PA_STAMP_FLUSH(g_phase_stamps_wide, NW)
    return;
  }

  // ---- per-lane LDS offsets ----
  // K: lane (m = n, g) reads chunk 2j + g of key pi(n); j even/odd differ in bit 1 of
  // the chunk, the rest of j is an immediate (64 bytes per 4 chunks)
  const int kkey = sw_pi(n);
  int koff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) koff[par] = (kkey * CH + sw_pos(2 * par + g, kkey)) * 16;
  // V (transposing 8-bit read): 16-lane group gi = lane/16 covers dims 16*(gi&1) of a
  // 32-dim block and keys 8*(gi>>1) of a 16-key half; source lane s of the group
  // addresses key +(s>>1), bytes 8*(s&1) of its 16-dim chunk
  int voff[2];
  {
    const int gi = lane >> 4, s = lane & 15;
    const int vkey = 8 * (gi >> 1) + (s >> 1);
#pragma unroll
    for (int par = 0; par < 2; ++par)
      voff[par] = (vkey * CH + sw_pos(12 + 2 * par + (gi & 1), vkey)) * 16 + 8 * (s & 1);
  }
  // DMA: slot u*64 + lane of a tile holds chunk (slot % 20) ^ swizzle of key slot / 20;
  // instructions 0-4 cover keys 0-15, 5-9 keys 16-31 (one 16-key group each)
  const int ssb = (int)a.c.ss;                   // bytes between consecutive slots (fp8)
  int dkey[NINS], dbyte[NINS];
#pragma unroll
  for (int u = 0; u < NINS; ++u) {
    const int slot = u * 64 + lane;
    const int kt = slot / CH;
    dkey[u] = kt;
    dbyte[u] = sw_pos(slot - kt * CH, kt) * 16;
  }

  char* ring = smem + wave * NST * TILE_BYTES;
  const uint8_t* head_base = a.c.data + (int64_t)kvh * a.c.sh;

  auto group_base = [&](int j) {                 // first row of the 16-key group at key j
    const int64_t blk = load_uniform(btrow + (j >> bs_shift));
    return head_base + blk * a.c.sb + (int64_t)(j & bs_mask) * a.c.ss;
  };
  auto issue = [&](int ti, int stage) {
    char* buf = ring + stage * TILE_BYTES;
    const int t0 = __builtin_amdgcn_readfirstlane(start + ti * TT);
    if (t0 + TT - 1 <= end - 1) {                // whole tile inside the partition
      const uint8_t* base0 = group_base(t0);
      const uint8_t* base1 = group_base(t0 + 16);
#pragma unroll
      for (int u = 0; u < NINS; ++u)
        dma16_nt_s((dkey[u] & 15) * ssb + dbyte[u], u < NINS / 2 ? base0 : base1, lds_addr(buf + u * 1024));
    } else {                                      // keys past the partition re-read its last key
      const int last = end - 1;
      const int g0 = t0, g1 = min(t0 + 16, last & ~15);
      const uint8_t* base0 = group_base(g0);
      const uint8_t* base1 = group_base(g1);
#pragma unroll
      for (int u = 0; u < NINS; ++u) {
        const int gs = u < NINS / 2 ? g0 : g1;
        const int j = min(t0 + dkey[u], last);
        dma16_nt_s((j - gs) * ssb + dbyte[u], u < NINS / 2 ? base0 : base1, lds_addr(buf + u * 1024));
      }
    }
  };

  // ---- Q row n (B operand): k-step ks holds dims 32(ks/2) + 16g + 8(ks%2) .. +8, the
  // order in which one 16-byte fp8 chunk of K feeds two k-steps ----
  const int qi = n / G, hh = n - qi * G;
  const bool live = qi < L && qi < a.max_q;
  const int hi = live ? min(S - L + qi, end - 1) : -1;   // last key row n sees here
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? qi : 0)) * a.q_st + (int64_t)(kvh * G + hh) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0, 0, 0, 0};
      if (live) w = *reinterpret_cast<const u32x4*>(qp + 32 * (ks >> 1) + 16 * g + 8 * (ks & 1));
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  float kscale = 1.0f, vscale = 1.0f;
  if (a.c.scale_mode != 0) {
    kscale = a.c.scale_mode == 2 ? a.c.k_scale[kvh] : a.c.k_scale[0];
    vscale = a.c.scale_mode == 2 ? a.c.v_scale[kvh] : a.c.v_scale[0];
  }
  float sl2 = a.scale * kLog2e * kscale;
  if (sl2 < 0.f) {                               // s * sl2 == (-s) * (-sl2): negate Q (exact)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qreg[ks]) ^ 0x80008000u);
    sl2 = -sl2;
  }
  // a zero scale would meet masked (-inf) scores as -inf * 0 = NaN; the smallest
  // normal scale gives the same uniform weights to within fp32 rounding
  sl2 = fmaxf(sl2, 1.17549435e-38f);
  // last key every live row sees: tiles ending at or before it need no mask
  // (the live rows' limits min(S - L + qi, end - 1) are smallest for token 0, whose rows
  // are always here)
  const int vis_hi = min(L, a.max_q) > 0 ? min(S - L, end - 1) : 0x7fffffff;

  f32x16 acc[DBW];
#pragma unroll
  for (int db = 0; db < DBW; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = kNegInf, l = 0.f;

  // Q and the scales are complete from here on: the compiler, which counts only the loads
  // it issued, sees this wait and adds none of its own for them.  Only then is the ring
  // issued -- every stage before the first tile is waited for, so the opening burst requests
  // NST tiles per wave -- and the loop's explicit waits, which count DMA instructions only,
  // let tile 0 be computed as soon as it lands.  (Issued before Q, the ring made this
  // vmcnt(0) wait for all NST prologue tiles: the call was 4% slower.)
  __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)
  PA_STAMP(2)                                    // Q landed
#pragma unroll
  for (int k = 0; k < NST; ++k)
    if (wave + k * NW < nt) issue(wave + k * NW, k);
  PA_STAMP(1)                                    // ring prologue issued

  auto compute = [&](int ti, int stage) {
    const char* buf = ring + stage * TILE_BYTES;
    const int j0 = start + ti * TT;
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KS / 2; ++j) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(buf + koff[j & 1] + (j >> 1) * 64);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(w[0], w[1]), qreg[2 * j], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(w[2], w[3]), qreg[2 * j + 1], s, 0, 0, 0);
    }
    // lane element i is key j0 + 16*(i/8) + 8g + i%8 of row n
    const bool nomask = j0 + TT - 1 <= vis_hi;
    float mx = kNegInf;
    if (nomask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = j0 + 16 * (i >> 3) + 8 * g + (i & 7);
        s[i] = key <= hi ? s[i] : kNegInf;
        mx = fmaxf(mx, s[i]);
      }
    }
    {
      float x = mx, y = mx;
      swap_rows32(x, y);
      mx = fmaxf(x, y) * sl2;                    // sl2 > 0; -inf stays -inf
    }
    // lazy rescaling: the exp2 base moves only when the max grows by more than 8
    const float mn = fmaxf(m, mx);
    const bool grow = mn > m + 8.0f;             // true on the first visible key (m = -inf)
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m - mn) : 1.0f;
      m = grow ? mn : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DBW; ++db) acc[db] *= alpha;
    }
    const float nbase = m == kNegInf ? 0.f : -m;
    uint32_t pk[8];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // masked scores are -inf: fma(-inf, sl2 > 0, .) = -inf -> p = 0
      const float p0 = fast_exp2(__builtin_fmaf(s[2 * i], sl2, nbase));
      const float p1 = fast_exp2(__builtin_fmaf(s[2 * i + 1], sl2, nbase));
      ps += p0 + p1;
      pk[i] = pack_bf16x2(p0, p1);
    }
    l += ps;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]});
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(buf + voff[db & 1] + (db >> 1) * 64 + kk * 16 * CH * 16));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(v[0], v[1]), pb, acc[db], 0, 0, 0);
      }
    }
  };

  // ---- this wave's tiles wave, wave+NW, ...: one consumed while up to NST-1 fly ----
  {
    int stage = 0;
    for (int ti = wave; ti < nt; ti += NW) {
      const int tn = ti + (NST - 1) * NW;        // the first step's tile came with the prologue
      if (ti != wave && tn < nt) issue(tn, (stage + NST - 1) % NST);
      const int later = min(NST - 1, (nt - 1 - ti) / NW);
      static_assert(NST <= 3, "waits below cover up to 2 tiles in flight");
      if (NST > 2 && later >= 2) wait_vm<(NST > 2 ? 2 : 0) * NINS>();
      else if (later >= 1) wait_vm<NINS>();
      else wait_vm<0>();
      PA_STAMP_TILE_WAITED
      compute(ti, stage);
      PA_STAMP_TILE_DONE
      stage = (stage + 1) % NST;
    }
  }

  // ---- merge the NW waves: each writes its scaled accumulator to its own LDS slab
  // (independent stores, no read-modify-write chain), then all threads sum the slabs
  // in wave order and write the partials of the live rows ----
  PA_STAMP(60)
  {
    float x = l, y = l;                          // row n's two halves of the keys
    swap_rows32(x, y);
    l = x + y;
  }
  __syncthreads();                               // rings are dead from here on
  PA_STAMP(61)
  float* mw = reinterpret_cast<float*>(smem);    // [NW][ROWS]
  float* lw = mw + NW * ROWS;                    // [NW][ROWS]
  float* slab = lw + NW * ROWS;                  // [NW][ROWS][MERGE_PITCH]
  if (g == 0) {
    mw[wave * ROWS + n] = m;
    lw[wave * ROWS + n] = l;
  }
  __syncthreads();
  float M = kNegInf;
  for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * ROWS + n]);
  float Ls = 0.f;
  if (M != kNegInf)
    for (int w = 0; w < NW; ++w) Ls += lw[w * ROWS + n] * fast_exp2(mw[w * ROWS + n] - M);
  const float f = (M == kNegInf || Ls == 0.f) ? 0.f : fast_exp2(m - M) / Ls * vscale;
#pragma unroll
  for (int db = 0; db < DBW; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)                  // acc[db][4q + r] is dim 32db + 8q + 4g + r of row n
      *reinterpret_cast<f32x4*>(slab + (wave * ROWS + n) * MERGE_PITCH + 32 * db + 8 * q + 4 * g) =
          f32x4{acc[db][4 * q], acc[db][4 * q + 1], acc[db][4 * q + 2], acc[db][4 * q + 3]} * f;
  __syncthreads();
  const int64_t Hq = a.num_q_heads;
  const int live_rows = min(min(L, a.max_q) * G, ROWS);   // row r is live iff r / G < min(L, max_q)
  for (int idx = threadIdx.x; idx < live_rows * (DV / 4); idx += NW * 64) {
    const int r = idx / (DV / 4), c4 = idx - r * (DV / 4);
    const int rq = r / G, rh = r - rq * G;
    const int64_t tok = q0 + rq, head = kvh * G + rh;
    f32x4 v = *reinterpret_cast<const f32x4*>(slab + r * MERGE_PITCH + c4 * 4);
    for (int w = 1; w < NW; ++w) v += *reinterpret_cast<const f32x4*>(slab + (w * ROWS + r) * MERGE_PITCH + c4 * 4);
    store_partial4<true>(a.part_out + ((tok * Hq + head) * P + part) * DV + c4 * 4, v);
  }
  if (threadIdx.x < ROWS) {
    const int r = threadIdx.x;
    const int rq = r / G, rh = r - rq * G;
    if (rq < L && rq < a.max_q) {
      float Mx = kNegInf, Lx = 0.f;
      for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, mw[w * ROWS + r]);
      if (Mx != kNegInf)
        for (int w = 0; w < NW; ++w) Lx += lw[w * ROWS + r] * fast_exp2(mw[w * ROWS + r] - Mx);
      const int64_t tok = q0 + rq, head = kvh * G + rh;
      store_partial1<true>(a.part_lse + (tok * Hq + head) * P + part,
                     (Mx == kNegInf || Lx == 0.f) ? kNegInf : (Mx + __builtin_log2f(Lx)) * kLn2);
    }
  }
  PA_STAMP_FLUSH(g_phase_stamps_wide, NW)
}

// fp8 DiffKV rows with 17..32 query rows per KV head, power-of-two block size >= 16.
bool splitkv_wide_eligible(const SplitArgs& a) {
  const int bs = a.c.block_size;
  const int rows = a.max_q * (a.num_q_heads / a.c.num_kv_heads);
  return a.c.esize == 1 && a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192 && (bs & (bs - 1)) == 0 &&
         bs >= 16 && rows > 16 && rows <= 32;
}

void launch_splitkv_wide(const SplitArgs& a, hipStream_t s) {
  constexpr int NW = 4;
  dim3 grid(a.num_partitions, a.c.num_kv_heads, a.num_seqs), block(NW * 64);
  hipLaunchKernelGGL((splitkv_wide_fp8_kernel<NW, 2, 2>), grid, block, 0, s, a);
}

}  // namespace pa

#ifdef PA_PHASE_STAMPS
// The fp8 verify kernel's stamps (layout in phase_stamps.hpp): copies the first `words`
// (at most kStampWaves * 64) to host memory `dst`; returns the hipError_t of the copy.
extern "C" int attn_phase_stamps_read_wide(void* dst, size_t words) {
  if (!dst || words > (size_t)pa::kStampWaves * 64) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(pa::g_phase_stamps_wide), words * 4, 0, hipMemcpyDeviceToHost);
}
#endif
