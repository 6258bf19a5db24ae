// Split-KV partial kernel for multi-token verify over the MLA latent row: the waves of a
// workgroup share one LDS ring of K/V tiles, two waves per query token.
//
// Same contract as the other split-KV partial kernels (per (partition, KV head,
// sequence) normalised partial outputs and log-sum-exps of the KV head's query rows over
// the partition's keys).  Shape served: the 576-wide bf16 latent row whose first 512
// columns are V (vLLM PR #50371, "Purpose"), 2 or more query tokens per sequence with up
// to 16 query heads per KV head -- the multi-token verify of the 12-head MLA model, which
// the single-token MLA path of that PR leaves to another kernel (PR #50371, review thread).
//
// Why per token: a 16-row MFMA tile holds one token's (up to) 16 heads, and its 512-wide
// fp32 output accumulator alone takes 128 registers per lane, so a wave cannot hold the
// rows of several tokens.  The tokens of a sequence see the same keys (each up to its own
// causal limit), so the K/V rows are read from HBM once per workgroup into a shared ring
// and reused from LDS by every token.  A workgroup takes up to 4 tokens with 8 waves:
// wave (token t, half h) consumes the 32-key tiles 2j + h, so the two waves of a token
// split the keys (no score or accumulator is computed twice) and each SIMD runs two waves.
// At the end the two halves of a token merge through LDS and the token's rows are written
// straight out.  Longer drafts take more workgroups along grid y (each reading the K/V
// again).
//
// Ring: 4 stages of one 32-key tile (36 KB): step j covers tiles 2j and 2j + 1; each
// tile's direct global->LDS loads are shared by the 4 waves of its half (9 instructions
// each: a wave's share lies in one 16-key half, hence in one block).  A wave waits for its
// own share, one workgroup barrier per step publishes the step's tiles and frees the
// stages of the step before, which the same step refills with step j + 1: each wave
// issues its share after the third k-step of its QK^T chains, so that the loads have
// nearly the whole step to land (issued between QK^T and PV, they had only the PV's time
// and the next step waited for them) while the 8 waves' loads still do not all queue at
// the barrier.
//   QK^T  S^T[16 keys x 16 rows] = K Q^T per 16-key half (two independent MFMA chains),
//         v_mfma_f32_16x16x32_bf16, K from LDS (ds_read_b128, XOR-swizzled chunks).
//   PV    O^T[16 dims x 16 rows] += V^T P^T over the 32 keys at once,
//         v_mfma_f32_16x16x32_bf16; V^T by two ds_read_b64_tr_b16 (keys 4g..4g+3 of each
//         16-key half), P^T in the same key order.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_layout.hpp"
#include "phase_stamps.hpp"

namespace pa {
#ifdef PA_PHASE_STAMPS
__device__ uint32_t g_phase_stamps_tokens[kStampWaves * 64];   // this kernel's stamps (phase_stamps.hpp)
#endif
namespace stk {
constexpr int NTOK = 4;                // query tokens per workgroup
constexpr int NW = 2 * NTOK;           // waves: two per token
constexpr int TT = 32;                 // keys per tile
constexpr int NST = 4;                 // ring stages (two steps of two tiles)
constexpr int DK = 576, DV = 512;      // latent row; V = its first DV columns
}  // namespace stk

// The ring rows (1152 bytes) use lds_layout.hpp's row_chunk_swz: it depends on the row mod
// 16 only, so both 16-key halves of a tile share it.

__global__ __launch_bounds__(stk::NW * 64, 1) void splitkv_tokens_kernel(SplitArgs a) {
  using namespace stk;
  constexpr int ROWB = DK * 2;                     // 1152 bytes per row
  constexpr int CH = ROWB / 16;                    // 72 chunks per row
  constexpr int NINS = TT * CH / 64;               // DMA instructions per tile (36)
  constexpr int SHARE = NINS / NTOK;               // per wave of the tile's half (9)
  constexpr int TILE_BYTES = TT * ROWB;
  constexpr int KS = DK / 32;
  constexpr int DB = DV / 16;
  constexpr int SLAB_PITCH = DV + 4;               // floats per row of the end-merge slab
  static_assert(SHARE * 64 * 2 == 16 * CH, "two waves' shares cover one 16-key half");
  static_assert(NTOK * 16 * SLAB_PITCH * 4 + NTOK * 32 * 4 <= NST * TILE_BYTES, "end merge fits the ring");
  __shared__ __attribute__((aligned(16))) char ring[NST * TILE_BYTES];

  const int part = blockIdx.x, b = blockIdx.z;
  const int TG = ceil_div(a.max_q, NTOK);          // token groups per KV head
  const int kvh = blockIdx.y / TG, tg = blockIdx.y - kvh * TG;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int tw = wave & (NTOK - 1), h = wave / NTOK;   // token slot, key half
  PA_STAMP_DECL
  PA_STAMP(0)
  const int P = a.num_partitions;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  // the per-sequence scalars in one round trip (a NULL qsl reads zeros)
  const int32_t* qslp = a.qsl ? a.qsl + b : reinterpret_cast<const int32_t*>(kZeroScalars);
  const int S = load_uniform(a.seq_lens + b);
  const int qs0 = load_uniform(qslp), qs1 = load_uniform(qslp + 1);
  const int q0 = a.qsl ? qs0 : b;
  const int L = a.qsl ? qs1 - qs0 : 1;
  const int Lq = min(L, a.max_q);
  if (tg * NTOK >= Lq) {                           // no token of this sequence here (uniform)
    PA_STAMP_FLUSH(g_phase_stamps_tokens, NW)
    return;
  }
  const int chunk = ceil_div(ceil_div(S, active_splits(a.pol, S, P)), 16) * 16;
  const int start = min(part * chunk, S);
  const int end = min(start + chunk, S);
  const int nt = ceil_div(end - start, TT);
  if (nt == 0) {                                 // an empty key range: empty partials at once
    write_empty_partials<true>(a, q0, tg * NTOK, min(NTOK, Lq - tg * NTOK), G, kvh, part, DV, NW * 64);
    PA_STAMP_FLUSH(g_phase_stamps_tokens, NW)
    return;
  }
  const int nsteps = ceil_div(nt, 2);
  const int bs_shift = __builtin_ctz(a.c.block_size);
  const int bs_mask = a.c.block_size - 1;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;
  const int t = tg * NTOK + tw;                    // this wave's token
  const bool live = t < Lq;
  const int hi = live ? min(S - L + t, end - 1) : -1;   // last key the token sees here

  const uint8_t* head_base = a.c.data + (int64_t)kvh * a.c.sh * 2;
  const int ssb = (int)(a.c.ss * 2);
  // this wave's share of tile k (a tile of half h): instructions tw*SHARE .. +SHARE, all
  // in the 16-key half r0 = 16*(tw/2) of the tile, which sits in one block (block sizes
  // are powers of two >= 16).  Keys past the partition re-read its last key, whose block
  // is the one looked up then (never used: past every token's limit).
  auto issue = [&](int k) {
    char* buf = ring + (k & (NST - 1)) * TILE_BYTES;
    const int t0 = __builtin_amdgcn_readfirstlane(start + k * TT);
    const int kmax = end - 1 - t0;
    const int r0 = min(16 * (tw >> 1), kmax);
    const int64_t blk = load_uniform(btrow + ((t0 + r0) >> bs_shift));
    const uint8_t* base = head_base + (blk * a.c.sb + (int64_t)((t0 + r0) & bs_mask) * a.c.ss) * 2;
    // the lane index passes through an empty asm so that the share's offsets are computed
    // here, at each issue, instead of being hoisted and held in registers for the whole
    // loop (which spilled, and left the QK^T loop no registers to read ahead)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < SHARE; ++i) {
      const int u = tw * SHARE + i;
      const int slot = u * 64 + ln;
      const int key = slot / CH;
      const int c = (slot - key * CH) ^ row_chunk_swz(key);
      dma16_nt_s((uint32_t)((min(key, kmax) - r0) * ssb + c * 16), base, lds_addr(buf + u * 1024));
    }
  };

  // ---- the token's Q rows (B operand; heads >= G are zero rows) ----
  bf16x8 qreg[KS];
  {
    const bool row = live && n < G;
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? t : 0)) * a.q_st + (int64_t)(kvh * G + (row ? n : 0)) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {              // dead rows read a live row, then zero it
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
      qreg[ks] = __builtin_bit_cast(bf16x8, row ? w : u32x4{0, 0, 0, 0});
    }
  }
  float sl2 = a.scale * kLog2e;
  if (sl2 < 0.f) {                                 // s * sl2 == (-s) * (-sl2): negate Q (exact)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qreg[ks]) ^ 0x80008000u);
    sl2 = -sl2;
  }

  // lane byte offsets inside a tile: K operand chunk 4ks+g of key n (per ks parity; the
  // rest of ks is an immediate) and the transposed V source (per 16-dim block, mod 4);
  // the second 16-key half is 16 rows further
  const int sw = row_chunk_swz(n);
  int koff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) koff[par] = (n * CH + ((4 * par + g) ^ sw)) * 16;
  int voff[4];
  {
    const int vkey = 4 * g + (n >> 2);
    const int vsw = row_chunk_swz(vkey);
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
      const int ch = 2 * d4 + ((n & 3) >> 1);      // chunk of dims 16*d4 + 4*(n&3)
      voff[d4] = (vkey * CH + ((ch & ~7) | ((ch & 7) ^ vsw))) * 16 + (n & 1) * 8;
    }
  }
  constexpr int HALF = 16 * ROWB;

  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;
  // Q is complete from here on (the compiler, which does not count the DMA, sees this wait
  // and adds none of its own for Q).  Only then goes the prologue -- steps 0 and 1 (tiles
  // 0..3), each wave its share of its half's tiles -- so that step 0 waits for its own
  // share alone, not for step 1's as well (issued before Q, the prologue made this
  // vmcnt(0) wait for both: the B1 call was 3% slower)
  __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
  PA_STAMP(2)                                       // Q landed
  for (int k = h; k < min(NST, nt); k += 2) issue(k);
  PA_STAMP(1)                                       // ring prologue issued

  // tile k, and this wave's share of tile kn (kn < 0: none) issued after k-step
  // kIssueStep of the QK^T chains (MLA verify B1 call -3%, B16 kernel -1.4% against the
  // issue after the last k-step; issuing right after the barrier: -3% and -0.6%)
  constexpr int kIssueStep = 2;
  auto compute = [&](int k, int kn) {
    const char* buf = ring + (k & (NST - 1)) * TILE_BYTES;
    const int j0 = start + k * TT;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    // the K operands are read KPF k-steps ahead of their MFMAs, and a scheduling barrier
    // after each k-step keeps that order (left to itself the compiler reads each operand
    // right before its MFMA, and the two dependent chains wait on every LDS read)
    constexpr int KPF = 2;
    bf16x8 kb0[KPF + 1], kb1[KPF + 1];
#pragma unroll
    for (int j = 0; j < KPF; ++j) {
      kb0[j] = *reinterpret_cast<const bf16x8*>(buf + koff[j & 1] + (j >> 1) * 128);
      kb1[j] = *reinterpret_cast<const bf16x8*>(buf + HALF + koff[j & 1] + (j >> 1) * 128);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int jn = ks + KPF;
      if (jn < KS) {
        kb0[jn % (KPF + 1)] = *reinterpret_cast<const bf16x8*>(buf + koff[jn & 1] + (jn >> 1) * 128);
        kb1[jn % (KPF + 1)] = *reinterpret_cast<const bf16x8*>(buf + HALF + koff[jn & 1] + (jn >> 1) * 128);
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb0[ks % (KPF + 1)], qreg[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb1[ks % (KPF + 1)], qreg[ks], s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks == kIssueStep && kn >= 0) issue(kn);  // the refill: behind three k-steps
    }
    // lane (n, g): keys j0 + 4g + i (s0) and j0 + 16 + 4g + i (s1) of row n.  A tile the
    // token sees whole needs no mask, and the scale folds into one fma
    const bool nomask = j0 + TT - 1 <= hi;
    float x[8];
    float mx = kNegInf;
    if (nomask) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = max_over_groups(mx) * sl2;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (j0 + 4 * g + i <= hi) ? s0[i] * sl2 : kNegInf;
        x[4 + i] = (j0 + 16 + 4 * g + i <= hi) ? s1[i] * sl2 : kNegInf;
        mx = fmaxf(mx, fmaxf(x[i], x[4 + i]));
      }
      mx = max_over_groups(mx);
    }
    // lazy rescaling: the exp2 base moves only when the tile's max exceeds it by more
    // than 8 (log2 units); (m, l, acc) stay consistent throughout
    const float mn = fmaxf(m, mx);
    const bool grow = mn > m + 8.0f;               // true on the first visible key (m = -inf)
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m - mn) : 1.0f;
      m = grow ? mn : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float base = (m == kNegInf) ? 0.f : m;
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(nomask ? __builtin_fmaf(s0[i], sl2, -base) : x[i] - base);
      p[4 + i] = fast_exp2(nomask ? __builtin_fmaf(s1[i], sl2, -base) : x[4 + i] - base);
      ps += p[i] + p[4 + i];
    }
    l += ps;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                                       pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
    // V^T operands read three MFMAs ahead behind a scheduling barrier per MFMA (the compiler's
    // own order read one ahead, so every PV MFMA waited most of an LDS round trip: B16 kernel
    // -2% in paired runs, same registers)
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    auto vread = [&](int db) -> bf16x8 {
      const char* vp = buf + voff[db & 3] + (db >> 2) * 128;     // +64 dims per 4 blocks
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + HALF));
      return __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    };
    constexpr int VPF = 3;
    bf16x8 vq[VPF + 1];
#pragma unroll
    for (int q = 0; q < VPF; ++q) vq[q] = vread(q);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + VPF < DB) vq[(db + VPF) % (VPF + 1)] = vread(db + VPF);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vq[db % (VPF + 1)], pb, acc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- steps: wait for this wave's share of its tile, a barrier publishes the step (and
  // frees the stages of the step before, refilled here with step j + 1), every live wave
  // consumes its tile of the step ----
  for (int j = 0; j < nsteps; ++j) {
    const int k = 2 * j + h;                       // this wave's tile
    if (j == 0 && h + 2 < nt) wait_vm<SHARE>();   // step 0's share landed; step 1's may fly
    else wait_vm<0>();                             // the share issued at step j - 1 (or the prologue's)
    __syncthreads();
    PA_STAMP_TILE_WAITED
    const int kn = 2 * (j + 1) + h;
    const bool refill = j >= 1 && kn < nt;
    if (live && k < nt) compute(k, refill ? kn : -1);
    else if (refill) issue(kn);
    PA_STAMP_TILE_DONE
  }

  // ---- the token's two halves merge through LDS: half 1 leaves (m, l, acc), half 0
  // combines them and writes the normalised partial and log-sum-exp ----
  PA_STAMP(60)
  l = sum_over_groups(l);
  __syncthreads();                                 // the ring is free from here on
  PA_STAMP(61)
  float* slab = reinterpret_cast<float*>(ring) + tw * 16 * SLAB_PITCH;
  float* ml = reinterpret_cast<float*>(ring) + NTOK * 16 * SLAB_PITCH + tw * 32;
  if (h == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(slab + n * SLAB_PITCH + db * 16 + 4 * g) = acc[db];
    if (g == 0) {
      ml[n] = m;
      ml[16 + n] = l;
    }
  }
  __syncthreads();
  if (h == 0 && live && n < G) {
    const float m1 = ml[n], l1 = ml[16 + n];
    const float M = fmaxf(m, m1);
    const float a0 = M == kNegInf ? 0.f : fast_exp2(m - M);
    const float a1 = M == kNegInf ? 0.f : fast_exp2(m1 - M);
    const float Ls = l * a0 + l1 * a1;
    const bool empty = (M == kNegInf || Ls == 0.f);
    const float f = empty ? 0.f : 1.0f / Ls;
    const int64_t rh = (int64_t)(q0 + t) * a.num_q_heads + kvh * G + n;
    float* dst = a.part_out + (rh * P + part) * DV + 4 * g;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(slab + n * SLAB_PITCH + db * 16 + 4 * g);
      store_partial4<false>(dst + db * 16, (acc[db] * a0 + o1 * a1) * f);   // plain stores measured faster here
    }
    if (g == 0) store_partial1<false>(a.part_lse + rh * P + part, empty ? kNegInf : (M + __builtin_log2f(Ls)) * kLn2);
  }
  PA_STAMP_FLUSH(g_phase_stamps_tokens, NW)
}

// bf16 MLA rows, 2 or more query tokens, up to 16 query heads per KV head, power-of-two
// block size of at least 16 (a 16-key half tile sits in one block).
bool splitkv_tokens_eligible(const SplitArgs& a) {
  const int bs = a.c.block_size;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  return a.c.esize == 2 && a.c.dk == stk::DK && a.c.dv == stk::DV && a.c.v_off == 0 && a.max_q >= 2 &&
         a.max_q * G > 16 && G <= 16 && (bs & (bs - 1)) == 0 && bs >= 16;
}

void launch_splitkv_tokens(const SplitArgs& a, hipStream_t s) {
  const int tg = (a.max_q + stk::NTOK - 1) / stk::NTOK;
  dim3 grid(a.num_partitions, a.c.num_kv_heads * tg, a.num_seqs), block(stk::NW * 64);
  hipLaunchKernelGGL(splitkv_tokens_kernel, grid, block, 0, s, a);
}

}  // namespace pa

#ifdef PA_PHASE_STAMPS
// The MLA verify token kernel's stamps (layout in phase_stamps.hpp; 8 waves per workgroup, a
// "tile" is one step of the wave): copies the first `words` (at most kStampWaves * 64) to
// host memory `dst`; returns the hipError_t of the copy.
extern "C" int attn_phase_stamps_read_tokens(void* dst, size_t words) {
  if (!dst || words > (size_t)pa::kStampWaves * 64) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(pa::g_phase_stamps_tokens), words * 4, 0, hipMemcpyDeviceToHost);
}
#endif
