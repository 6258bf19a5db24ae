// Causal chunked prefill over the paged cache (bf16 or fp8 K/V, bf16 Q).
//
// The pages' prefill kernel is FA2-style with one CTA per 8 tokens x 16 GQA heads
// and fp8 K/V converted in the load path (diffbot MiMo-V2.6-Flash model card,
// "What the kernels do"); 4096-token chunks, causal, GQA.  The gfx950 design:
//
//   workgroup  = 4 waves = 32 query tokens x G heads of one KV head (G = 8:
//                256 rows); row r of a wave = token r / G, head r % G, so every
//                K/V tile read from LDS feeds all G heads of the group.
//   per 32-key step: the workgroup stages K [32 x Dk] and V [32 x Dv] in LDS
//                (double-buffered, register prefetch of the next step), then
//                each wave does
//                S^T[32 keys x 64 rows] = K Q^T      48 x v_mfma_f32_16x16x32_bf16
//                online softmax (exp2, log2(e) folded into the scale)
//                O^T[128 x 64] += V^T P^T             32 x v_mfma_f32_16x16x32_bf16
//                V^T comes from two ds_read_b64_tr_b16 (keys 4g.., 16+4g..) whose
//                key order matches the lane's own probabilities, so P never moves.
//   masking:   only steps that cross the diagonal evaluate the causal mask;
//                steps past a wave's last visible key are skipped by that wave.
//   order:     heaviest query tiles first (they see the most keys).
#include "common.hpp"
#include "kernels.hpp"
#include "lds_layout.hpp"

namespace pa {

// A row's normalisation, with an optional sink logit sk2 (log2 units; -inf: none) that
// joins the denominator as one more term with a zero value row: denominator
// l*2^(m-M) + 2^(sk2-M), M = max(m, sk2); num scales the accumulator.  Without a sink
// this is num/l and m + log2(l) (0 and -inf for a row that saw no key).
__device__ __forceinline__ void softmax_finish(float m, float l, float sk2, float num, float& inv, float& lse) {
  if (sk2 == kNegInf) {
    inv = l > 0.f ? num / l : 0.f;
    lse = l > 0.f ? (m + __builtin_log2f(l)) * kLn2 : kNegInf;
    return;
  }
  const float M = fmaxf(m, sk2);
  const float e0 = l > 0.f ? fast_exp2(m - M) : 0.f;
  const float den = l * e0 + fast_exp2(sk2 - M);
  inv = num * e0 / den;
  lse = (M + __builtin_log2f(den)) * kLn2;
}

template <int DK, int DV, int VOFF, bool FP8>
__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillArgs a) {
  constexpr int NW = 4;                 // waves
  constexpr int NR = 4;                 // 16-row groups per wave -> 64 rows
  constexpr int KS = DK / 32;
  constexpr int DB = DV / 16;
  constexpr int KP = DK + 8;            // LDS pitch (elements) of K rows
  constexpr int VPp = DV + 16;          // LDS pitch of V rows
  constexpr int KT = 32;                // keys per step
  constexpr int KBUF = KT * KP, VBUF = KT * VPp;
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int ROWB = (DK + (VOFF >= DK ? DV : 0)) * EB;   // bytes per key row that we load
  constexpr int CH = ROWB / 16;         // 16-byte chunks per key row
  constexpr int NLOAD = (KT * CH + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t kl[2][KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t vl[2][VBUF];

  const int kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int tok_per_wave = 64 / G;
  const int QT = NW * tok_per_wave;
  const int q0 = a.qsl[b];
  const int L = a.qsl[b + 1] - q0;
  const int S = a.seq_lens[b];
  const int ntile = ceil_div(L, QT);
  const int tile = ntile - 1 - (int)blockIdx.x;        // heaviest first
  if (tile < 0) return;
  const int wt0 = tile * QT + wave * tok_per_wave;      // first query index of this wave
  const int off = S - L;                                 // position of query i is off + i

  // Q rows into registers; hi = last visible key of the lane's rows
  bf16x8 qreg[NR][KS];
  int hi[NR];
  int wave_hi = -1;
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const int r = rg * 16 + n;
    const int qi = wt0 + r / G, hh = r % G;
    const bool live = qi < L;
    hi[rg] = live ? min(off + qi, S - 1) : -1;
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? qi : 0)) * a.q_st + (int64_t)(kvh * G + hh) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0, 0, 0, 0};
      if (live) w = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
      qreg[rg][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  {
    const int last_q = min(wt0 + tok_per_wave, L) - 1;
    wave_hi = last_q >= wt0 ? min(off + last_q, S - 1) : -1;
  }
  // workgroup key range: 0 .. position of its last query
  const int wg_last_q = min(tile * QT + QT, L) - 1;
  const int wg_hi = min(off + wg_last_q, S - 1);
  const int nsteps = wg_hi >= 0 ? ceil_div(wg_hi + 1, KT) : 0;
  const int wave_lo_q = wt0;                               // first query of the wave
  const int wave_lo = off + wave_lo_q;                     // its position: keys <= this are visible to all rows

  float kscale = 1.f, vscale = 1.f;
  if (FP8 && a.c.scale_mode != 0) {
    kscale = a.c.scale_mode == 2 ? a.c.k_scale[kvh] : a.c.k_scale[0];
    vscale = a.c.scale_mode == 2 ? a.c.v_scale[kvh] : a.c.v_scale[0];
  }
  const float sl2 = a.scale * kLog2e * kscale;

  f32x4 acc[NR][DB];
  float m[NR], l[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    m[rg] = kNegInf;
    l[rg] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;
  u32x4 pre[NLOAD];
  auto gload = [&](int step) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int c = i * 256 + threadIdx.x;
      if (c < KT * CH) {
        const int key = c / CH, piece = c - key * CH;
        const int j = min(step * KT + key, S - 1);
        const int64_t blk = btrow[j / a.c.block_size];
        const int64_t pos = j % a.c.block_size;
        const uint8_t* row = a.c.data + (blk * a.c.sb + pos * a.c.ss + (int64_t)kvh * a.c.sh) * EB;
        const int byte = piece * 16;
        const int kb = DK * EB;
        pre[i] = *reinterpret_cast<const u32x4*>(row + (byte < kb ? byte : VOFF * EB + (byte - kb)));
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int c = i * 256 + threadIdx.x;
      if (c < KT * CH) {
        const int key = c / CH, piece = c - key * CH;
        const int byte = piece * 16;
        const int kb = DK * EB;
        if constexpr (!FP8) {
          if (byte < kb) *reinterpret_cast<u32x4*>(&kl[buf][key * KP + byte / 2]) = pre[i];
          else *reinterpret_cast<u32x4*>(&vl[buf][key * VPp + (byte - kb) / 2]) = pre[i];
        } else {
          u32x2 t0 = fp8x4_to_bf16x4(pre[i][0]), t1 = fp8x4_to_bf16x4(pre[i][1]);
          u32x2 t2 = fp8x4_to_bf16x4(pre[i][2]), t3 = fp8x4_to_bf16x4(pre[i][3]);
          u32x4 lo = {t0[0], t0[1], t1[0], t1[1]}, hi2 = {t2[0], t2[1], t3[0], t3[1]};
          uint16_t* dst = byte < kb ? &kl[buf][key * KP + byte] : &vl[buf][key * VPp + (byte - kb)];
          *reinterpret_cast<u32x4*>(dst) = lo;
          *reinterpret_cast<u32x4*>(dst + 8) = hi2;
        }
      }
    }
  };

  if (nsteps > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  const int tr_row = 4 * g + (n >> 2), tr_col = 4 * (n & 3);
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
    const int j0 = step * KT;
    if (j0 <= wave_hi) {
      // S^T for keys j0..j0+31 (two 16-key halves)
      f32x4 s[2][NR];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rg = 0; rg < NR; ++rg) s[h][rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&kl[cur][(16 * h + n) * KP + ks * 32 + g * 8]);
#pragma unroll
          for (int rg = 0; rg < NR; ++rg) s[h][rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[rg][ks], s[h][rg], 0, 0, 0);
        }
      }
      const bool need_mask = j0 + KT - 1 > wave_lo;          // some key past some row's position
      bf16x8 pb[NR];
#pragma unroll
      for (int rg = 0; rg < NR; ++rg) {
        float x[8];
        float mx = kNegInf;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s[h][rg][i] * sl2;
            if (need_mask) {
              const int j = j0 + 16 * h + 4 * g + i;
              v = (j <= hi[rg]) ? v : kNegInf;
            }
            x[h * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = max_over_groups(mx);
        const float mn = fmaxf(m[rg], mx);
        const float base = (mn == kNegInf) ? 0.f : mn;
        const float alpha = fast_exp2(m[rg] - base);
        float ps = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = fast_exp2(x[2 * i] - base), p1 = fast_exp2(x[2 * i + 1] - base);
          ps += p0 + p1;
          pk[i] = pack_bf16x2(p0, p1);
        }
        l[rg] = l[rg] * alpha + ps;
        m[rg] = mn;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[rg][db] *= alpha;
        }
        pb[rg] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(&vl[cur][tr_row * VPp + db * 16 + tr_col]));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(&vl[cur][(16 + tr_row) * VPp + db * 16 + tr_col]));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
#pragma unroll
        for (int rg = 0; rg < NR; ++rg) acc[rg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[rg], acc[rg][db], 0, 0, 0);
      }
    }
    if (step + 1 < nsteps) lstore(cur ^ 1);
    __syncthreads();
  }

  // normalise and write: lane holds dims db*16+4g..+3 of row rg*16+n
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const float lt = sum_over_groups(l[rg]);
    const int r = rg * 16 + n;
    const int qi = wt0 + r / G, hh = r % G;
    if (qi >= L) continue;
    const int64_t tok = q0 + qi, head = kvh * G + hh;
    float inv, lse;
    softmax_finish(m[rg], lt, a.sinks ? a.sinks[head] * kLog2e : kNegInf, vscale, inv, lse);
    uint16_t* op = a.out + (tok * a.num_q_heads + head) * DV;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 v = acc[rg][db] * inv;
      u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(op + db * 16 + 4 * g) = pk;
    }
    if (a.out_lse && g == 0) a.out_lse[tok * a.num_q_heads + head] = lse;
  }
}

bool prefill_supported(const PrefillArgs& a) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  if (G < 1 || 64 % G != 0) return false;
  return a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192;
}

bool prefill_fast_eligible(const PrefillArgs& a);
void launch_prefill_fast(const PrefillArgs& a, hipStream_t s);

bool launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (prefill_fast_eligible(a)) {
    launch_prefill_fast(a, s);
    return true;
  }
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int QT = 4 * (64 / G);
  const int tiles = (a.max_q + QT - 1) / QT;
  if (tiles == 0 || a.num_seqs == 0) return true;
  dim3 grid(tiles, a.c.num_kv_heads, a.num_seqs), block(256);
  if (a.c.esize == 1) hipLaunchKernelGGL((prefill_kernel<192, 128, 192, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((prefill_kernel<192, 128, 192, false>), grid, block, 0, s, a);
  return true;
}

// ===========================================================================
// Fast path: bf16 DiffKV rows (K 192 / V 128), block size a power of two >= 16.
//
//   rows      workgroup = 8 waves x 32 rows (32 query tokens x 8 GQA heads for G = 8);
//             a wave's 32 rows are one v_mfma_f32_32x32x16_bf16 column block, whose
//             output gives a lane 16 keys of one row: a row max needs a single
//             cross-lane step (lanes l and l^32).  ~200 registers per wave, so two
//             waves share each SIMD and the hardware overlaps one wave's MFMAs with
//             the other's softmax.
//   K/V       64-key stages land in LDS straight from HBM/L2 with
//             global_load_lds_dwordx4 (16 B per lane at base + 16*lane): no VGPR
//             staging.  A 3-stage ring keeps two stages (80 KB) in flight while one
//             is consumed; completion is tracked with explicit vmcnt waits (the
//             compiler does not track LDS-DMA writes) and one s_barrier per stage.
//             The kernel must not spill: a scratch reload is a vector-memory op
//             issued behind the DMA, and waiting for it would drain the ring.
//             Slots are XOR-swizzled so K operand reads (ds_read_b128) and the
//             transposing V reads (ds_read_b64_tr_b16) are bank-conflict free.
//   softmax   lazy rescaling: the running max used for exp2 only moves when the true
//             max exceeds it by more than 8 (log2 units), so p <= 256 and the
//             accumulator is rescaled rarely; the scale is folded into one fma.
//   order     workgroups of one KV head stay on the same XCDs (they share the K/V
//             prefix in that XCD's L2); heaviest query tiles first.
namespace pf {
constexpr int DK = 192, DV = 128, VOFF = 192;
constexpr int KT = 64;                   // keys per stage
constexpr int NSTAGE = 3;                // one consumed, two in flight
constexpr int NW = 8;
constexpr int ROWS_W = 32;               // rows per wave
constexpr int KCH = DK * 2 / 16;         // 24 chunks of 16 B per K row
constexpr int VCH = DV * 2 / 16;         // 16 chunks per V row
constexpr int KSLOTS = KT * KCH;         // 1536
constexpr int SLOTS = KT * (KCH + VCH);  // 2560
constexpr int PER_WAVE = SLOTS / 64 / NW;  // 5 DMA instructions per wave per stage
constexpr int STAGE_BYTES = SLOTS * 16;  // 40 KB
constexpr int BT_MAX = 4096;             // block-table entries staged in LDS
constexpr int KS = DK / 16;              // 12 k-steps
constexpr int DB = DV / 32;              // 4 output dim blocks
static_assert(SLOTS % (64 * NW) == 0, "stage must split evenly over the waves");
}  // namespace pf

// chunk swizzles of the stage rows: lds_layout.hpp (prefill_k_swz for the 384-byte K rows,
// prefill_v_swz for the 256-byte V rows)
__device__ __forceinline__ int pf_k_slot(int key, int c) { return key * pf::KCH + (c ^ prefill_k_swz(key)); }
__device__ __forceinline__ int pf_v_slot(int key, int c) { return pf::KSLOTS + key * pf::VCH + (c ^ prefill_v_swz(key)); }

#define PF_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
__device__ __forceinline__ void pf_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(512, 1) void prefill_fast_kernel(PrefillArgs a, int ntile_max) {
  using namespace pf;
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * STAGE_BYTES];
  __shared__ int btl[BT_MAX];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int Hkv = a.c.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int TPW = ROWS_W / G;                   // query tokens per wave
  const int QT = NW * TPW;                      // query tokens per workgroup
  // ---- workgroup -> (sequence, KV head, tile): XCD-aware, heaviest first ----
  const int NH = a.num_seqs * Hkv;
  const int lin = blockIdx.x;
  int hg, rank;
  if (NH < 8 && 8 % NH == 0) {
    const int per = 8 / NH, xcd = lin & 7;
    hg = xcd / per;
    rank = (lin >> 3) * per + xcd % per;
  } else {
    hg = lin % NH;
    rank = lin / NH;
  }
  const int b = hg / Hkv, kvh = hg - b * Hkv;
  const int q0 = a.qsl[b];
  const int L = a.qsl[b + 1] - q0;
  const int S = a.seq_lens[b];
  const int ntile = ceil_div(L, QT);
  if (rank >= ntile) return;
  const int tile = ntile - 1 - rank;
  const int off = S - L;
  const int wt0 = tile * QT + wave * TPW;
  const int wg_last_q = min(tile * QT + QT, L) - 1;
  const int wg_hi = min(off + wg_last_q, S - 1);
  const int nsteps = wg_hi >= 0 ? wg_hi / KT + 1 : 0;
  const int bs_shift = __builtin_ctz(a.c.block_size);   // block size is a power of two here
  const int bs_mask = a.c.block_size - 1;
  const int nblk = wg_hi >= 0 ? (wg_hi >> bs_shift) + 1 : 0;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;
  for (int i = threadIdx.x; i < nblk; i += NW * 64) btl[i] = btrow[i];

  // ---- Q rows of this wave into registers (B operand), visibility limit ----
  bf16x8 qreg[KS];
  const int qi_lane = wt0 + n32 / G;
  const bool live = qi_lane < L;
  const int hi = live ? min(off + qi_lane, S - 1) : -1;
  {
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? qi_lane : 0)) * a.q_st + (int64_t)(kvh * G + n32 % G) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0, 0, 0, 0};
      if (live) w = *reinterpret_cast<const u32x4*>(qp + ks * 16 + g * 8);
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const int wave_last_q = min(wt0 + TPW, L) - 1;
  const int wave_hi = wave_last_q >= wt0 ? min(off + wave_last_q, S - 1) : -1;
  const int wave_lo = off + wt0;                // keys <= wave_lo are visible to every live row
  const float sl2 = a.scale * kLog2e;

  // the (key, byte-in-row) each lane fetches per DMA instruction does not depend on the stage
  int dkey[PER_WAVE], dbyte[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int slot = (wave * PER_WAVE + u) * 64 + lane;
    if (slot < KSLOTS) {
      dkey[u] = slot / KCH;
      dbyte[u] = ((slot - dkey[u] * KCH) ^ prefill_k_swz(dkey[u])) * 16;
    } else {
      const int vs = slot - KSLOTS;
      dkey[u] = vs / VCH;
      dbyte[u] = VOFF * 2 + ((vs - dkey[u] * VCH) ^ prefill_v_swz(dkey[u])) * 16;
    }
  }
  const uint8_t* head_base = a.c.data + (int64_t)kvh * a.c.sh * 2;
  // lane byte offsets of the K operand reads (per r = ks % 4) and of the transposed V
  // reads (per 32-dim block), relative to the stage buffer
  int koff[4], voff[DB];
  {
    const int sw = prefill_k_swz(n32);                 // = prefill_k_swz(32h + n32) for both halves
#pragma unroll
    for (int r = 0; r < 4; ++r) koff[r] = (n32 * KCH + ((2 * r + g) ^ sw)) * 16;
    const int s16 = lane & 15, half = (lane >> 4) & 1;
    const int vkey = 4 * g + (s16 >> 2);          // key within a 16-key chunk (the +8 row keeps key & 7)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dim = db * 32 + 16 * half + 4 * (s16 & 3);
      voff[db] = pf_v_slot(vkey, dim >> 3) * 16 + (dim & 7) * 2;
    }
  }
  __syncthreads();                              // block table staged; Q loads retired

  // keys past the workgroup's last visible key re-read that key: every block id used
  // comes from the staged part of the table (entries 0 .. wg_hi / BS)
  // Every DMA instruction's 64 lanes lie in one 16-key group (6 K and 4 V
  // instructions per 16 keys), hence in one block: on full stages the block base is
  // wave-uniform (SGPRs, from one table entry) and each lane adds a fixed 32-bit
  // offset, so issuing a stage costs no per-lane 64-bit address arithmetic.
  const int ss2 = (int)(a.c.ss * 2);
  const int64_t sb2 = a.c.sb * 2;
  const int pmask = min(bs_mask, KT - 1);        // in-block position bits a stage can vary
  int loff[PER_WAVE], ikey[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    loff[u] = (dkey[u] & pmask) * ss2 + dbyte[u];
    const int slot0 = __builtin_amdgcn_readfirstlane((wave * PER_WAVE + u) * 64);
    ikey[u] = slot0 < KSLOTS ? slot0 / KCH : (slot0 - KSLOTS) / VCH;   // the instruction's first key
  }
  auto issue = [&](int st) {
    char* buf = smem + (st % NSTAGE) * STAGE_BYTES;
    const int j0 = st * KT;
    const int kmax = wg_hi - j0;
    if (kmax >= KT - 1) {
      const int64_t stage_in_block = (int64_t)(j0 & bs_mask & ~(KT - 1)) * ss2;   // non-zero for BS > 64
      int blk[PER_WAVE];                          // all table reads first: one LDS wait
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) blk[u] = btl[(j0 + ikey[u]) >> bs_shift];
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const uint8_t* base = head_base + (int64_t)__builtin_amdgcn_readfirstlane(blk[u]) * sb2 + stage_in_block;
        dma16_s(loff[u], base, lds_addr(buf + (wave * PER_WAVE + u) * 1024));
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int j = j0 + min(dkey[u], kmax);
      const int64_t blk = btl[j >> bs_shift];
      const int64_t pos = j & bs_mask;
      const uint8_t* src = head_base + (blk * a.c.sb + pos * a.c.ss) * 2 + dbyte[u];
      // inline asm (dma16): the compiler would otherwise answer the LDS-DMA with
      // vmcnt(0) before some LDS reads; every wait on the ring is explicit
      dma16(src, lds_addr(buf + (wave * PER_WAVE + u) * 1024));
    }
  };

  f32x16 acc[DB];
  float m = kNegInf, l = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // one 32-key half of a stage: QK^T, online softmax, PV (each half updates (m, l, acc))
  auto half_step = [&](int j, int h) {
    const char* buf = smem + (j % NSTAGE) * STAGE_BYTES;
    const int kb = j * KT + 32 * h;                // first key of the half
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    // chunk 2ks+g of key 32h+n32: ks = 4t+r -> slot = key*24 + 8t + ((2r+g) ^ swizzle), so
    // the lane-dependent part is koff[r] and t, h enter as immediate offsets
    const char* kbuf = buf + h * (32 * KCH * 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kbuf + koff[ks & 3] + (ks >> 2) * 128);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[ks], s, 0, 0, 0);
    }
    // online softmax on raw scores; the scale (> 0) is folded into one fma per score
    float mx = kNegInf;
    if (kb + 31 > wave_lo) {                       // the causal diagonal crosses this half
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + 8 * (i >> 2) + 4 * g + (i & 3);
        s[i] = key <= hi ? s[i] : kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
    const float mn = fmaxf(m, mx);
    const bool grow = mn > m + 8.0f;             // true on the first visible key (m = -inf)
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m - mn) : 1.0f;
      m = grow ? mn : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float nbase = m == kNegInf ? 0.f : -m;
    uint32_t pk[8];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(s[2 * i], sl2, nbase));
      const float p1 = fast_exp2(__builtin_fmaf(s[2 * i + 1], sl2, nbase));
      ps += p0 + p1;
      pk[i] = pack_bf16x2(p0, p1);
    }
    l += ps;
    // O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] P^T[16 keys x 32 rows]; the lane's
    // k order (keys 16kh+4g+0..3, then 16kh+8+4g+0..3) matches its own probabilities
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * kh], pk[4 * kh + 1], pk[4 * kh + 2], pk[4 * kh + 3]});
      // source row key = 32h + 16kh + (4g + s16/4) [+ 8]: the swizzle depends only on the lane
      // part, so h, kh and the +8 row are immediate offsets on voff[db]
      const char* vbuf = buf + (32 * h + 16 * kh) * (VCH * 16);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbuf + voff[db]));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbuf + voff[db] + 8 * VCH * 16));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb, acc[db], 0, 0, 0);
      }
    }
  };

  // A whole stage with no causal mask (every key visible to every live row of the wave),
  // software-pipelined inside the wave:  QK0 | QK1 + softmax0 | PV0 + softmax1 | PV1.
  // The scheduler is asked to interleave one MFMA with a few VALU/transcendental ops in
  // the two overlapped regions; the rare accumulator rescale sits between regions.
  auto qk_half = [&](const char* buf, int h, f32x16& s) {
    const char* kbuf = buf + h * (32 * KCH * 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kbuf + koff[ks & 3] + (ks >> 2) * 128);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[ks], s, 0, 0, 0);
    }
  };
  // the same QK^T with its K operands read four k-steps ahead, the order held by a
  // scheduling barrier after each k-step: the block that runs at raised priority, where
  // the compiler's own order read each operand right before its MFMA and waited for it
  auto qk_half_ahead = [&](const char* buf, int h, f32x16& s) {
    constexpr int KPF = 4;
    const char* kbuf = buf + h * (32 * KCH * 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    bf16x8 kb[KPF + 1];
#pragma unroll
    for (int j = 0; j < KPF; ++j) kb[j] = *reinterpret_cast<const bf16x8*>(kbuf + koff[j & 3] + (j >> 2) * 128);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int jn = ks + KPF;
      if (jn < KS) kb[jn % (KPF + 1)] = *reinterpret_cast<const bf16x8*>(kbuf + koff[jn & 3] + (jn >> 2) * 128);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[ks % (KPF + 1)], qreg[ks], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // softmax of one unmasked half: updates m and l, returns P as bf16 and the factor the
  // accumulator must be scaled by before this half's PV (1 unless the max grew)
  auto softmax_half = [&](f32x16& s, uint32_t (&pk)[8]) -> float {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
    const float mn = fmaxf(m, mx);
    const bool grow = mn > m + 8.0f;
    const float alpha = grow ? fast_exp2(m - mn) : 1.0f;
    m = grow ? mn : m;
    const float nbase = -m;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(s[2 * i], sl2, nbase));
      const float p1 = fast_exp2(__builtin_fmaf(s[2 * i + 1], sl2, nbase));
      ps += p0 + p1;
      pk[i] = pack_bf16x2(p0, p1);
    }
    l = l * alpha + ps;
    return alpha;
  };
  auto pv_half = [&](const char* buf, int h, const uint32_t (&pk)[8]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * kh], pk[4 * kh + 1], pk[4 * kh + 2], pk[4 * kh + 3]});
      const char* vbuf = buf + (32 * h + 16 * kh) * (VCH * 16);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbuf + voff[db]));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbuf + voff[db] + 8 * VCH * 16));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb, acc[db], 0, 0, 0);
      }
    }
  };
  auto bulk_stage = [&](int j) {
    const char* buf = smem + (j % NSTAGE) * STAGE_BYTES;
    f32x16 s0, s1;
    uint32_t p0[8], p1[8];
    // The two blocks that are MFMAs only (the first half's QK^T, the second half's PV)
    // run at raised wave priority: while the SIMD's other wave is in a mixed region, the
    // arbiter issues this wave's MFMAs first and the other wave's softmax fills the
    // matrix core's gaps (chunked prefill 1.3% faster; the same schedule without the
    // priority is 2% slower, and raising it over region 1 as well, 2-3% slower).
    __builtin_amdgcn_s_setprio(1);
    qk_half_ahead(buf, 0, s0);
    __builtin_amdgcn_s_setprio(0);
    // region 1: QK of the second half while the first half's softmax runs: 12 K-operand
    // reads running three MFMAs ahead (a read issued just before its MFMA exposes a whole
    // LDS round trip per k-step), the softmax's VALU work between the MFMAs.
    qk_half(buf, 1, s1);
    const float a0 = softmax_half(s0, p0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 1);     // ds_read: operands 0-2
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // mfma i
      if (i + 3 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);       // ds_read i + 3
      __builtin_amdgcn_sched_group_barrier(0x402, 5, 1);   // valu / trans
    }
    if (__any(a0 != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= a0;
    }
    // region 2: PV of the first half while the second half's softmax runs
    pv_half(buf, 0, p0);
    const float a1 = softmax_half(s1, p1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);     // ds_read: operands of MFMAs 0-1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);   // mfma i
      if (i + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);   // two transposed reads, MFMA i + 2
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 2);   // valu / trans
    }
    if (__any(a1 != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= a1;
    }
    __builtin_amdgcn_s_setprio(1);
    pv_half(buf, 1, p1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 3);     // ds_read: operands of MFMAs 0-1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);   // mfma i
      if (i + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);   // MFMA i + 2's reads
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Q is complete from here on.  A wait the compiler sees (the ring's waits are inline
  // asm, invisible to it): otherwise it assumes Q may still be in flight and answers its
  // first use on each path with vmcnt(0), which would drain the ring.
  __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)
  // ---- pipeline: stage j is consumed while stages j+1, j+2 are in flight ----
  if (nsteps > 0) issue(0);
  if (nsteps > 1) issue(1);
  for (int j = 0; j < nsteps; ++j) {
    if (j + 1 < nsteps) PF_WAIT_VM(5);             // stage j landed; stage j+1 may still fly
    else PF_WAIT_VM(0);
    pf_barrier();                                  // stage j resident for all waves; stage j-1 dead
    if (j + 2 < nsteps) issue(j + 2);
    if (wave_hi >= 0 && j * KT + KT - 1 <= wave_lo) {
      bulk_stage(j);                               // no key of the stage is masked for this wave
    } else {
      if (j * KT <= wave_hi) half_step(j, 0);
      if (j * KT + 32 <= wave_hi) half_step(j, 1);
    }
  }

  // ---- normalise and write: lane holds dims db*32 + 8q + 4g + 0..3 of its row ----
  const float lt = l + __shfl_xor(l, 32, 64);
  if (live) {
    const int64_t tok = q0 + qi_lane, head = kvh * G + n32 % G;
    float inv, lse;
    softmax_finish(m, lt, a.sinks ? a.sinks[head] * kLog2e : kNegInf, 1.0f, inv, lse);
    uint16_t* op = a.out + (tok * a.num_q_heads + head) * DV;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        u32x2 pk = {pack_bf16x2(acc[db][4 * qq] * inv, acc[db][4 * qq + 1] * inv),
                    pack_bf16x2(acc[db][4 * qq + 2] * inv, acc[db][4 * qq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + db * 32 + 8 * qq + 4 * g) = pk;
      }
    if (a.out_lse && g == 0) a.out_lse[tok * a.num_q_heads + head] = lse;
  }
}

bool prefill_fast_eligible(const PrefillArgs& a) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int bs = a.c.block_size;
  return a.c.esize == 2 && a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192 && bs >= 16 && (bs & (bs - 1)) == 0 &&
         G >= 1 && pf::ROWS_W % G == 0 && a.bt_stride <= pf::BT_MAX && a.scale > 0.f;
}

void launch_prefill_fast(const PrefillArgs& a, hipStream_t s) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int QT = pf::NW * (pf::ROWS_W / G);
  const int ntile_max = (a.max_q + QT - 1) / QT;
  const int NH = a.num_seqs * a.c.num_kv_heads;
  int grid;
  if (NH < 8 && 8 % NH == 0) {
    const int per = 8 / NH;
    grid = (ntile_max + per - 1) / per * per * NH;
  } else {
    grid = ntile_max * NH;
  }
  if (grid == 0) return;
  hipLaunchKernelGGL(prefill_fast_kernel, dim3(grid), dim3(pf::NW * 64), 0, s, a, ntile_max);
}

}  // namespace pa
