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

namespace pa {

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
    const float inv = lt > 0.f ? vscale / lt : 0.f;
    const int64_t tok = q0 + qi, head = kvh * G + hh;
    uint16_t* op = a.out + (tok * a.num_q_heads + head) * DV;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 v = acc[rg][db] * inv;
      u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(op + db * 16 + 4 * g) = pk;
    }
    if (a.out_lse && g == 0)
      a.out_lse[tok * a.num_q_heads + head] = lt > 0.f ? (m[rg] + __builtin_log2f(lt)) * kLn2 : kNegInf;
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
// Fast path: bf16 DiffKV rows (K 192 / V 128), block size a multiple of 16.
//
//   rows      wave = 64 rows = 2 groups of 32 for v_mfma_f32_32x32x16_bf16; the
//             32x32 output gives a lane 16 keys of one row, so a row max needs a
//             single cross-lane step (lanes l and l^32).
//   K/V       32-key stages land in LDS straight from HBM/L2 with
//             global_load_lds_dwordx4 (16 B per lane at base + 16*lane): no VGPR
//             staging.  A 6-stage ring keeps four stages (80 KB) in flight while one
//             is consumed, enough to cover L2/MALL latency at ~1 us per step;
//             completion is tracked with explicit vmcnt waits (the compiler does
//             not track LDS-DMA writes) and one s_barrier per step.  The kernel
//             must not spill: a scratch reload is a vector-memory op issued after
//             the DMA, so waiting for it would drain the whole ring.
//             Slots are XOR-swizzled so the K operand reads (ds_read_b128) and
//             the transposing V reads (ds_read_b64_tr_b16) are bank-conflict free.
//   softmax   lazy rescaling: the running max used for exp2 is only moved when
//             the true max exceeds it by more than 8 (in log2 units), so p <= 256
//             and the accumulator is rescaled rarely.
//   order     workgroups of one KV head stay on the same XCDs (they share the
//             K/V prefix in that XCD's L2); heaviest query tiles first.
namespace pf {
constexpr int DK = 192, DV = 128, VOFF = 192;
constexpr int KT = 32;                   // keys per stage
constexpr int NSTAGE = 6;                // ring: one stage consumed, up to four in flight
constexpr int NW = 4;
constexpr int KCH = DK * 2 / 16;         // 24 chunks of 16 B per K row
constexpr int VCH = DV * 2 / 16;         // 16 chunks per V row
constexpr int KSLOTS = KT * KCH;         // 768
constexpr int SLOTS = KT * (KCH + VCH);  // 1280
constexpr int PER_WAVE = SLOTS / 64 / NW;  // 5 DMA instructions per wave per stage
constexpr int STAGE_BYTES = SLOTS * 16;  // 20 KB
constexpr int BT_MAX = 4096;             // block-table entries staged in LDS
constexpr int KS = DK / 16;              // 12 k-steps
constexpr int DB = DV / 32;              // 4 output dim blocks
}  // namespace pf

__device__ __forceinline__ int pf_k_slot(int key, int c) { return key * pf::KCH + (c ^ ((key >> 1) & 7)); }
__device__ __forceinline__ int pf_v_slot(int key, int c) { return pf::KSLOTS + key * pf::VCH + (c ^ ((key & 7) << 1)); }

#define PF_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
__device__ __forceinline__ void pf_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(256, 1) void prefill_fast_kernel(PrefillArgs a, int ntile_max) {
  using namespace pf;
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * STAGE_BYTES];
  __shared__ int btl[BT_MAX];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int Hkv = a.c.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int TPW = 64 / G;                       // query tokens per wave
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
  const int BS = a.c.block_size;
  const int nblk = wg_hi >= 0 ? wg_hi / BS + 1 : 0;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;
  for (int i = threadIdx.x; i < nblk; i += 256) btl[i] = btrow[i];

  // ---- Q rows of this wave into registers (B operand), visibility limits ----
  bf16x8 qreg[2][KS];
  int hi[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int r = rg * 32 + n32;
    const int qi = wt0 + r / G, hh = r % G;
    const bool live = qi < L;
    hi[rg] = live ? min(off + qi, S - 1) : -1;
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? qi : 0)) * a.q_st + (int64_t)(kvh * G + hh) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0, 0, 0, 0};
      if (live) w = *reinterpret_cast<const u32x4*>(qp + ks * 16 + g * 8);
      qreg[rg][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const int wave_last_q = min(wt0 + TPW, L) - 1;
  const int wave_hi = wave_last_q >= wt0 ? min(off + wave_last_q, S - 1) : -1;
  const int wave_lo = off + wt0;                // keys <= wave_lo are visible to every live row
  const float sl2 = a.scale * kLog2e;
  __syncthreads();                              // block table staged; Q loads retired

  auto issue = [&](int st) {
    char* buf = smem + (st % NSTAGE) * STAGE_BYTES;
    const int j0 = st * KT;
    // keys past the workgroup's last visible key re-read that key: every block id used
    // comes from the staged part of the table (entries 0 .. wg_hi / BS)
    const int kmax = wg_hi - j0;
    const int64_t B0 = btl[j0 / BS];
    const int64_t B1 = btl[min(j0 + 16, wg_hi) / BS];
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int i = wave * PER_WAVE + u;
      const int slot = i * 64 + lane;
      int key, byte;
      if (slot < KSLOTS) {
        key = slot / KCH;
        byte = ((slot - key * KCH) ^ ((key >> 1) & 7)) * 16;
      } else {
        const int vs = slot - KSLOTS;
        key = vs / VCH;
        byte = VOFF * 2 + ((vs - key * VCH) ^ ((key & 7) << 1)) * 16;
      }
      const int kc = min(key, kmax);
      const int64_t blk = kc < 16 ? B0 : B1;
      const int64_t pos = (j0 + kc) % BS;
      const uint8_t* src = a.c.data + (blk * a.c.sb + pos * a.c.ss + (int64_t)kvh * a.c.sh) * 2 + byte;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, 0, 0);
    }
  };

  auto qk = [&](int st, f32x16 (&s)[2]) {
    const char* buf = smem + (st % NSTAGE) * STAGE_BYTES;
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[rg][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(buf + pf_k_slot(n32, 2 * ks + g) * 16);
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) s[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[rg][ks], s[rg], 0, 0, 0);
    }
  };

  f32x16 acc[2][DB];
  float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rg][db][i] = 0.f;

  auto softmax_pv = [&](int j, const f32x16 (&s)[2]) {
    const bool need_mask = j * KT + KT - 1 > wave_lo;
    bf16x8 pb[2][2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float x[16];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[rg][i] * sl2;
        if (need_mask) {
          const int key = j * KT + 8 * (i >> 2) + 4 * g + (i & 3);
          v = key <= hi[rg] ? v : kNegInf;
        }
        x[i] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m[rg], mx);
      const bool grow = mn > m[rg] + 8.0f;       // true on the first visible key (m = -inf)
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2(m[rg] - mn) : 1.0f;
        m[rg] = grow ? mn : m[rg];
        l[rg] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rg][db] *= alpha;
      }
      const float base = m[rg] == kNegInf ? 0.f : m[rg];
      float ps = 0.f;
      uint32_t pk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = fast_exp2(x[2 * i] - base), p1 = fast_exp2(x[2 * i + 1] - base);
        ps += p0 + p1;
        pk[i] = pack_bf16x2(p0, p1);
      }
      l[rg] += ps;
      pb[rg][0] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      pb[rg][1] = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
    }
    // O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] P^T[16 keys x 32 rows]; the lane's
    // k order (keys 16kh+4g+0..3, then 16kh+8+4g+0..3) matches its own probabilities
    const char* buf = smem + (j % NSTAGE) * STAGE_BYTES;
    const int s16 = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int key0 = 16 * kh + 4 * g + (s16 >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dim = db * 32 + 16 * half + 4 * (s16 & 3);
        const int c = dim >> 3, inb = (dim & 7) * 2;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(buf + pf_v_slot(key0, c) * 16 + inb));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(buf + pf_v_slot(key0 + 8, c) * 16 + inb));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          acc[rg][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[rg][kh], acc[rg][db], 0, 0, 0);
      }
    }
  };

  // ---- pipeline: stage j is consumed while stages j+1 .. j+NSTAGE-2 are in flight ----
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st)
    if (st < nsteps) issue(st);
  for (int j = 0; j < nsteps; ++j) {
    const int ahead = min(NSTAGE - 2, nsteps - 1 - j);   // stages issued after stage j
    if (ahead >= 4) PF_WAIT_VM(20);
    else if (ahead == 3) PF_WAIT_VM(15);
    else if (ahead == 2) PF_WAIT_VM(10);
    else if (ahead == 1) PF_WAIT_VM(5);
    else PF_WAIT_VM(0);
    pf_barrier();                                  // stage j resident for all waves; stage j-1 dead
    if (j + NSTAGE - 1 < nsteps) issue(j + NSTAGE - 1);
    if (j * KT <= wave_hi) {
      f32x16 s[2];
      qk(j, s);
      softmax_pv(j, s);
    }
  }

  // ---- normalise and write ----
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const float lt = l[rg] + __shfl_xor(l[rg], 32, 64);
    const int r = rg * 32 + n32;
    const int qi = wt0 + r / G, hh = r % G;
    if (qi >= L) continue;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int64_t tok = q0 + qi, head = kvh * G + hh;
    uint16_t* op = a.out + (tok * a.num_q_heads + head) * DV;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        u32x2 pk = {pack_bf16x2(acc[rg][db][4 * qq] * inv, acc[rg][db][4 * qq + 1] * inv),
                    pack_bf16x2(acc[rg][db][4 * qq + 2] * inv, acc[rg][db][4 * qq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + db * 32 + 8 * qq + 4 * g) = pk;
      }
    if (a.out_lse && g == 0)
      a.out_lse[tok * a.num_q_heads + head] = lt > 0.f ? (m[rg] + __builtin_log2f(lt)) * kLn2 : kNegInf;
  }
}

bool prefill_fast_eligible(const PrefillArgs& a) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  return a.c.esize == 2 && a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192 && a.c.block_size % 16 == 0 &&
         G >= 1 && 64 % G == 0 && a.bt_stride <= pf::BT_MAX;
}

void launch_prefill_fast(const PrefillArgs& a, hipStream_t s) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int QT = pf::NW * (64 / G);
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
  hipLaunchKernelGGL(prefill_fast_kernel, dim3(grid), dim3(256), 0, s, a, ntile_max);
}

}  // namespace pa
