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
#include "lds_layout.hpp"
#include "phase_stamps.hpp"

namespace pa {

#ifdef PA_PHASE_STAMPS
__device__ uint32_t g_phase_stamps[kStampWaves * 64];   // this kernel's stamps (phase_stamps.hpp)
#endif

namespace sd {
constexpr int NW = 4;
constexpr int TT = 16;                 // keys per tile
}  // namespace sd

// chunk swizzles of the ring rows: lds_layout.hpp (bf16 rows row_chunk_swz, fp8 rows
// fp8_chunk_swz)

// FP8: E4M3FN rows; K chunks are converted to bf16 at the MFMA, V chunks are converted
// into a per-wave bf16 [key][dim] tile for the transposing read.  NTL: nontemporal DMA.
template <int DK, int DV, int VOFF, int NR, int NST, int MINW, bool FP8, bool NTL>
__global__ __launch_bounds__(sd::NW * 64, MINW) void splitkv_dma_kernel(SplitArgs a) {
  using namespace sd;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int ROWB = (VOFF >= DK ? DK + DV : DK) * ESZ; // bytes of a row that are read
  constexpr int CH = ROWB / 16;                           // 16-byte chunks per row
  constexpr int NINS = TT * CH / 64;                      // DMA instructions per tile
  constexpr int TILE_BYTES = TT * CH * 16;
  constexpr int KS = DK / 32;
  constexpr int DB = DV / 16;
  constexpr int ROWS = NR * 16;
  constexpr int VP = DV + 16;                             // fp8: bf16 V tile pitch (elements)
  constexpr int WAVE_BYTES = NST * TILE_BYTES;
  static_assert(!FP8 || TT * VP * 2 <= TILE_BYTES, "fp8: the bf16 V tile reuses its stage");
  constexpr int MERGE_PITCH = DV + 4;
  constexpr int RING = NW * WAVE_BYTES;
  constexpr int MERGE = NW * ROWS * 2 * 4 + NW * ROWS * MERGE_PITCH * 4;
  constexpr int LDS_BYTES = RING > MERGE ? RING : MERGE;
  static_assert(CH % (FP8 ? 4 : 8) == 0 && (TT * CH) % 64 == 0, "row must be whole swizzle groups");
  static_assert(!FP8 || (VOFF == DK && DK % 64 == 0 && DV % 64 == 0), "fp8: V follows K, 64-byte pieces");
  static_assert(VOFF % 8 == 0 && (VOFF >= DK || VOFF + DV <= DK), "V must be whole chunks of the row");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int P = a.num_partitions;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  PA_STAMP_DECL
  PA_STAMP(0)
  // every per-sequence scalar in one round trip (NULL arguments read zeros): the block ids
  // of the first tiles wait on seq_len, and nothing else should sit in front of them
  const int32_t* qslp = a.qsl ? a.qsl + b : reinterpret_cast<const int32_t*>(kZeroScalars);
  const int64_t* aslp = a.aslot ? a.aslot + b : kZeroScalars;
  const int S = load_uniform(a.seq_lens + b);
  const int qs0 = load_uniform(qslp), qs1 = load_uniform(qslp + 1);
  const int64_t new_slot = a.aslot ? load_uniform64(aslp) : -1;
  const int q0 = a.qsl ? qs0 : b;
  const int L = a.qsl ? qs1 - qs0 : 1;
  const int chunk = ceil_div(ceil_div(S, active_splits(a.pol, S, P)), TT) * TT;
  const int start = min(part * chunk, S);
  const int end = min(start + chunk, S);
  const int nt = ceil_div(end - start, TT);
  const int bs_shift = __builtin_ctz(a.c.block_size);
  const int bs_mask = a.c.block_size - 1;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;

  // ---- fused new-token write (decode): the workgroup whose key range holds key S-1
  // (partition 0 when S == 0) owns token b's K/V row of this KV head.  DiffKV rows: its
  // lanes load the row (chunk c of the row as it lies in the cache: lane c % 64) with Q,
  // store it into the slot after the prologue's wait, and the wave that consumes the last
  // tile copies it into that tile's LDS stage over whatever the DMA fetched for key S-1 (and
  // for the keys past the partition, which re-read key S-1): the LDS then holds exactly
  // what it would after a completed write, and no read waits on the store.  MLA rows, whose
  // kernel has no registers to spare for the row: the owner writes it first and waits for
  // the stores before any of its waves issues a read (its partition is the sequence's last
  // and no longer than the others, so the wait is off the critical path) ----
  constexpr bool kPatchRow = DK <= 256;
  constexpr int RCH = (CH + 63) / 64;
  constexpr int KCH = DK * ESZ / 16;             // chunks of the row that are K
  const bool own = new_slot >= 0 && (S > 0 ? (start <= S - 1 && S - 1 < end) : part == 0);   // uniform
  auto new_row_chunk = [&](int c) -> u32x4 {     // chunk c (16 bytes) of the new row, encoded
    const bool isk = c < KCH;
    const int e0 = (isk ? c : c - KCH) * (16 / ESZ);   // first element of the chunk
    const uint16_t* src = isk ? a.ak + (int64_t)b * a.ak_st + (int64_t)kvh * a.ak_sh + e0
                              : a.av + (int64_t)b * a.av_st + (int64_t)kvh * a.av_sh + e0;
    if constexpr (FP8) {
      const float* sp = isk ? a.c.k_scale : a.c.v_scale;
      const float sc = a.c.scale_mode == 2 ? sp[kvh] : sp[0];
      const u32x2 lo = bf16x8_to_e4m3fn(*reinterpret_cast<const u32x4*>(src), sc);
      const u32x2 hi2 = bf16x8_to_e4m3fn(*reinterpret_cast<const u32x4*>(src + 8), sc);
      return u32x4{lo[0], lo[1], hi2[0], hi2[1]};
    } else {
      return *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto new_row_base = [&]() -> uint8_t* {
    const int64_t blk = new_slot / a.c.block_size;
    return a.c.data + (blk * a.c.sb + (new_slot - blk * a.c.block_size) * a.c.ss + (int64_t)kvh * a.c.sh) * ESZ;
  };

  // ---- an empty key range (no key of the sequence here): empty partials at once, and the
  // new row of a sequence without keys still goes to its slot ----
  if (nt == 0) {                                 // workgroup-uniform
    if (own && wave == 0) {
      uint8_t* row = new_row_base();
      for (int c = lane; c < CH; c += 64) *reinterpret_cast<u32x4*>(row + c * 16) = new_row_chunk(c);
    }
    write_empty_partials<(DK > 256)>(a, q0, 0, min(min(L, a.max_q), ROWS / G), G, kvh, part, DV, NW * 64);
    PA_STAMP_FLUSH(g_phase_stamps, sd::NW)
    return;
  }

  if (!kPatchRow && own) {                       // workgroup-uniform
    uint8_t* row = new_row_base();
    for (int c = threadIdx.x; c < CH; c += NW * 64) *reinterpret_cast<u32x4*>(row + c * 16) = new_row_chunk(c);
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): the row is in L2
    __syncthreads();
  }

  char* ring = smem + wave * WAVE_BYTES;
  const uint8_t* head_base = a.c.data + (int64_t)kvh * a.c.sh * ESZ;

  // lane's source offset (bytes from the tile's first row) for DMA instruction u:
  // 16-byte slot u*64 + lane of the tile holds chunk c of key `key`, swizzled
  const int ssb = (int)(a.c.ss * ESZ);           // bytes between consecutive slots
  auto dma_off = [&](int u, int kmax) {
    const int slot = u * 64 + lane;
    const int key = slot / CH;
    const int c = (slot - key * CH) ^ (FP8 ? fp8_chunk_swz(key) : row_chunk_swz(key));
    return min(key, kmax) * ssb + c * 16;
  };
  constexpr bool kKeepOff = NINS <= 10;          // precomputed offsets (MLA rows: registers are full)
  int off[kKeepOff ? NINS : 1];
#pragma unroll
  for (int u = 0; u < (kKeepOff ? NINS : 0); ++u) off[u] = dma_off(u, TT - 1);

  auto issue = [&](int ti, int stage) {
    char* buf = ring + stage * TILE_BYTES;
    // block_size is a multiple of 16: the tile sits in one block, whose id is
    // wave-uniform and comes in by a scalar load (lgkmcnt, not the DMA's vmcnt)
    const int t0 = __builtin_amdgcn_readfirstlane(start + ti * TT);
    const int64_t blk = load_uniform(btrow + (t0 >> bs_shift));
    const uint8_t* tile = head_base + (blk * a.c.sb + (int64_t)(t0 & bs_mask) * a.c.ss) * ESZ;
    const int kmax = end - 1 - t0;                // keys past the partition re-read its last key
    const bool full = kmax >= TT - 1;
#pragma unroll
    for (int u = 0; u < NINS; ++u) {
      const uint32_t o = (kKeepOff && full) ? off[u] : dma_off(u, kmax);
      if constexpr (NTL) dma16_nt_s(o, tile, lds_addr(buf + u * 1024));
      else dma16_s(o, tile, lds_addr(buf + u * 1024));
    }
  };

  // Every stage of the ring is issued before the first tile is waited for, so that the
  // opening burst requests NST tiles per wave (a single tile per wave leaves HBM half idle
  // until the first ones land).  Order against Q: the compiler does not count the DMA, so
  // the wait it must see for Q (and the new row) is a vmcnt(0), which also covers every DMA
  // issued before it.  DiffKV rows issue the ring first (that vmcnt(0) then waits for the
  // whole prologue, but Q's round trip stays under the burst); MLA rows load Q first and
  // issue the ring after its wait, so tile 0 is computed as soon as it lands instead of
  // after the last prologue stage (MLA B1 step 29.2 -> 28.3 us; DiffKV B1/B8 ~1% slower
  // that way, so they keep the first order).
  constexpr bool kQFirst = DK > 256;
  if constexpr (!kQFirst) {
#pragma unroll
    for (int k = 0; k < NST; ++k)
      if (wave + k * NW < nt) issue(wave + k * NW, k);
  }

  u32x4 nrow[RCH];                               // the owner's new row, loaded with Q
#pragma unroll
  for (int r = 0; r < RCH; ++r) nrow[r] = u32x4{0, 0, 0, 0};
  if (kPatchRow && own) {
#pragma unroll
    for (int r = 0; r < RCH; ++r)
      if (lane + 64 * r < CH) nrow[r] = new_row_chunk(lane + 64 * r);
  }

  if constexpr (!kQFirst) {
    PA_STAMP(1)                                  // ring prologue issued
  }
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
      // fp8 pairs k-steps so that one 16-byte chunk of 16 fp8 values feeds two of them
      const int d0 = FP8 ? (ks >> 1) * 64 + g * 16 + (ks & 1) * 8 : ks * 32 + g * 8;
      u32x4 w = {0, 0, 0, 0};
      if (live) w = *reinterpret_cast<const u32x4*>(qp + d0);
      qreg[rg][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  float kscale = 1.0f, vscale = 1.0f;
  if (FP8 && a.c.scale_mode != 0) {
    kscale = a.c.scale_mode == 2 ? a.c.k_scale[kvh] : a.c.k_scale[0];
    vscale = a.c.scale_mode == 2 ? a.c.v_scale[kvh] : a.c.v_scale[0];
  }
  float sl2 = a.scale * kLog2e * kscale;
  if (sl2 < 0.f) {                               // s * sl2 == (-s) * (-sl2): negate Q (exact)
#pragma unroll
    for (int rg = 0; rg < NR; ++rg)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qreg[rg][ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qreg[rg][ks]) ^ 0x80008000u);
    sl2 = -sl2;
  }
  // last key that every live row of this workgroup sees (tiles ending at or before it
  // need no mask): the live rows' limits min(S - L + qi, end - 1) are smallest for token
  // 0, whose rows are always here (row 0); rows past the query tokens see no key
  const int vis_hi = min(L, a.max_q) > 0 ? min(S - L, end - 1) : 0x7fffffff;

  // lane byte offsets inside a tile: K operand chunk 4ks+g of key n (per ks parity; the
  // rest of ks is an immediate) and the transposed V source (per 16-dim block, mod 4)
  const int sw = FP8 ? fp8_chunk_swz(n) : row_chunk_swz(n);
  int koff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) koff[par] = (n * CH + ((4 * par + g) ^ sw)) * 16;
  int voff[4];
  if constexpr (FP8) {
    // transposing reads from the bf16 V tile: key 4g + n/4, dims 16*db + 4*(n%4)
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) voff[d4] = ((4 * g + (n >> 2)) * VP + 16 * d4 + 4 * (n & 3)) * 2;
  } else {
    const int vkey = 4 * g + (n >> 2);
    const int vsw = row_chunk_swz(vkey);
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
  // Q is complete from here on (and, when the ring went first, the prologue's tiles): the
  // explicit vmcnt waits below count DMA instructions only, and the compiler, which counts
  // only the loads it issued, sees this wait and adds none of its own for Q
  __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)
  PA_STAMP(2)                                    // Q landed
  if constexpr (kQFirst) {
#pragma unroll
    for (int k = 0; k < NST; ++k)
      if (wave + k * NW < nt) issue(wave + k * NW, k);
    PA_STAMP(1)                                  // ring prologue issued
  }
  if (kPatchRow && own && wave == 0) {           // the new row into its cache slot
    uint8_t* row = new_row_base();
#pragma unroll
    for (int r = 0; r < RCH; ++r)
      if (lane + 64 * r < CH) *reinterpret_cast<u32x4*>(row + (lane + 64 * r) * 16) = nrow[r];
  }
  // the last tile's LDS rows from key S-1 on: the new row (see above)
  auto patch_new_row = [&](int stage, int k, const u32x4 (&row)[RCH]) {
    char* buf = ring + stage * TILE_BYTES;
    for (int kk = k; kk < TT; ++kk) {
      const int sw = FP8 ? fp8_chunk_swz(kk) : row_chunk_swz(kk);
#pragma unroll
      for (int r = 0; r < RCH; ++r) {
        const int c = lane + 64 * r;
        if (c < CH) *reinterpret_cast<u32x4*>(buf + (kk * CH + (c ^ sw)) * 16) = row[r];
      }
    }
  };

  auto compute = [&](int ti, int stage) {
    char* buf = ring + stage * TILE_BYTES;
    const int j0 = start + ti * TT;
    f32x4 s[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) s[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FP8) {
      // the tile's fp8 K and V chunks into registers; the stage is then free for the
      // bf16 [key][dim] V tile that the transposing reads need
      u32x4 kw[KS / 2], vw[DV / 64];
#pragma unroll
      for (int j = 0; j < KS / 2; ++j) kw[j] = *reinterpret_cast<const u32x4*>(buf + koff[0] + j * 64);
#pragma unroll
      for (int i = 0; i < DV / 64; ++i) vw[i] = *reinterpret_cast<const u32x4*>(buf + koff[0] + (VOFF / 16 + 4 * i) * 16);
#pragma unroll
      for (int i = 0; i < DV / 64; ++i) {
        const u32x2 t0 = fp8x4_to_bf16x4(vw[i][0]), t1 = fp8x4_to_bf16x4(vw[i][1]);
        const u32x2 t2 = fp8x4_to_bf16x4(vw[i][2]), t3 = fp8x4_to_bf16x4(vw[i][3]);
        char* dst = buf + (n * VP + i * 64 + g * 16) * 2;
        *reinterpret_cast<u32x4*>(dst) = u32x4{t0[0], t0[1], t1[0], t1[1]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{t2[0], t2[1], t3[0], t3[1]};
      }
      // K: one 16-byte chunk (dims 64j + 16g .. +16) feeds k-steps 2j and 2j + 1
#pragma unroll
      for (int j = 0; j < KS / 2; ++j) {
        const u32x4 w = kw[j];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x2 c0 = fp8x4_to_bf16x4(w[2 * h]), c1 = fp8x4_to_bf16x4(w[2 * h + 1]);
          const bf16x8 kop = __builtin_bit_cast(bf16x8, u32x4{c0[0], c0[1], c1[0], c1[1]});
#pragma unroll
          for (int rg = 0; rg < NR; ++rg)
            s[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[rg][2 * j + h], s[rg], 0, 0, 0);
        }
      }
    } else if constexpr (DK > 256) {
      // MLA rows: 18 dependent k-steps on one wave per SIMD.  The K operands are read KPF
      // k-steps ahead of their MFMAs, and a scheduling barrier after each k-step keeps that
      // order (left to itself the compiler reads each operand right before its MFMA, and
      // the chain waits on every LDS read)
      static_assert(NR == 1, "MLA rows: one row group");
      constexpr int KPF = 3;
      bf16x8 kb[KPF + 1];
#pragma unroll
      for (int j = 0; j < KPF; ++j) kb[j] = *reinterpret_cast<const bf16x8*>(buf + koff[j & 1] + (j >> 1) * 128);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int jn = ks + KPF;
        if (jn < KS) kb[jn % (KPF + 1)] = *reinterpret_cast<const bf16x8*>(buf + koff[jn & 1] + (jn >> 1) * 128);
        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks % (KPF + 1)], qreg[0][ks], s[0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(buf + koff[ks & 1] + (ks >> 1) * 128);
#pragma unroll
        for (int rg = 0; rg < NR; ++rg)
          s[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[rg][ks], s[rg], 0, 0, 0);
      }
    }
    s16x4 pb[NR];
    // every live row sees every key of the tile: no mask, and the scale (>= 0 here)
    // folds into the max and into one fma per score
    const bool nomask = j0 + TT - 1 <= vis_hi;
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      float x[4];
      float mx = kNegInf;
      if (nomask) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rg][i]);
        mx = max_over_groups(mx) * sl2;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 4 * g + i;
          x[i] = (j <= hi[rg]) ? s[rg][i] * sl2 : kNegInf;
          mx = fmaxf(mx, x[i]);
        }
        mx = max_over_groups(mx);
      }
      // lazy rescaling: the running max used as the exp2 base moves only when the
      // tile's max exceeds it by more than 8 (log2 units), so p <= 256 and the
      // accumulator is rescaled on few tiles; (m, l, acc) stay consistent throughout
      const float mn = fmaxf(m[rg], mx);
      const bool grow = mn > m[rg] + 8.0f;        // true on the first visible key (m = -inf)
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2(m[rg] - mn) : 1.0f;
        m[rg] = grow ? mn : m[rg];
        l[rg] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rg][db] *= alpha;
      }
      const float base = (m[rg] == kNegInf) ? 0.f : m[rg];
      float p[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(nomask ? __builtin_fmaf(s[rg][i], sl2, -base) : x[i] - base);
        ps += p[i];
      }
      l[rg] += ps;
      u32x2 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      pb[rg] = __builtin_bit_cast(s16x4, pk);
    }
    __builtin_amdgcn_wave_barrier();
    const char* vsrc = buf;                       // fp8: the bf16 V tile written above
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const s16x4 vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vsrc + voff[db & 3] + (db >> 2) * 128));   // +64 dims
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        acc[rg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pb[rg], acc[rg][db], 0, 0, 0);
    }
  };

  // ---- this wave's tiles wave, wave+NW, ...: one consumed while up to NST-1 fly ----
  {
    int stage = 0;
    for (int ti = wave; ti < nt; ti += NW) {
      // tile to start now, into the slot freed last step (the first step's came with the prologue)
      const int tn = ti + (NST - 1) * NW;
      if (ti != wave && tn < nt) issue(tn, (stage + NST - 1) % NST);
      // tiles issued after ti: min(NST-1, remaining) -> wait until only those are in flight
      const bool patch = kPatchRow && own && ti == nt - 1;   // wave-uniform: the owner's last tile
      const int later = min(NST - 1, (nt - 1 - ti) / NW);
      static_assert(NST <= 4, "waits below cover up to 3 tiles in flight");
      if (NST > 3 && later >= 3) wait_vm<(NST > 3 ? 3 : 0) * NINS>();
      else if (NST > 2 && later >= 2) wait_vm<(NST > 2 ? 2 : 0) * NINS>();
      else if (later >= 1) wait_vm<NINS>();
      else wait_vm<0>();
      PA_STAMP_TILE_WAITED
      if (patch) patch_new_row(stage, S - 1 - (start + ti * TT), nrow);
      compute(ti, stage);
      PA_STAMP_TILE_DONE
      stage = (stage + 1) % NST;
    }
  }

  // ---- merge the NW waves: each writes its scaled accumulator to its own LDS slab
  // (independent stores, no read-modify-write chain), then all threads sum the slabs
  // in wave order and write the partials of the live rows ----
  PA_STAMP(60)
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) l[rg] = sum_over_groups(l[rg]);
  __syncthreads();                                // rings are dead from here on
  PA_STAMP(61)
  float* mw = reinterpret_cast<float*>(smem);     // [NW][ROWS]
  float* lw = mw + NW * ROWS;                     // [NW][ROWS]
  float* slab = lw + NW * ROWS;                   // [NW][ROWS][MERGE_PITCH]
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
    f[rg] = (M == kNegInf || Ls == 0.f) ? 0.f : fast_exp2(m[rg] - M) / Ls * vscale;
  }
#pragma unroll
  for (int rg = 0; rg < NR; ++rg)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4*>(slab + (wave * ROWS + rg * 16 + n) * MERGE_PITCH + db * 16 + 4 * g) =
          acc[rg][db] * f[rg];
  __syncthreads();
  const int64_t Hq = a.num_q_heads;
  const int live_rows = min(min(L, a.max_q) * G, ROWS);   // row r is live iff r / G < min(L, max_q)
  for (int idx = threadIdx.x; idx < live_rows * (DV / 4); idx += NW * 64) {
    const int r = idx / (DV / 4), c4 = idx - r * (DV / 4);
    const int qi = r / G, hh = r - qi * G;
    const int64_t tok = q0 + qi, head = kvh * G + hh;
    f32x4 v = *reinterpret_cast<const f32x4*>(slab + r * MERGE_PITCH + c4 * 4);
    for (int w = 1; w < NW; ++w) v += *reinterpret_cast<const f32x4*>(slab + (w * ROWS + r) * MERGE_PITCH + c4 * 4);
    store_partial4<(DK > 256)>(a.part_out + ((tok * Hq + head) * P + part) * DV + c4 * 4, v);
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
      store_partial1<(DK > 256)>(a.part_lse + (tok * Hq + head) * P + part,
                     (M == kNegInf || Ls == 0.f) ? kNegInf : (M + __builtin_log2f(Ls)) * kLn2);
    }
  }
  PA_STAMP_FLUSH(g_phase_stamps, sd::NW)
}

// Eligible shapes: DiffKV rows, bf16 or fp8 (up to 32 rows per KV head), and bf16 MLA
// rows (one row group), with a power-of-two block size of at least 16.
static bool dma_is_diffkv(const SplitArgs& a) { return a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192; }
static bool dma_is_mla(const SplitArgs& a) { return a.c.dk == 576 && a.c.dv == 512 && a.c.v_off == 0; }
constexpr bool kFp8Nontemporal = true;
constexpr int kFp8Stages = 3, kFp8MinWaves = 2;   // ring depth; waves per SIMD the registers must allow

bool splitkv_dma_eligible(const SplitArgs& a) {
  const int bs = a.c.block_size;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int rows = a.max_q * G;
  if ((bs & (bs - 1)) != 0 || bs < sd::TT) return false;
  return (dma_is_diffkv(a) && rows <= 32) || (a.c.esize == 2 && dma_is_mla(a) && rows <= 16);
}

bool splitkv_append_fusable(const SplitArgs& a) {
  auto al = [](const void* p, int n) { return ((uintptr_t)p % n) == 0; };
  const bool mla = a.c.dk == 576 && a.c.dv == 512 && a.c.v_off == 0;
  bool ok = a.qsl == nullptr && splitkv_uses_dma(a) && al(a.ak, 16) && a.ak_st % 8 == 0 && a.ak_sh % 8 == 0;
  if (a.av) ok = ok && !mla && al(a.av, 16) && a.av_st % 8 == 0 && a.av_sh % 8 == 0;
  else ok = ok && mla;                           // a DiffKV row needs its V columns
  return ok;
}

void launch_splitkv_dma(const SplitArgs& a, hipStream_t s) {
  dim3 grid(a.num_partitions, a.c.num_kv_heads, a.num_seqs), block(sd::NW * 64);
  const int rows = a.max_q * (a.num_q_heads / a.c.num_kv_heads);
  if (dma_is_mla(a))
    hipLaunchKernelGGL((splitkv_dma_kernel<576, 512, 0, 1, 2, 1, false, true>), grid, block, 0, s, a);
  else if (a.c.esize == 1 && rows <= 16)
    hipLaunchKernelGGL((splitkv_dma_kernel<192, 128, 192, 1, kFp8Stages, kFp8MinWaves, true, kFp8Nontemporal>), grid, block, 0, s, a);
  else if (a.c.esize == 1)
    hipLaunchKernelGGL((splitkv_dma_kernel<192, 128, 192, 2, kFp8Stages, kFp8MinWaves, true, kFp8Nontemporal>), grid, block, 0, s, a);
  else if (rows <= 16)
    hipLaunchKernelGGL((splitkv_dma_kernel<192, 128, 192, 1, 2, 2, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((splitkv_dma_kernel<192, 128, 192, 2, 2, 2, false, true>), grid, block, 0, s, a);
}

}  // namespace pa

#ifdef PA_PHASE_STAMPS
// Copies the first `words` stamp words (at most kStampWaves * 64) to host memory `dst`;
// returns the hipError_t of the copy.
extern "C" int attn_phase_stamps_read(void* dst, size_t words) {
  if (!dst || words > (size_t)pa::kStampWaves * 64) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(pa::g_phase_stamps), words * 4, 0, hipMemcpyDeviceToHost);
}
#endif
