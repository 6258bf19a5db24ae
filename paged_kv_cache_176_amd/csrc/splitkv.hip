// Split-KV paged attention: per (partition, KV head, sequence) one workgroup
// computes the softmax-normalised partial output and log-sum-exp of every query
// row that uses this KV head, over the partition's key range.  This file holds
// the dispatch (launch_splitkv_partial), the merge kernel and the register-prefetch
// partial kernel; the shapes that matter most have faster kernels:
//   splitkv_wide.hip  fp8 DiffKV rows, 17-32 rows per KV head (verify)
//   splitkv_dma.hip   bf16 DiffKV up to 32 rows, fp8 DiffKV up to 16 rows, bf16 MLA
//                     up to 16 rows (block size a power of two >= 16)
//   splitkv_tokens.hip  bf16 MLA with 2 or more query tokens (verify), up to 16 heads
//                     per KV head (block size a power of two >= 16)
// and the kernel below serves everything else (other block sizes, 33-64 rows).
//
// The "rows" of a KV head are its query tokens x its GQA query heads, row r =
// token_index * G + head_in_group:
//   decode  1 token x G heads        (G = 8 for MiMo's 32/4 heads)
//   verify  L tokens x G heads       (L = 4: 3 drafts + 1, causal among themselves)
//   MLA     1 token x 12 heads over one 576-wide latent row, V = its first 512
// Prior art on the pages: split-KV two-stage decode with a device-side,
// graph-stable split count (vLLM PR #50371, review thread), split-KV kept for
// multi-token verify and one program per whole verify so every row of a KV head
// shares one K/V read (diffbot MiMo-V2.6-Flash model card, "Benchmarks" and
// "What the kernels do").
//
// gfx950 mapping of the register-prefetch kernel (wave64, MFMA):
//   QK^T   S^T[16 keys x 16 rows] += K[16 keys x 32 dims] * Q^T[32 dims x 16 rows]
//          v_mfma_f32_16x16x32_bf16.  The K operand (lane: key l%16, dims
//          8*(l/16)..+8) is exactly one 16-byte load of the cache row, so K goes
//          HBM -> VGPR -> MFMA with no LDS.  Q lives in VGPRs for the whole run.
//   softmax each lane holds 4 keys of one row; the row max needs two cross-group
//          exchanges (v_permlane32_swap / v_permlane16_swap).  exp2 with log2(e)
//          folded into the scale.
//   PV     O^T[16 dims x 16 rows] += V^T[16 dims x 16 keys] * P^T[16 keys x 16 rows]
//          v_mfma_f32_16x16x16_bf16.  P^T is the lane's own 4 probabilities
//          (same lane layout as the S^T output); V^T comes from a per-wave LDS
//          tile through ds_read_b64_tr_b16 (a transposing LDS read).
//   fp8 K/V are converted to bf16 in the load path (exact); the K scale is
//   applied to the fp32 scores, the V scale to the final output.
// Work split: the workgroup's NW waves take interleaved 16-key tiles of the
// partition through a ring of 2-3 register buffers, then merge their (m, l, acc)
// through LDS in a fixed order (deterministic).
#include "common.hpp"
#include "kernels.hpp"

namespace pa {

template <int DK, int DV, int VOFF, bool FP8>
struct TileRegs {
  static constexpr bool kVInK = !FP8 && (VOFF + DV <= DK) && (VOFF % 32 == 0);
  static constexpr int kK = FP8 ? DK / 64 : DK / 32;          // 16-byte K loads per lane
  static constexpr int kV = kVInK ? 1 : (FP8 ? DV / 64 : DV / 32);   // 16-byte V loads per lane
  u32x4 k[kK];
  u32x4 v[kV];
};

// BLK16: block_size is a multiple of 16, so a 16-key tile (tiles start at multiples
// of 16) sits in one block and its table entry is wave-uniform.
template <int DK, int DV, int VOFF, int NR, bool FP8, int NW, bool BLK16>
__global__ __launch_bounds__(NW * 64, (FP8 && NR == 2) ? 2 : 1) void splitkv_partial_kernel(SplitArgs a) {
  using Regs = TileRegs<DK, DV, VOFF, FP8>;
  constexpr int NBUF = (FP8 && NR == 1) ? 3 : 2;  // fp8 tiles are half the bytes: two in flight where registers allow
  constexpr int KS = DK / 32;        // MFMA k-steps of QK^T
  constexpr int DB = DV / 16;        // 16-dim blocks of PV
  constexpr int VP = DV + 16;        // LDS row pitch of the V tile (elements), 32 B pad
  constexpr int ROWS = NR * 16;
  constexpr int VTILE = 16 * VP;     // elements per wave's V tile
  constexpr int MERGE_PITCH = DV + 4;
  constexpr int LDS_V = NW * VTILE * 2;
  constexpr int LDS_M = NW * ROWS * 2 * 4 + NW * ROWS * MERGE_PITCH * 4;
  constexpr int LDS_BYTES = LDS_V > LDS_M ? LDS_V : LDS_M;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int P = a.num_partitions;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int S = a.seq_lens[b];
  const int q0 = a.qsl ? a.qsl[b] : b;
  const int L = a.qsl ? a.qsl[b + 1] - q0 : 1;
  const int chunk = ceil_div(ceil_div(S, active_splits(a.pol, S, P)), 16) * 16;
  const int start = min(part * chunk, S);
  const int end = min(start + chunk, S);
  const int nt = ceil_div(end - start, 16);

  // ---- Q rows of this KV head into registers (B operand of QK^T) ----
  bf16x8 qreg[NR][KS];
  int hi[NR];                                   // last visible key of the lane's row
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const int r = rg * 16 + n;
    const int qi = r / G, hh = r - qi * G;
    const bool live = qi < L && qi < a.max_q;
    hi[rg] = live ? min(S - L + qi, end - 1) : -1;
    const uint16_t* qp = a.q + (int64_t)(q0 + (live ? qi : 0)) * a.q_st + (int64_t)(kvh * G + hh) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // k-step ks covers dims {base(ks, g') .. +8 : g' = 0..3}; fp8 pairs k-steps so
      // that one 16-byte load of 16 fp8 values feeds two of them
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
  const float sl2 = a.scale * kLog2e * kscale;
  // Q is complete in registers from here on.  Without this wait the compiler, which
  // counts vector loads in issue order, would wait at Q's first use in the loop for
  // every K/V load issued after it, emptying the prefetch on each tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  f32x4 acc[NR][DB];
  float m[NR], l[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    m[rg] = kNegInf;
    l[rg] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * VTILE;
  const uint8_t* cbase = a.c.data;
  const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;
  const int esz = FP8 ? 1 : 2;

  // With BLK16 the tile's block id comes in by a scalar load, which leaves the
  // vector memory counter to the K/V prefetch alone; otherwise each lane looks up
  // its own key's block (and that load's wait also drains the prefetch).
  auto load_tile = [&](Regs& R, int ti) {
    int64_t blk;
    int pos;
    if constexpr (BLK16) {
      const int j0 = __builtin_amdgcn_readfirstlane(start + ti * 16);
      blk = load_uniform(btrow + j0 / a.c.block_size);
      pos = j0 % a.c.block_size + min(n, S - 1 - j0);      // clamp: never past the sequence
    } else {
      const int j = min(start + ti * 16 + n, S - 1);
      blk = btrow[j / a.c.block_size];
      pos = j % a.c.block_size;
    }
    const uint8_t* row = cbase + (blk * a.c.sb + pos * a.c.ss + (int64_t)kvh * a.c.sh) * esz;
    // K/V rows are read once per launch: nontemporal loads (the nt bit) stream them
    // past the caches, measured ~15% more read bandwidth than default loads here
#pragma unroll
    for (int i = 0; i < Regs::kK; ++i)
      R.k[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(row + (FP8 ? i * 64 + g * 16 : (i * 32 + g * 8) * 2)));
    if constexpr (!Regs::kVInK) {
#pragma unroll
      for (int i = 0; i < Regs::kV; ++i)
        R.v[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(row + (FP8 ? VOFF + i * 64 + g * 16 : (VOFF + i * 32 + g * 8) * 2)));
    }
    // keep the scheduler from sinking these loads below the next tile's compute
    // (it would then wait for that tile before issuing them: one tile in flight)
    if constexpr (NR != 4) __builtin_amdgcn_sched_barrier(0);
  };

  auto compute_tile = [&](const Regs& R, int ti) {
    const int j0 = start + ti * 16;
    // V rows of the 16 keys into this wave's LDS tile, as bf16 [key][dim]
    __builtin_amdgcn_wave_barrier();
    if constexpr (Regs::kVInK) {
#pragma unroll
      for (int i = 0; i < DV / 32; ++i)
        *reinterpret_cast<u32x4*>(vt + n * VP + i * 32 + g * 8) = R.k[VOFF / 32 + i];
    } else if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < Regs::kV; ++i) *reinterpret_cast<u32x4*>(vt + n * VP + i * 32 + g * 8) = R.v[i];
    } else {
#pragma unroll
      for (int i = 0; i < Regs::kV; ++i) {
        u32x4 lo, hi2;
        u32x2 t0 = fp8x4_to_bf16x4(R.v[i][0]), t1 = fp8x4_to_bf16x4(R.v[i][1]);
        u32x2 t2 = fp8x4_to_bf16x4(R.v[i][2]), t3 = fp8x4_to_bf16x4(R.v[i][3]);
        lo = u32x4{t0[0], t0[1], t1[0], t1[1]};
        hi2 = u32x4{t2[0], t2[1], t3[0], t3[1]};
        *reinterpret_cast<u32x4*>(vt + n * VP + i * 64 + g * 16) = lo;
        *reinterpret_cast<u32x4*>(vt + n * VP + i * 64 + g * 16 + 8) = hi2;
      }
    }
    // S^T = K Q^T
    f32x4 s[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) s[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 kop;
      if constexpr (FP8) {
        const u32x4& w = R.k[ks >> 1];
        u32x2 c0 = fp8x4_to_bf16x4((ks & 1) ? w[2] : w[0]);
        u32x2 c1 = fp8x4_to_bf16x4((ks & 1) ? w[3] : w[1]);
        kop = __builtin_bit_cast(bf16x8, u32x4{c0[0], c0[1], c1[0], c1[1]});
      } else {
        kop = __builtin_bit_cast(bf16x8, R.k[ks]);
      }
#pragma unroll
      for (int rg = 0; rg < NR; ++rg) s[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[rg][ks], s[rg], 0, 0, 0);
    }
    // online softmax; lane holds keys j0+4g+i (i<4) of row rg*16+n
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
      const float base = (mn == kNegInf) ? 0.f : mn;      // all masked so far: p = 0, no NaN
      const float alpha = fast_exp2(m[rg] - base);          // m = -inf -> 0
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
    // O^T += V^T P^T
    __builtin_amdgcn_wave_barrier();
    const int tr_row = 4 * g + (n >> 2), tr_col = 4 * (n & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const s16x4 vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vt + tr_row * VP + db * 16 + tr_col));
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        acc[rg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pb[rg], acc[rg][db], 0, 0, 0);
    }
  };

  // ---- main loop: this wave's tiles wave, wave+NW, ... through a ring of NBUF
  // register buffers, NBUF - 1 tiles in flight while one is computed.  Loads are
  // issued unconditionally (indices past the end re-read the partition's last tile,
  // which is in cache) so that every compute waits for exactly its own buffer: a
  // skipped load on some path would make the compiler's in-order load counting
  // wait for the whole ring.
  if constexpr (NR == 4) {
    // 64 rows fill the register file: the unconditional form spills here, so the
    // loads past the end are skipped instead
    Regs b0, b1;
    int ti = wave;
    if (ti < nt) load_tile(b0, ti);
    while (ti < nt) {
      const int t1 = ti + NW;
      if (t1 < nt) load_tile(b1, t1);
      compute_tile(b0, ti);
      if (t1 >= nt) break;
      const int t2 = t1 + NW;
      if (t2 < nt) load_tile(b0, t2);
      compute_tile(b1, t1);
      ti = t2;
    }
  } else if (wave < nt) {
    // one exit per loop (a break in mid-body gives the structurizer an extra edge
    // into the loop header that carries the previous half's loads as pending)
    auto ahead = [&](int t) { return min(t, nt - 1); };
    int ti = wave;
    if constexpr (NBUF == 2) {
      Regs b0, b1;
      load_tile(b0, ti);
      while (ti + NW < nt) {
        load_tile(b1, ti + NW);
        compute_tile(b0, ti);
        load_tile(b0, ahead(ti + 2 * NW));
        compute_tile(b1, ti + NW);
        ti += 2 * NW;
      }
      if (ti < nt) compute_tile(b0, ti);
    } else {
      static_assert(NBUF == 3, "register ring of 2 or 3 tiles");
      Regs b0, b1, b2;
      load_tile(b0, ti);
      load_tile(b1, ahead(ti + NW));
      while (ti + 2 * NW < nt) {
        load_tile(b2, ti + 2 * NW);
        compute_tile(b0, ti);
        load_tile(b0, ahead(ti + 3 * NW));
        compute_tile(b1, ti + NW);
        load_tile(b1, ahead(ti + 4 * NW));
        compute_tile(b2, ti + 2 * NW);
        ti += 3 * NW;
      }
      if (ti < nt) compute_tile(b0, ti);
      if (ti + NW < nt) compute_tile(b1, ti + NW);
    }
  }

  // ---- merge the NW waves: each writes its scaled accumulator to its own LDS slab,
  // then all threads sum the slabs in wave order and write the live rows' partials ----
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) l[rg] = sum_over_groups(l[rg]);
  __syncthreads();                                   // V tiles are dead from here on
  float* mw = reinterpret_cast<float*>(smem);        // [NW][ROWS]
  float* lw = mw + NW * ROWS;                        // [NW][ROWS]
  float* slab = lw + NW * ROWS;                      // [NW][ROWS][MERGE_PITCH]
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
    store_partial4<false>(a.part_out + ((tok * Hq + head) * P + part) * DV + c4 * 4, v);
  }
  if (threadIdx.x < ROWS) {
    const int r = threadIdx.x;
    const int qi = r / G, hh = r - qi * G;
    if (qi < L && qi < a.max_q) {
      float M = kNegInf, Ls = 0.f;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * ROWS + r]);
      if (M != kNegInf)
        for (int w = 0; w < NW; ++w) Ls += lw[w * ROWS + r] * fast_exp2(mw[w * ROWS + r] - M);
      const float lse = (M == kNegInf || Ls == 0.f) ? kNegInf : (M + __builtin_log2f(Ls)) * kLn2;
      const int64_t tok = q0 + qi, head = kvh * G + hh;
      store_partial1<false>(a.part_lse + (tok * Hq + head) * P + part, lse);
    }
  }
}

// ---------------------------------------------------------------------------
// Merge (attn_merge_lse, and the second kernel of attn_decode_splitkv / attn_verify).
// Grid: (row * Hq + head, slice of 4*SLOTS output dims).  The workgroup's threads
// are SLOTS float4 columns x NG partition groups; each thread's partial loads are
// issued before the log-sum-exp pass; group sums are combined in LDS in a fixed
// order.  w_p = exp(lse_p - M), out = sum w_p o_p / sum w_p, lse = M + ln sum w_p;
// M = -inf (no partition saw a key) gives out = 0, lse = -inf, never NaN.
template <int NT, int SLOTS>
__global__ __launch_bounds__(NT) void merge_kernel(MergeArgs a) {
  constexpr int NG = NT / SLOTS;
  extern __shared__ float wsh[];                     // [P] weights
  __shared__ float red[NT / 64];
  __shared__ f32x4 gs[NG][SLOTS];
  const int64_t rh = blockIdx.x;                     // row * Hq + head
  const int P = a.num_partitions, DV = a.dv;
  // partitions past the row's active count are empty: not read
  const int Pa = a.seq_lens ? active_splits(a.pol, a.seq_lens[rh / a.num_q_heads], P) : P;
  const int slot = threadIdx.x % SLOTS, grp = threadIdx.x / SLOTS;
  const int c4 = blockIdx.y * SLOTS + slot;          // float4 column
  const bool col_ok = c4 * 4 < DV;
  const float* po = a.part_out + rh * P * DV + c4 * 4;
  // this thread's first PRE partials are loaded before the log-sum-exp pass, so that
  // for P <= PRE * NG (256 partitions) the whole merge waits on memory once
  constexpr int PRE = 8;
  f32x4 pre[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int p = grp + k * NG;
    pre[k] = (col_ok && p < Pa) ? load_partial4(po + (int64_t)p * DV) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* lse = a.part_lse + rh * P;
  float mx = kNegInf;
  for (int p = threadIdx.x; p < Pa; p += NT) mx = fmaxf(mx, lse[p]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  float M = kNegInf;
  for (int w = 0; w < NT / 64; ++w) M = fmaxf(M, red[w]);
  const float sk = a.sinks ? a.sinks[rh % a.num_q_heads] : kNegInf;   // sink: one more term, value 0
  M = fmaxf(M, sk);
  __syncthreads();
  float sum = 0.f;
  for (int p = threadIdx.x; p < Pa; p += NT) {
    const float w = (M == kNegInf) ? 0.f : fast_exp2((lse[p] - M) * kLog2e);
    wsh[p] = w;
    sum += w;
  }
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < NT / 64; ++w) tot += red[w];
  tot += sk == kNegInf ? 0.f : fast_exp2((sk - M) * kLog2e);
  const bool empty = (M == kNegInf || tot == 0.f);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int p = grp + k * NG;
    if (p < Pa) acc += pre[k] * wsh[p];
  }
  if (col_ok)
    for (int p = grp + PRE * NG; p < Pa; p += NG) acc += load_partial4(po + (int64_t)p * DV) * wsh[p];
  gs[grp][slot] = acc;
  __syncthreads();
  if (threadIdx.x < SLOTS && c4 * 4 < DV) {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int g2 = 0; g2 < NG; ++g2) t += gs[g2][slot];
    t *= empty ? 0.f : 1.0f / tot;
    u32x2 pk = {pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
    *reinterpret_cast<u32x2*>(a.out + rh * DV + c4 * 4) = pk;
  }
  if (a.out_lse && blockIdx.y == 0 && threadIdx.x == 0) a.out_lse[rh] = empty ? kNegInf : M + __builtin_logf(tot);
}

// Merge for few partitions (P <= PMAX): one thread per (row * Hq + head, float4
// column), all of its P log-sum-exps and partial float4s loaded at once, no LDS and no
// barrier.  32 consecutive threads share a row-head (broadcast log-sum-exp loads) and
// read 512 contiguous bytes of each partial.  Same arithmetic as merge_kernel; the
// partial sums are added in partition order.
template <int PMAX>
__global__ __launch_bounds__(64) void merge_few_kernel(MergeArgs a) {
  const int P = a.num_partitions, DV = a.dv, c4n = a.dv / 4;
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (int64_t)a.rows * a.num_q_heads * c4n) return;
  const int64_t rh = idx / c4n;
  const int c4 = (int)(idx - rh * c4n);
  const float* lse = a.part_lse + rh * P;
  const float* po = a.part_out + rh * P * DV + c4 * 4;
  // partitions past the row's active count are empty: not read
  const int Pa = a.seq_lens ? active_splits(a.pol, a.seq_lens[rh / a.num_q_heads], P) : P;
  float lp[PMAX];
  f32x4 op[PMAX];
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    lp[p] = p < Pa ? load_partial1(lse + p) : kNegInf;
    op[p] = p < Pa ? load_partial4(po + (int64_t)p * DV) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float M = kNegInf;
#pragma unroll
  for (int p = 0; p < PMAX; ++p) M = fmaxf(M, lp[p]);
  const float sk = a.sinks ? a.sinks[rh % a.num_q_heads] : kNegInf;   // sink: one more term, value 0
  M = fmaxf(M, sk);
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != kNegInf) {
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
      const float w = p < Pa ? fast_exp2((lp[p] - M) * kLog2e) : 0.f;
      tot += w;
      acc += op[p] * w;
    }
  }
  tot += sk == kNegInf ? 0.f : fast_exp2((sk - M) * kLog2e);
  const bool empty = (M == kNegInf || tot == 0.f);
  acc *= empty ? 0.f : 1.0f / tot;
  *reinterpret_cast<u32x2*>(a.out + rh * DV + c4 * 4) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  if (a.out_lse && c4 == 0) a.out_lse[rh] = empty ? kNegInf : M + __builtin_logf(tot);
}

// ---------------------------------------------------------------------------
template <int DK, int DV, int VOFF, int NR, bool FP8, int NW>
struct SplitKernel {
  static constexpr int kRows = NR * 16;
  static constexpr int kVTile = 16 * (DV + 16);
  static constexpr int kLdsV = NW * kVTile * 2;
  static constexpr int kLdsM = NW * kRows * 2 * 4 + NW * kRows * (DV + 4) * 4;
  static constexpr int kLds = kLdsV > kLdsM ? kLdsV : kLdsM;
  static void launch(const SplitArgs& a, hipStream_t s) {
    dim3 grid(a.num_partitions, a.c.num_kv_heads, a.num_seqs), block(NW * 64);
    if ((a.c.block_size & 15) == 0)
      hipLaunchKernelGGL((splitkv_partial_kernel<DK, DV, VOFF, NR, FP8, NW, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((splitkv_partial_kernel<DK, DV, VOFF, NR, FP8, NW, false>), grid, block, 0, s, a);
  }
};

static int rows_groups(const SplitArgs& a) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int rows = a.max_q * G;
  return rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 64 ? 4 : 0;
}

static bool is_diffkv(const SplitArgs& a) { return a.c.dk == 192 && a.c.dv == 128 && a.c.v_off == 192; }
static bool is_mla(const SplitArgs& a) { return a.c.dk == 576 && a.c.dv == 512 && a.c.v_off == 0 && a.c.esize == 2; }

// Dispatch on (layout, dtype, row groups); F is called with the kernel type.
template <typename F>
static bool dispatch(const SplitArgs& a, F&& f) {
  const int nr = rows_groups(a);
  const bool fp8 = a.c.esize == 1;
  if (nr == 0) return false;
  if (is_diffkv(a)) {
    if (fp8) {
      if (nr == 1) f(SplitKernel<192, 128, 192, 1, true, 4>{});
      else if (nr == 2) f(SplitKernel<192, 128, 192, 2, true, 4>{});
      else f(SplitKernel<192, 128, 192, 4, true, 4>{});
    } else {
      if (nr == 1) f(SplitKernel<192, 128, 192, 1, false, 4>{});
      else if (nr == 2) f(SplitKernel<192, 128, 192, 2, false, 4>{});
      else f(SplitKernel<192, 128, 192, 4, false, 4>{});
    }
    return true;
  }
  if (is_mla(a) && nr == 1) {
    f(SplitKernel<576, 512, 0, 1, false, 4>{});
    return true;
  }
  return false;
}

bool splitkv_supported(const SplitArgs& a) {
  return splitkv_tokens_eligible(a) || dispatch(a, [](auto) {});
}

bool splitkv_uses_dma(const SplitArgs& a) { return !splitkv_wide_eligible(a) && splitkv_dma_eligible(a); }

bool launch_splitkv_partial(const SplitArgs& a, hipStream_t s) {
  if (splitkv_tokens_eligible(a)) {
    launch_splitkv_tokens(a, s);
    return true;
  }
  if (splitkv_wide_eligible(a)) {
    launch_splitkv_wide(a, s);
    return true;
  }
  if (splitkv_dma_eligible(a)) {
    launch_splitkv_dma(a, s);
    return true;
  }
  return dispatch(a, [&](auto k) { decltype(k)::launch(a, s); });
}

bool launch_merge(const MergeArgs& a, hipStream_t s) {
  constexpr int NT = 256, SLOTS = 8;
  const int64_t n = (int64_t)a.rows * a.num_q_heads;
  if (n == 0) return true;
  if (a.num_partitions <= 32 && a.dv % 4 == 0) {
    const unsigned blocks = (unsigned)((n * (a.dv / 4) + 63) / 64);
    if (a.num_partitions <= 8) hipLaunchKernelGGL(merge_few_kernel<8>, dim3(blocks), dim3(64), 0, s, a);
    else if (a.num_partitions <= 16) hipLaunchKernelGGL(merge_few_kernel<16>, dim3(blocks), dim3(64), 0, s, a);
    else hipLaunchKernelGGL(merge_few_kernel<32>, dim3(blocks), dim3(64), 0, s, a);
    return true;
  }
  const int slices = (a.dv / 4 + SLOTS - 1) / SLOTS;
  hipLaunchKernelGGL((merge_kernel<NT, SLOTS>), dim3((unsigned)n, slices), dim3(NT),
                     a.num_partitions * sizeof(float), s, a);
  return true;
}

}  // namespace pa
