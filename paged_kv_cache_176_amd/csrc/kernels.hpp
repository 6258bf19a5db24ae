// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Host-side argument checking is done before these are called; the launchers
// only pick a template instance and enqueue on the given stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pa {

struct CacheView {
  uint8_t* data;        // base of the cache (bytes)
  int32_t num_blocks, block_size, num_kv_heads, row_dim;
  int32_t dk, dv, v_off;
  int64_t sb, ss, sh;   // strides in elements
  int32_t esize;        // 2 (bf16) or 1 (fp8)
  int32_t scale_mode;   // 0 none, 1 per tensor, 2 per head
  const float* k_scale;
  const float* v_scale;
};

struct CacheWriteArgs {
  const uint16_t* key; int64_t k_st, k_sh;
  const uint16_t* value; int64_t v_st, v_sh;   // value may be null
  const int64_t* slots; int32_t num_tokens;
  CacheView c;
};

// Returns false if no kernel instance matches (caller reports UNSUPPORTED).
bool launch_cache_write(const CacheWriteArgs& a, hipStream_t s);

// Device-side split policy (context buckets -> active partitions), one table read by
// every partial kernel and by the merge: a sequence of seq_len S uses the first
// active_splits(pol, S, P) of the launch's P partitions, the others come out empty.
constexpr int kMaxSplitBuckets = 8;
struct SplitPolicy {
  int32_t n;                            // buckets in use; 0: all P partitions active
  int32_t max_len[kMaxSplitBuckets];    // ascending upper bounds (inclusive)
  int32_t splits[kMaxSplitBuckets];
};
__host__ __device__ inline int active_splits(const SplitPolicy& pol, int S, int P) {
  if (pol.n <= 0) return P;
  int k = pol.splits[pol.n - 1];
  for (int i = pol.n - 1; i >= 0; --i)
    if (S <= pol.max_len[i]) k = pol.splits[i];   // ends on the first bucket holding S
  return k < 1 ? 1 : (k > P ? P : k);
}

struct SplitArgs {
  const uint16_t* q; int64_t q_st, q_sh;
  const int32_t* qsl;       // null: row b is sequence b with one query
  int32_t num_seqs, num_q_heads, max_q;
  CacheView c;
  const int32_t* bt; int32_t bt_stride;
  const int32_t* seq_lens;
  float scale;
  int32_t num_partitions;
  SplitPolicy pol;
  float* part_out; float* part_lse;
  int32_t rows;             // total query rows (tokens)
  // decode only: token b's new K/V row, written into slot aslot[b] (-1: none) by the
  // workgroup whose key range holds key seq_len-1, before that workgroup reads any
  // key.  aslot null: no write.  av null: K columns only (MLA).
  const int64_t* aslot;
  const uint16_t* ak; int64_t ak_st, ak_sh;
  const uint16_t* av; int64_t av_st, av_sh;
};

// Partials of a workgroup whose key range is empty (a sequence with no keys, a partition past
// its end, or one a split policy leaves unused): output 0 and lse -inf for query tokens
// tok_lo .. tok_lo + ntok - 1 of the sequence (starting at q0), heads kvh*G .. kvh*G + G - 1.
// Written at once, without the kernel's load pipeline.
template <bool WT>
__device__ __forceinline__ void write_empty_partials(const SplitArgs& a, int q0, int tok_lo, int ntok, int G, int kvh,
                                                     int part, int dv, int nthreads) {
  const int64_t Hq = a.num_q_heads, P = a.num_partitions;
  const int rows = ntok * G, c4n = dv / 4;
  for (int idx = threadIdx.x; idx < rows * c4n; idx += nthreads) {
    const int r = idx / c4n, c4 = idx - r * c4n;
    const int qi = r / G, hh = r - qi * G;
    const int64_t rh = (int64_t)(q0 + tok_lo + qi) * Hq + kvh * G + hh;
    store_partial4<WT>(a.part_out + (rh * P + part) * dv + c4 * 4, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  for (int r = threadIdx.x; r < rows; r += nthreads) {
    const int qi = r / G, hh = r - qi * G;
    const int64_t rh = (int64_t)(q0 + tok_lo + qi) * Hq + kvh * G + hh;
    store_partial1<WT>(a.part_lse + rh * P + part, -__builtin_inff());
  }
}

bool splitkv_supported(const SplitArgs& a);
bool launch_splitkv_partial(const SplitArgs& a, hipStream_t s);
// 32-row fp8 variant on 32x32 MFMA tiles (splitkv_wide.hip)
bool splitkv_wide_eligible(const SplitArgs& a);
void launch_splitkv_wide(const SplitArgs& a, hipStream_t s);
// LDS-streamed variant for bf16 rows (splitkv_dma.hip)
bool splitkv_dma_eligible(const SplitArgs& a);
// the launch runs the LDS-streamed kernel (eligible, and not taken by the 32-row fp8 one)
bool splitkv_uses_dma(const SplitArgs& a);
// the new-token write can ride in the partial kernel (the launch runs the DMA kernel, one
// query per sequence, 16-byte aligned sources): otherwise the caller launches the cache
// write first
bool splitkv_append_fusable(const SplitArgs& a);
void launch_splitkv_dma(const SplitArgs& a, hipStream_t s);
// bf16 MLA rows with 2 or more query tokens (rows > 16): one wave per token over a
// shared LDS ring (splitkv_tokens.hip)
bool splitkv_tokens_eligible(const SplitArgs& a);
void launch_splitkv_tokens(const SplitArgs& a, hipStream_t s);

struct MergeArgs {
  const float* part_out; const float* part_lse;
  int32_t rows, num_q_heads, dv, num_partitions;
  uint16_t* out; float* out_lse;
  const float* sinks;       // [num_q_heads] extra denominator logits, or null
  // rows that are sequences (decode): row r reads only the first
  // active_splits(pol, seq_lens[r], P) partials (the rest are empty); null: all P
  const int32_t* seq_lens;
  SplitPolicy pol;
};
bool launch_merge(const MergeArgs& a, hipStream_t s);

struct PrefillArgs {
  const uint16_t* q; int64_t q_st, q_sh;
  const int32_t* qsl; int32_t num_seqs, num_tokens, max_q, num_q_heads;
  CacheView c;
  const int32_t* bt; int32_t bt_stride;
  const int32_t* seq_lens;
  float scale;
  uint16_t* out; float* out_lse;
  const float* sinks;       // [num_q_heads] extra denominator logits, or null
};
bool prefill_supported(const PrefillArgs& a);
bool launch_prefill(const PrefillArgs& a, hipStream_t s);

}  // namespace pa
