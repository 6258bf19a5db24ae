/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged-KV attention library.
 *
 * Paged-KV attention with asymmetric K/V head dims, and the cache write that
 * feeds it.  Two row layouts are served by one descriptor:
 *   - the packed DiffKV row: per KV head one row of head_dim_k + head_dim_v
 *     elements, K in the first head_dim_k columns and V in the next head_dim_v
 *     (MiMo-V2.6: 192 + 128, 4 KV heads; vLLM PR #64064 "[...] asymmetric K/V",
 *     sections "Overview", "Tests", "Details");
 *   - the shared MLA latent row: one KV head of 576 elements whose first 512
 *     columns are also V (12 query heads per rank; vLLM PR #50371 "[ROCm] Enable
 *     12-head MLA persistent decode", sections "Purpose", "Test Plan").
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     keeps no pointer after a call returns and never allocates, frees, reads
 *     device memory on the host, or synchronises: every call only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the default stream).  The caller
 *     keeps the buffers alive until that work completes.
 *   - Strides are in ELEMENTS of the tensor they describe.
 *   - Alignment (else ATTN_E_UNSUPPORTED): q and the cache base, strides and
 *     v_offset 16 bytes; bf16 outputs `out` 8 bytes; fp32 arrays (lse, sinks)
 *     4 bytes; split-KV workspaces 256 bytes (ATTN_E_INVALID).
 *   - Status: ATTN_OK, or ATTN_E_INVALID for bad host-side arguments (null
 *     pointers, negative sizes, inconsistent geometry, a workspace that is too
 *     small), ATTN_E_UNSUPPORTED when no kernel exists for a shape or dtype
 *     (the caller falls back, as a backend that cannot serve a head-size pair
 *     does in vLLM PR #64064, "Known limitations"), ATTN_E_HIP when the HIP
 *     runtime reports a launch error.  Nothing aborts or throws across the ABI;
 *     attn_last_error() gives a thread-local message for the last non-OK status.
 *   - Device-resident values are PRECONDITIONS, not checked by the library:
 *     every slot < num_blocks * block_size, every block id < num_blocks, no two
 *     tokens write the same slot, seq_len <= bt_stride * block_size, and the
 *     block-table entries a sequence uses are valid.  Entries past
 *     ceil(seq_len / block_size) are never read.
 *   - Numerics: Q, K, V are bf16 (or fp8 E4M3FN cache bytes); dot products and
 *     softmax in fp32; output bf16 (round to nearest even); LSE natural log, fp32.
 *     Query head h uses KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,
  ATTN_E_UNSUPPORTED = 2,
  ATTN_E_HIP = 3
} attn_status;

/* Cache element type.  FP8 is the OCP E4M3FN byte format (no infinities, 0x7F /
 * 0xFF NaN, max finite 448); the diffbot MiMo-V2.6-Flash model card ("FP8 (E4M3)
 * KV cache") and vLLM PR #64064 ("Tests": bf16 and fp8 caches). */
typedef enum { ATTN_KV_BF16 = 0, ATTN_KV_FP8_E4M3FN = 1 } attn_kv_dtype;

/* fp8 dequantisation scales: one fp32 per tensor ([1]) or one per KV head
 * ([num_kv_heads]), separate for K and V (vLLM PR #64064, "Tests": per-tensor
 * and per-head scales).  Ignored for bf16 caches. */
typedef enum { ATTN_SCALE_NONE = 0, ATTN_SCALE_PER_TENSOR = 1, ATTN_SCALE_PER_HEAD = 2 } attn_scale_mode;

/* Paged KV cache descriptor.
 * Element (block b, slot-in-block s, KV head h, column c) lives at
 *   data + b*stride_block + s*stride_slot + h*stride_head + c        (elements)
 * Key j of a sequence with block table row bt is in block bt[j / block_size],
 * slot j % block_size.  K occupies columns [0, head_dim_k), V occupies
 * [v_offset, v_offset + head_dim_v); both must fit in row_dim.  The default
 * (NHD) strides are stride_head = row_dim, stride_slot = num_kv_heads*row_dim,
 * stride_block = block_size*stride_slot; HND swaps the slot and head strides
 * (stride_slot = row pitch, stride_head = block_size*row pitch).  Strides must
 * be positive and must not let two rows share an element: ordered by stride, the
 * slot and head strides (of dims with more than one index) must each be at
 * least the extent of what nests inside them, starting from row_dim, and
 * stride_block at least one block's extent; else ATTN_E_INVALID.
 * DiffKV: row_dim 320, head_dim_k 192, head_dim_v 128, v_offset 192.
 * MLA:    row_dim 576, head_dim_k 576, head_dim_v 512, v_offset 0.          */
typedef struct {
  void* data;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t row_dim;
  int32_t head_dim_k;
  int32_t head_dim_v;
  int32_t v_offset;
  int32_t reserved0;
  int64_t stride_block;
  int64_t stride_slot;
  int64_t stride_head;
  attn_kv_dtype dtype;
  attn_scale_mode scale_mode;
  const float* k_scale; /* device, [1] or [num_kv_heads]; NULL iff scale_mode NONE */
  const float* v_scale; /* device, [1] or [num_kv_heads]; NULL iff scale_mode NONE */
} attn_cache_desc;

/* Split policy: how many of a launch's num_partitions a sequence actually uses,
 * chosen on the device from its seq_len by context buckets, so that the launch
 * shape stays fixed (graph-stable) while short and long contexts get their own
 * split count, and the partial and merge kernels read the same table (vLLM PR
 * #50371, review thread: active splits derived from device-side sequence lengths
 * in both stages, context buckets -- e.g. 96 for a 100K context -- and the wish
 * for one table shared by the two stages).  Bucket i holds seq_len <=
 * max_seq_len[i] (ascending); a longer sequence takes the last bucket.  A
 * sequence uses min(splits[i], num_partitions) partitions of ceil(seq_len /
 * that) keys (rounded up to the 16-key tile); the others are empty.  The table is
 * read on the host at the call and travels by value with the launch.          */
#define ATTN_MAX_SPLIT_BUCKETS 8
typedef struct {
  int32_t num_buckets;                          /* 0..8; 0: all partitions active  */
  int32_t max_seq_len[ATTN_MAX_SPLIT_BUCKETS];  /* strictly ascending bounds        */
  int32_t splits[ATTN_MAX_SPLIT_BUCKETS];       /* active partitions, >= 1          */
} attn_split_policy;

/* ---------------------------------------------------------------------------
 * attn_cache_write -- write new tokens' K and V into their cache slots.
 * vLLM PR #64064, sections "Claims" and "Details": V is read with ITS OWN head
 * stride and written with ITS OWN width head_dim_v at column v_offset, not with
 * K's; section "Tests": the cache must match one built slot by slot, K in the
 * first head_dim_k columns of a row and V in the remaining head_dim_v, and the
 * bytes past the cache end stay untouched.
 *
 *   key    [num_tokens, num_kv_heads, head_dim_k] bf16; element (t,h,d) at
 *          key + t*key_stride_tok + h*key_stride_head + d.
 *   value  [num_tokens, num_kv_heads, head_dim_v] bf16, own strides; may be
 *          NULL, then only the K columns are written (MLA latent rows, whose V
 *          is the row's first head_dim_v columns).  A value whose columns
 *          [v_offset, v_offset + head_dim_v) overlap K's [0, head_dim_k) is
 *          ATTN_E_INVALID (the two writes would race on the shared bytes).
 *   slot_mapping [num_tokens] int64: slot = block*block_size + slot-in-block;
 *          -1 skips the token (padding).
 *   For ATTN_KV_FP8_E4M3FN the stored byte is E4M3FN(fp32(x) / fp32(scale)):
 *   correctly rounded binary32 division, round to nearest even, saturation to
 *   +-448, NaN -> 0x7F, signed zero kept.  bf16 caches get the bits unchanged.
 *   num_tokens == 0 is a no-op.                                              */
attn_status attn_cache_write(const void* key, int64_t key_stride_tok, int64_t key_stride_head,
                             const void* value, int64_t val_stride_tok, int64_t val_stride_head,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             const attn_cache_desc* cache, void* stream);

/* ---------------------------------------------------------------------------
 * Split-KV workspace.  Partials of `rows` query rows over num_partitions key
 * ranges: part_out [rows, num_q_heads, num_partitions, head_dim_v] fp32 (each
 * normalised by its own softmax sum) at byte 0, then part_lse [rows,
 * num_q_heads, num_partitions] fp32 (-inf for an empty range) at the next
 * 256-byte boundary.  Contents need no initialisation.  Two calls that share a
 * workspace must not run concurrently.  Returns the bytes needed (0 for invalid
 * arguments, or a size that does not fit in 62 bits).                          */
size_t attn_splitkv_workspace_bytes(int32_t rows, int32_t num_q_heads, int32_t head_dim_v,
                                    int32_t num_partitions);

/* ---------------------------------------------------------------------------
 * Sink logits (every attention entry point below takes `sinks`): NULL, or a
 * device array [num_q_heads] fp32 of per-query-head logits that join every row's
 * softmax denominator as one extra term with a zero value row (the attention
 * sink read as an extra softmax-denominator logit: diffbot model card, "Update
 * 2026-10-01: three correctness fixes", the item on the vision encoder's sink).  In the units of softmax_scale*q.k:
 *   out = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink_h}),
 *   lse = ln(sum_j e^{s_j} + e^{sink_h})   (the denominator actually applied).
 * A row with no visible key then outputs 0 and lse = sink_h.  -inf entries (and
 * NULL) give exactly the results without a sink.  With split-KV the partials
 * never include the sink; the merge adds it once.                            */

/* ---------------------------------------------------------------------------
 * attn_decode_splitkv -- one query token per sequence over its paged context.
 * Split-KV (flash-decoding) with a runtime, device-side choice of each
 * partition's key range and a log-sum-exp merge: vLLM PR #50371, review thread
 * (two-stage decode, split count derived from device-side sequence lengths with
 * a graph-stable launch shape; 100K context best near 96 splits); diffbot model
 * card, "What the kernels do" (split-KV needed to fill the GPU at long context).
 * GQA: the num_q_heads/num_kv_heads query heads of a KV head share each K/V read.
 *
 *   q        [num_seqs, num_q_heads, head_dim_k] bf16, element (b,h,d) at
 *            q + b*q_stride_tok + h*q_stride_head + d.  The query of sequence b
 *            is at position seq_lens[b]-1 and sees keys 0..seq_lens[b]-1.
 *   block_tables [num_seqs, bt_stride] int32; seq_lens [num_seqs] int32 >= 0.
 *   softmax_scale  multiplies q.k (fp32), e.g. 1/sqrt(head_dim_k).
 *   num_partitions P >= 1: each sequence's keys are cut into P ranges of
 *            ceil(seq_len/P) keys (rounded up to the kernel's 16-key tile).
 *   policy   NULL, or the split policy above (then P is the launch's maximum).
 *   workspace      >= attn_splitkv_workspace_bytes(num_seqs, num_q_heads,
 *            head_dim_v, P) bytes of device memory, 256-byte aligned.
 *   out      [num_seqs, num_q_heads, head_dim_v] bf16 contiguous.  If out is
 *            NULL only the partials are produced, left in the workspace for
 *            attn_merge_lse (e.g. after partials of other key ranges are added).
 *   out_lse  [num_seqs, num_q_heads] fp32 or NULL.
 *   A sequence with seq_len 0 outputs exact zeros and lse -inf.             */
attn_status attn_decode_splitkv(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                int32_t num_seqs, int32_t num_q_heads,
                                const attn_cache_desc* cache, const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* seq_lens, float softmax_scale, int32_t num_partitions,
                                const attn_split_policy* policy, void* workspace, size_t workspace_bytes,
                                void* out, float* out_lse, const float* sinks, void* stream);

/* ---------------------------------------------------------------------------
 * attn_decode_splitkv_noalloc -- attn_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and the same results
 * bit for bit, with the split-KV partials in a fixed workspace that the library
 * holds in its own device code object (ATTN_NOALLOC_WORKSPACE_BYTES = 16 MiB per
 * GPU, resident from the first call on that GPU until the process ends).  The
 * call allocates and frees nothing; the caller still passes q, the cache, the
 * index arrays and the outputs.
 *   Arguments as attn_decode_splitkv without workspace / workspace_bytes; out is
 *   required (NULL with num_seqs > 0 is ATTN_E_INVALID: the partials cannot be
 *   read back).  A call whose attn_splitkv_workspace_bytes(num_seqs,
 *   num_q_heads, head_dim_v, num_partitions) exceeds the fixed size returns
 *   ATTN_E_INVALID before touching the GPU.
 *   The workspace used is the one on the GPU that `stream` belongs to (the
 *   current device's for the NULL stream).
 *   Every call on one GPU shares that GPU's workspace (it keeps the last call's
 *   partials): calls that overlap on one GPU -- on different streams, or from
 *   different threads -- race and must be ordered by the caller.  Its contents
 *   need no initialisation (every partition writes its own partial).        */
#define ATTN_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)
attn_status attn_decode_splitkv_noalloc(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        const attn_cache_desc* cache, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, float softmax_scale, int32_t num_partitions,
                                        const attn_split_policy* policy, void* out, float* out_lse,
                                        const float* sinks, void* stream);

/* ---------------------------------------------------------------------------
 * attn_decode_splitkv_append -- one decode step with its new token: the result
 * (cache contents, out, out_lse, workspace partials) is that of
 *   attn_cache_write(key, value, slot_mapping, num_tokens = num_seqs)
 * followed by attn_decode_splitkv on the same arguments, i.e. the reshape-and-
 * cache of the step's K/V (vLLM PR #64064, "Details": V with its own head stride
 * and width) and the split-KV decode that reads it (vLLM PR #50371, review
 * thread).  Where the decode kernel can take it (power-of-two block size >= 16,
 * the DiffKV row or the bf16 MLA row, 16-byte aligned sources and strides that are
 * multiples of 8, value given for DiffKV and NULL for MLA) the write happens inside
 * the partial kernel: the workgroup whose key range holds key seq_lens[b]-1 writes
 * row b before reading any key, which saves a launch; otherwise the two kernels
 * run in that order.
 *   key / value / slot_mapping: as attn_cache_write, one token per sequence
 *            (token b belongs to sequence b; value NULL writes K columns only).
 *   Extra precondition: slot_mapping[b] is -1 or the slot of key seq_lens[b]-1 of
 *            sequence b (bt[b][(seq_lens[b]-1)/block_size]*block_size +
 *            (seq_lens[b]-1)%block_size), the decode step's own key.
 *   All other arguments as attn_decode_splitkv.                              */
attn_status attn_decode_splitkv_append(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       const attn_cache_desc* cache, const int32_t* block_tables, int32_t bt_stride,
                                       const int32_t* seq_lens, float softmax_scale, int32_t num_partitions,
                                       const attn_split_policy* policy, const void* key, int64_t key_stride_tok, int64_t key_stride_head,
                                       const void* value, int64_t val_stride_tok, int64_t val_stride_head,
                                       const int64_t* slot_mapping,
                                       void* workspace, size_t workspace_bytes,
                                       void* out, float* out_lse, const float* sinks, void* stream);

/* ---------------------------------------------------------------------------
 * attn_merge_lse -- combine split-KV partials.  Per (row, head): M = max_p lse_p;
 * if M = -inf (no partition saw a key) out = 0 and lse = -inf, never NaN (the
 * empty-row fix of the split-KV reducer: diffbot model card, "Update
 * 2026-10-01"); otherwise w_p = exp(lse_p - M), out = sum w_p o_p / sum w_p,
 * lse = M + ln sum w_p.  With sinks, sink_h joins as one more partial with
 * lse = sink_h and a zero output (see "Sink logits").
 *   part_out [rows, num_q_heads, num_partitions, head_dim_v] fp32 contiguous,
 *            16-byte aligned;
 *   part_lse [rows, num_q_heads, num_partitions] fp32 contiguous;
 *   out [rows, num_q_heads, head_dim_v] bf16 contiguous; out_lse fp32 or NULL.
 *   head_dim_v must be a multiple of 4 and num_partitions <= 4096, else
 *   ATTN_E_UNSUPPORTED.                                                        */
attn_status attn_merge_lse(const float* part_out, const float* part_lse, int32_t rows, int32_t num_q_heads,
                           int32_t head_dim_v, int32_t num_partitions,
                           void* out, float* out_lse, const float* sinks, void* stream);

/* ---------------------------------------------------------------------------
 * attn_prefill_causal -- causal attention of a batch of query chunks over the
 * paged cache (chunked prefill: 4096-token chunks, FA2-style tiles, GQA heads
 * sharing each K/V tile; diffbot model card, "What the kernels do").  The
 * chunk's K/V must already be in the cache (attn_cache_write first).
 *   q [num_tokens, num_q_heads, head_dim_k] bf16 with token/head strides.
 *   query_start_loc [num_seqs+1] int32: tokens of sequence b are
 *            query_start_loc[b] .. query_start_loc[b+1]-1; L_b is their count.
 *   seq_lens [num_seqs] int32: keys of sequence b INCLUDING this chunk; query i
 *            of b sits at position seq_lens[b] - L_b + i and sees keys 0..that.
 *   max_query_len  >= every L_b (sizes the launch); 0 with num_tokens > 0 is
 *            ATTN_E_INVALID.
 *   out [num_tokens, num_q_heads, head_dim_v] bf16 contiguous; out_lse
 *            [num_tokens, num_q_heads] fp32 or NULL.
 *   Rows with no visible key output 0 and lse -inf.                            */
attn_status attn_prefill_causal(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                int32_t max_query_len, int32_t num_q_heads,
                                const attn_cache_desc* cache, const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* seq_lens, float softmax_scale,
                                void* out, float* out_lse, const float* sinks, void* stream);

/* ---------------------------------------------------------------------------
 * attn_verify -- speculative-decode verify: a few query tokens per sequence
 * (e.g. 3 drafts + 1), causal among themselves, over a long paged context, with
 * split-KV kept for query_len > 1 and all query rows of a KV head sharing one
 * K/V read (diffbot model card, "What the kernels do" and "Benchmarks": "one
 * program per whole verify"); fp8 K/V converted to bf16 in the load path, the
 * scales applied after the dot products (Q stays bf16: fp8 QK^T was rejected,
 * "Benchmarks").  Padded rows (seq_len 0) output exact zeros ("Update
 * 2026-10-01").  Arguments as attn_prefill_causal, plus the split-KV
 * num_partitions, policy and workspace as attn_decode_splitkv (rows =
 * num_tokens; the merge of verify rows reads all num_partitions partials, the
 * inactive ones being empty).
 * DiffKV rows: max_query_len * (num_q_heads/num_kv_heads) must be <= 64.  The
 * bf16 MLA latent row: any max_query_len with <= 16 query heads per KV head
 * (vLLM PR #50371, review thread: the verify that the single-token MLA path
 * leaves to another kernel).                                                   */
attn_status attn_verify(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                        const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                        int32_t max_query_len, int32_t num_q_heads,
                        const attn_cache_desc* cache, const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* seq_lens, float softmax_scale, int32_t num_partitions,
                        const attn_split_policy* policy, void* workspace, size_t workspace_bytes,
                        void* out, float* out_lse, const float* sinks, void* stream);

/* Thread-local description of the last non-OK status returned on this thread. */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDATTN_H */
