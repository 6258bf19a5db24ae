// C ABI of the paged-KV attention library: host-side argument checks, dispatch
// to the HIP kernels, status codes and a thread-local error message.  Nothing
// here reads device memory, allocates, or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <utility>

#include "../../include/pagedattn.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

attn_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_E_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

attn_status make_view(const attn_cache_desc* d, pa::CacheView* v, const char* who) {
  if (!d) return fail(ATTN_E_INVALID, "%s: cache descriptor is NULL", who);
  if (!d->data) return fail(ATTN_E_INVALID, "%s: cache data is NULL", who);
  if (d->num_blocks <= 0 || d->block_size <= 0 || d->num_kv_heads <= 0 || d->row_dim <= 0)
    return fail(ATTN_E_INVALID, "%s: cache sizes must be positive (blocks %d, block_size %d, kv_heads %d, row %d)",
                who, d->num_blocks, d->block_size, d->num_kv_heads, d->row_dim);
  if (d->head_dim_k <= 0 || d->head_dim_v <= 0 || d->v_offset < 0)
    return fail(ATTN_E_INVALID, "%s: head dims must be positive and v_offset >= 0", who);
  if (d->head_dim_k > d->row_dim || (int64_t)d->v_offset + d->head_dim_v > d->row_dim)
    return fail(ATTN_E_INVALID, "%s: K [0,%d) or V [%d,%d) does not fit a row of %d", who, d->head_dim_k,
                d->v_offset, d->v_offset + d->head_dim_v, d->row_dim);
  if (d->stride_head <= 0 || d->stride_slot <= 0 || d->stride_block <= 0)
    return fail(ATTN_E_INVALID, "%s: cache strides must be positive", who);
  {
    // No two (block, slot, head) rows may share an element.  Sufficient test: order the
    // slot and head dims (those with more than one index) by stride; each stride must be
    // at least the extent of everything nested inside it, and so must the block stride.
    int64_t st[2], n[2];
    int k = 0;
    if (d->block_size > 1) st[k] = d->stride_slot, n[k++] = d->block_size;
    if (d->num_kv_heads > 1) st[k] = d->stride_head, n[k++] = d->num_kv_heads;
    if (k == 2 && st[0] > st[1]) std::swap(st[0], st[1]), std::swap(n[0], n[1]);
    int64_t ext = d->row_dim;
    for (int i = 0; i < k; ++i) {
      if (st[i] < ext)
        return fail(ATTN_E_INVALID, "%s: overlapping cache strides (block %lld, slot %lld, head %lld, row %d)", who,
                    (long long)d->stride_block, (long long)d->stride_slot, (long long)d->stride_head, d->row_dim);
      ext += (n[i] - 1) * st[i];
    }
    if (d->num_blocks > 1 && d->stride_block < ext)
      return fail(ATTN_E_INVALID, "%s: overlapping cache strides: block stride %lld < one block's extent %lld", who,
                  (long long)d->stride_block, (long long)ext);
  }
  if (d->dtype != ATTN_KV_BF16 && d->dtype != ATTN_KV_FP8_E4M3FN)
    return fail(ATTN_E_INVALID, "%s: unknown cache dtype %d", who, (int)d->dtype);
  if (d->scale_mode < ATTN_SCALE_NONE || d->scale_mode > ATTN_SCALE_PER_HEAD)
    return fail(ATTN_E_INVALID, "%s: unknown scale mode %d", who, (int)d->scale_mode);
  if (d->dtype == ATTN_KV_FP8_E4M3FN) {
    if (d->scale_mode == ATTN_SCALE_NONE || !d->k_scale || !d->v_scale)
      return fail(ATTN_E_INVALID, "%s: fp8 caches need k_scale and v_scale (per tensor or per head)", who);
  }
  v->data = static_cast<uint8_t*>(d->data);
  v->num_blocks = d->num_blocks;
  v->block_size = d->block_size;
  v->num_kv_heads = d->num_kv_heads;
  v->row_dim = d->row_dim;
  v->dk = d->head_dim_k;
  v->dv = d->head_dim_v;
  v->v_off = d->v_offset;
  v->sb = d->stride_block;
  v->ss = d->stride_slot;
  v->sh = d->stride_head;
  v->esize = d->dtype == ATTN_KV_FP8_E4M3FN ? 1 : 2;
  v->scale_mode = d->dtype == ATTN_KV_FP8_E4M3FN ? (int)d->scale_mode : 0;
  v->k_scale = d->k_scale;
  v->v_scale = d->v_scale;
  return ATTN_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// A written value must not share columns with the written key: two threads would store the
// same bytes in no fixed order (the MLA latent row, V = K's first columns, takes value NULL).
attn_status value_columns_ok(const pa::CacheView& c, const void* value, const char* who) {
  if (value && c.v_off < c.dk)   // [v_off, v_off+dv) meets [0, dk): v_off >= 0 and dv > 0
    return fail(ATTN_E_INVALID, "%s: V columns [%d,%d) overlap K columns [0,%d): pass value NULL when V is part of K",
                who, c.v_off, c.v_off + c.dv, c.dk);
  return ATTN_OK;
}

// Layout requirements of the attention kernels (16-byte row loads).
attn_status attention_layout_ok(const pa::CacheView& c, const void* q, int64_t q_st, int64_t q_sh, const char* who) {
  const int eb = c.esize;
  const int64_t vec = 16 / eb;                          // elements per 16 bytes
  if (!aligned(c.data, 16) || c.sb % vec || c.ss % vec || c.sh % vec || c.v_off % vec)
    return fail(ATTN_E_UNSUPPORTED, "%s: cache base/strides/v_offset must be 16-byte aligned", who);
  if (!aligned(q, 16) || q_st % 8 || q_sh % 8)
    return fail(ATTN_E_UNSUPPORTED, "%s: q base and strides must be 16-byte aligned", who);
  return ATTN_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: part_out | part_lse, each starting on a 256-byte boundary; 0 when the size
// does not fit in 62 bits (sizes the library rejects).
size_t splitkv_bytes(int64_t rows, int64_t hq, int64_t dv, int64_t P) {
  const unsigned __int128 n = (unsigned __int128)rows * hq * P;
  if (n * (dv + 1) * sizeof(float) >= ((unsigned __int128)1 << 62)) return 0;
  const size_t part = (size_t)(n * dv) * sizeof(float);
  const size_t lse = (size_t)n * sizeof(float);
  return align256(part) + align256(lse);
}

// Output buffers: bf16 rows are stored 4 elements (8 bytes) at a time, fp32 values singly.
attn_status outputs_aligned(const void* out, const float* out_lse, const float* sinks, const char* who) {
  if (!aligned(out, 8)) return fail(ATTN_E_UNSUPPORTED, "%s: out must be 8-byte aligned", who);
  if (!aligned(out_lse, 4) || !aligned(sinks, 4))
    return fail(ATTN_E_UNSUPPORTED, "%s: out_lse and sinks must be 4-byte aligned", who);
  return ATTN_OK;
}

// The caller's split policy -> the kernels' copy (ok == false: invalid table).
bool make_policy(const attn_split_policy* p, pa::SplitPolicy* out, const char* who, attn_status* st) {
  *out = pa::SplitPolicy{};
  if (!p) return true;
  if (p->num_buckets < 0 || p->num_buckets > ATTN_MAX_SPLIT_BUCKETS) {
    *st = fail(ATTN_E_INVALID, "%s: split policy with %d buckets (0..%d)", who, p->num_buckets, ATTN_MAX_SPLIT_BUCKETS);
    return false;
  }
  out->n = p->num_buckets;
  for (int i = 0; i < p->num_buckets; ++i) {
    if (p->splits[i] < 1 || (i > 0 && p->max_seq_len[i] <= p->max_seq_len[i - 1])) {
      *st = fail(ATTN_E_INVALID, "%s: split policy bucket %d: splits must be >= 1 and bounds strictly ascending",
                 who, i);
      return false;
    }
    out->max_len[i] = p->max_seq_len[i];
    out->splits[i] = p->splits[i];
  }
  return true;
}

// New tokens' K/V to write before a decode (attn_decode_splitkv_append).
struct Append {
  const void* key; int64_t k_st, k_sh;
  const void* value; int64_t v_st, v_sh;
  const int64_t* slots;
};

attn_status run_splitkv(const char* who, const void* q, int64_t q_st, int64_t q_sh, const int32_t* qsl,
                        int32_t num_seqs, int32_t rows, int32_t max_q, int32_t num_q_heads,
                        const attn_cache_desc* cache, const int32_t* bt, int32_t bt_stride, const int32_t* seq_lens,
                        float scale, int32_t P, const attn_split_policy* policy, void* ws, size_t ws_bytes,
                        void* out, float* out_lse, const float* sinks, void* stream, const Append* app = nullptr) {
  pa::CacheView c;
  attn_status st = make_view(cache, &c, who);
  if (st != ATTN_OK) return st;
  if (num_seqs < 0 || rows < 0 || num_q_heads <= 0 || max_q < 0)
    return fail(ATTN_E_INVALID, "%s: negative sizes or num_q_heads <= 0", who);
  if (num_q_heads % c.num_kv_heads)
    return fail(ATTN_E_INVALID, "%s: num_q_heads %d not a multiple of num_kv_heads %d", who, num_q_heads, c.num_kv_heads);
  if (P <= 0 || P > 4096) return fail(ATTN_E_INVALID, "%s: num_partitions %d out of [1, 4096]", who, P);
  if (!std::isfinite(scale)) return fail(ATTN_E_INVALID, "%s: softmax_scale is not finite", who);
  if (rows == 0 || num_seqs == 0) return ATTN_OK;
  if (!q || !bt || !seq_lens || !ws) return fail(ATTN_E_INVALID, "%s: NULL q, block_tables, seq_lens or workspace", who);
  if (app) {
    if (!app->key || !app->slots) return fail(ATTN_E_INVALID, "%s: NULL key or slot_mapping", who);
    if (app->k_st < 0 || app->k_sh < 0 || app->v_st < 0 || app->v_sh < 0)
      return fail(ATTN_E_INVALID, "%s: negative key/value strides", who);
    st = value_columns_ok(c, app->value, who);
    if (st != ATTN_OK) return st;
  }
  if (bt_stride <= 0) return fail(ATTN_E_INVALID, "%s: bt_stride must be positive", who);
  if (qsl && max_q == 0) return fail(ATTN_E_INVALID, "%s: %d query tokens but max_query_len 0", who, rows);
  const size_t need = splitkv_bytes(rows, num_q_heads, c.dv, P);
  if (need == 0) return fail(ATTN_E_INVALID, "%s: workspace size overflows", who);
  if (ws_bytes < need) return fail(ATTN_E_INVALID, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
  if (!aligned(ws, 256)) return fail(ATTN_E_INVALID, "%s: workspace must be 256-byte aligned", who);
  st = attention_layout_ok(c, q, q_st, q_sh, who);
  if (st != ATTN_OK) return st;
  st = outputs_aligned(out, out_lse, sinks, who);
  if (st != ATTN_OK) return st;
  pa::SplitArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_st;
  a.q_sh = q_sh;
  a.qsl = qsl;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_q = max_q;
  a.c = c;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.scale = scale;
  a.num_partitions = P;
  if (!make_policy(policy, &a.pol, who, &st)) return st;
  a.part_out = static_cast<float*>(ws);
  const size_t part_bytes = align256((size_t)rows * num_q_heads * P * c.dv * sizeof(float));
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + part_bytes);
  a.rows = rows;
  a.aslot = nullptr;
  a.ak = nullptr;
  a.av = nullptr;
  a.ak_st = a.ak_sh = a.av_st = a.av_sh = 0;
  if (!pa::splitkv_supported(a))
    return fail(ATTN_E_UNSUPPORTED, "%s: no kernel for head dims %d/%d, v_offset %d, %s cache, %d rows per KV head",
                who, c.dk, c.dv, c.v_off, c.esize == 1 ? "fp8" : "bf16", max_q * (num_q_heads / c.num_kv_heads));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (app) {
    a.aslot = app->slots;
    a.ak = static_cast<const uint16_t*>(app->key);
    a.ak_st = app->k_st;
    a.ak_sh = app->k_sh;
    a.av = static_cast<const uint16_t*>(app->value);
    a.av_st = app->v_st;
    a.av_sh = app->v_sh;
    if (!pa::splitkv_append_fusable(a)) {       // the write as its own kernel, first
      a.aslot = nullptr;
      st = attn_cache_write(app->key, app->k_st, app->k_sh, app->value, app->v_st, app->v_sh, app->slots, num_seqs,
                            cache, stream);
      if (st != ATTN_OK) return st;
    }
  }
  pa::launch_splitkv_partial(a, s);
  st = check_launch(who);
  if (st != ATTN_OK || !out) return st;
  // under a split policy, decode rows (rows are sequences) merge only their active partitions;
  // without one the merge never reads seq_lens
  pa::MergeArgs m{a.part_out, a.part_lse, rows, num_q_heads, c.dv, P, static_cast<uint16_t*>(out), out_lse, sinks,
                  (qsl || a.pol.n == 0) ? nullptr : seq_lens, a.pol};
  pa::launch_merge(m, s);
  return check_launch(who);
}

// Split-KV workspace of attn_decode_splitkv_noalloc: a file-scope device array, so that the
// call allocates nothing.  Each GPU holds its own copy (at its own address) from the first call
// on it until the process ends.  In host code `scratch` is only a stand-in for the symbol: the
// device address comes from hipGetSymbolAddress, taken once per device with that device current,
// and a call uses the copy on the GPU its stream belongs to.
constexpr size_t kScratchBytes = ATTN_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The copy of `scratch` on the GPU that runs `stream` (the current device for the NULL
// stream), or NULL with an error status in *st.  The symbol's address is taken once per
// device, with that device made current for the lookup and the caller's device restored.
void* scratch_for_stream(hipStream_t stream, const char* who, attn_status* st) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess || cur < 0) {
    *st = fail(ATTN_E_HIP, "%s: no current HIP device (%s)", who, hipGetErrorString(e));
    return nullptr;
  }
  int dev = cur;
  if (stream) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess || d < 0) {
      *st = fail(ATTN_E_HIP, "%s: cannot tell the stream's device (%s)", who, hipGetErrorString(e));
      return nullptr;
    }
    dev = d;
  }
  if (dev >= kMaxDevices) {
    *st = fail(ATTN_E_HIP, "%s: device %d is past the %d the library tracks", who, dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) {
      *st = fail(ATTN_E_HIP, "%s: hipSetDevice(%d) failed: %s", who, dev, hipGetErrorString(e));
      return nullptr;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !p) {
      *st = fail(ATTN_E_HIP, "%s: hipGetSymbolAddress of the workspace failed on device %d: %s", who, dev,
                 hipGetErrorString(e));
      return nullptr;
    }
    if (back != hipSuccess) {
      *st = fail(ATTN_E_HIP, "%s: restoring device %d failed: %s", who, cur, hipGetErrorString(back));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err; }

const char* attn_version(void) { return "pagedattn-gfx950 0.1"; }

attn_status attn_cache_write(const void* key, int64_t key_stride_tok, int64_t key_stride_head, const void* value,
                             int64_t val_stride_tok, int64_t val_stride_head, const int64_t* slot_mapping,
                             int32_t num_tokens, const attn_cache_desc* cache, void* stream) {
  const char* who = "attn_cache_write";
  pa::CacheView c;
  attn_status st = make_view(cache, &c, who);
  if (st != ATTN_OK) return st;
  if (num_tokens < 0) return fail(ATTN_E_INVALID, "%s: num_tokens %d < 0", who, num_tokens);
  if (num_tokens == 0) return ATTN_OK;
  if (!key || !slot_mapping) return fail(ATTN_E_INVALID, "%s: NULL key or slot_mapping", who);
  if (key_stride_tok < 0 || key_stride_head < 0 || val_stride_tok < 0 || val_stride_head < 0)
    return fail(ATTN_E_INVALID, "%s: negative source strides", who);
  st = value_columns_ok(c, value, who);
  if (st != ATTN_OK) return st;
  pa::CacheWriteArgs a;
  a.key = static_cast<const uint16_t*>(key);
  a.k_st = key_stride_tok;
  a.k_sh = key_stride_head;
  a.value = static_cast<const uint16_t*>(value);
  a.v_st = val_stride_tok;
  a.v_sh = val_stride_head;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.c = c;
  pa::launch_cache_write(a, static_cast<hipStream_t>(stream));
  return check_launch(who);
}

size_t attn_splitkv_workspace_bytes(int32_t rows, int32_t num_q_heads, int32_t head_dim_v, int32_t num_partitions) {
  if (rows < 0 || num_q_heads <= 0 || head_dim_v <= 0 || num_partitions <= 0) return 0;
  return splitkv_bytes(rows, num_q_heads, head_dim_v, num_partitions);
}

attn_status attn_decode_splitkv(const void* q, int64_t q_stride_tok, int64_t q_stride_head, int32_t num_seqs,
                                int32_t num_q_heads, const attn_cache_desc* cache, const int32_t* block_tables,
                                int32_t bt_stride, const int32_t* seq_lens, float softmax_scale,
                                int32_t num_partitions, const attn_split_policy* policy, void* workspace,
                                size_t workspace_bytes, void* out, float* out_lse, const float* sinks, void* stream) {
  return run_splitkv("attn_decode_splitkv", q, q_stride_tok, q_stride_head, nullptr, num_seqs, num_seqs, 1,
                     num_q_heads, cache, block_tables, bt_stride, seq_lens, softmax_scale, num_partitions, policy,
                     workspace, workspace_bytes, out, out_lse, sinks, stream);
}

attn_status attn_decode_splitkv_noalloc(const void* q, int64_t q_stride_tok, int64_t q_stride_head, int32_t num_seqs,
                                        int32_t num_q_heads, const attn_cache_desc* cache, const int32_t* block_tables,
                                        int32_t bt_stride, const int32_t* seq_lens, float softmax_scale,
                                        int32_t num_partitions, const attn_split_policy* policy, void* out,
                                        float* out_lse, const float* sinks, void* stream) {
  const char* who = "attn_decode_splitkv_noalloc";
  if (!out && num_seqs > 0)
    return fail(ATTN_E_INVALID, "%s: out is required (the partials stay in the library's own buffer)", who);
  if (num_seqs > 0 && num_q_heads > 0 && num_partitions > 0 && cache && cache->head_dim_v > 0) {
    const size_t need = splitkv_bytes(num_seqs, num_q_heads, cache->head_dim_v, num_partitions);
    if (need == 0 || need > kScratchBytes)
      return fail(ATTN_E_INVALID, "%s: %d sequences x %d heads x %d partitions x (%d + 1) floats need %zu bytes, "
                  "over the fixed workspace of %zu bytes", who, num_seqs, num_q_heads, num_partitions,
                  cache->head_dim_v, need, kScratchBytes);
  }
  void* ws = nullptr;
  if (num_seqs > 0) {
    attn_status st = ATTN_OK;
    ws = scratch_for_stream(static_cast<hipStream_t>(stream), who, &st);
    if (!ws) return st;
  }
  return run_splitkv(who, q, q_stride_tok, q_stride_head, nullptr, num_seqs, num_seqs, 1, num_q_heads, cache,
                     block_tables, bt_stride, seq_lens, softmax_scale, num_partitions, policy, ws, kScratchBytes, out,
                     out_lse, sinks, stream);
}

attn_status attn_decode_splitkv_append(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                       int32_t num_seqs, int32_t num_q_heads, const attn_cache_desc* cache,
                                       const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                       float softmax_scale, int32_t num_partitions, const attn_split_policy* policy,
                                       const void* key,
                                       int64_t key_stride_tok, int64_t key_stride_head, const void* value,
                                       int64_t val_stride_tok, int64_t val_stride_head, const int64_t* slot_mapping,
                                       void* workspace, size_t workspace_bytes, void* out, float* out_lse,
                                       const float* sinks, void* stream) {
  const Append app{key, key_stride_tok, key_stride_head, value, val_stride_tok, val_stride_head, slot_mapping};
  return run_splitkv("attn_decode_splitkv_append", q, q_stride_tok, q_stride_head, nullptr, num_seqs, num_seqs, 1,
                     num_q_heads, cache, block_tables, bt_stride, seq_lens, softmax_scale, num_partitions, policy,
                     workspace, workspace_bytes, out, out_lse, sinks, stream, &app);
}

attn_status attn_verify(const void* q, int64_t q_stride_tok, int64_t q_stride_head, const int32_t* query_start_loc,
                        int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
                        const attn_cache_desc* cache, const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* seq_lens, float softmax_scale, int32_t num_partitions,
                        const attn_split_policy* policy, void* workspace, size_t workspace_bytes, void* out,
                        float* out_lse, const float* sinks, void* stream) {
  if (num_seqs > 0 && !query_start_loc) return fail(ATTN_E_INVALID, "attn_verify: NULL query_start_loc");
  return run_splitkv("attn_verify", q, q_stride_tok, q_stride_head, query_start_loc, num_seqs, num_tokens,
                     max_query_len, num_q_heads, cache, block_tables, bt_stride, seq_lens, softmax_scale,
                     num_partitions, policy, workspace, workspace_bytes, out, out_lse, sinks, stream);
}

attn_status attn_merge_lse(const float* part_out, const float* part_lse, int32_t rows, int32_t num_q_heads,
                           int32_t head_dim_v, int32_t num_partitions, void* out, float* out_lse, const float* sinks,
                           void* stream) {
  const char* who = "attn_merge_lse";
  if (rows < 0 || num_q_heads <= 0 || head_dim_v <= 0 || num_partitions <= 0)
    return fail(ATTN_E_INVALID, "%s: bad sizes", who);
  if (rows == 0) return ATTN_OK;
  if (!part_out || !part_lse || !out) return fail(ATTN_E_INVALID, "%s: NULL pointer", who);
  if (num_partitions > 4096)
    return fail(ATTN_E_UNSUPPORTED, "%s: %d partitions exceed the merge kernel's limit of 4096", who, num_partitions);
  if (head_dim_v % 4) return fail(ATTN_E_UNSUPPORTED, "%s: head_dim_v must be a multiple of 4", who);
  if (!aligned(part_out, 16) || !aligned(part_lse, 4))
    return fail(ATTN_E_UNSUPPORTED, "%s: part_out must be 16-byte and part_lse 4-byte aligned", who);
  const attn_status st = outputs_aligned(out, out_lse, sinks, who);
  if (st != ATTN_OK) return st;
  pa::MergeArgs m{part_out, part_lse, rows, num_q_heads, head_dim_v, num_partitions, static_cast<uint16_t*>(out),
                  out_lse, sinks, nullptr, pa::SplitPolicy{}};
  pa::launch_merge(m, static_cast<hipStream_t>(stream));
  return check_launch(who);
}

attn_status attn_prefill_causal(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                int32_t max_query_len, int32_t num_q_heads, const attn_cache_desc* cache,
                                const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                float softmax_scale, void* out, float* out_lse, const float* sinks, void* stream) {
  const char* who = "attn_prefill_causal";
  pa::CacheView c;
  attn_status st = make_view(cache, &c, who);
  if (st != ATTN_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_q_heads <= 0)
    return fail(ATTN_E_INVALID, "%s: negative sizes or num_q_heads <= 0", who);
  if (num_q_heads % c.num_kv_heads)
    return fail(ATTN_E_INVALID, "%s: num_q_heads %d not a multiple of num_kv_heads %d", who, num_q_heads, c.num_kv_heads);
  if (!std::isfinite(softmax_scale)) return fail(ATTN_E_INVALID, "%s: softmax_scale is not finite", who);
  if (num_seqs == 0 || num_tokens == 0) return ATTN_OK;
  if (!q || !query_start_loc || !block_tables || !seq_lens || !out)
    return fail(ATTN_E_INVALID, "%s: NULL pointer argument", who);
  if (bt_stride <= 0) return fail(ATTN_E_INVALID, "%s: bt_stride must be positive", who);
  st = attention_layout_ok(c, q, q_stride_tok, q_stride_head, who);
  if (st != ATTN_OK) return st;
  st = outputs_aligned(out, out_lse, sinks, who);
  if (st != ATTN_OK) return st;
  if (max_query_len == 0) return fail(ATTN_E_INVALID, "%s: %d query tokens but max_query_len 0", who, num_tokens);
  pa::PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.qsl = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_q = max_query_len;
  a.num_q_heads = num_q_heads;
  a.c = c;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.out_lse = out_lse;
  a.sinks = sinks;
  if (!pa::prefill_supported(a))
    return fail(ATTN_E_UNSUPPORTED, "%s: no kernel for head dims %d/%d, v_offset %d, G %d", who, c.dk, c.dv, c.v_off,
                num_q_heads / c.num_kv_heads);
  pa::launch_prefill(a, static_cast<hipStream_t>(stream));
  return check_launch(who);
}

}  // extern "C"
