"""Paged-KV cache write, attention and log-sum-exp merge, in fp64 (test infrastructure).

Plain definitions, written for checking by eye against the pages:

* cache write: vLLM PR #64064, sections "Tests" and "Details" -- each new token's
  K goes to the first head_dim columns of its slot's row for every KV head, V to
  its own head_dim_v columns at V's own offset, read with V's own head stride;
  nothing else in the buffer (other slots, slack past the cache) changes.
* paged addressing: key j of sequence b lives at block  block_tables[b, j // BS],
  slot-in-block  j % BS  (the block-size / block-table convention the pages use).
* attention: exact softmax attention per (query, q-head); GQA maps q-head h to
  KV head h // (Hq // Hkv); a query at absolute position p sees keys 0..p.  Rows
  with no visible key output 0 and lse = -inf (diffbot model card, section
  "Update 2026-10-01": padded rows must come out 0, not NaN).
* split-KV partials and their merge: the two-stage decode of vLLM PR #50371
  (review thread: split sweep, runtime split count) and the split-KV reducer of
  the diffbot model card; the merge is the log-sum-exp identity.
* attention sink: a per-query-head logit that joins the softmax denominator as one
  more term (diffbot model card, "Update 2026-10-01: three correctness fixes", third
  item: the vision encoder's sink read as an extra softmax-denominator logit).  It is taken here as one more key whose score is
  the sink and whose value row is zero; lse is the log of the whole denominator.

fp8 caches are dequantised as code value x scale (per tensor or per KV head).
Everything is float64; Q/K/V come in as the exact bf16 / fp8 values.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from . import e4m3fn


def bf16_to_f64(bits) -> np.ndarray:
    return e4m3fn.bf16_bits_to_f32(bits).astype(np.float64)


class CacheSpec:
    """Element offsets inside a flat cache buffer (strides in elements)."""

    def __init__(self, num_blocks, block_size, num_kv_heads, row_dim, head_dim_k, head_dim_v, v_offset,
                 stride_block=None, stride_slot=None, stride_head=None, kv_dtype="bf16"):
        self.num_blocks, self.block_size, self.num_kv_heads = num_blocks, block_size, num_kv_heads
        self.row_dim, self.dk, self.dv, self.v_off = row_dim, head_dim_k, head_dim_v, v_offset
        self.stride_head = row_dim if stride_head is None else stride_head
        self.stride_slot = num_kv_heads * self.stride_head if stride_slot is None else stride_slot
        self.stride_block = block_size * self.stride_slot if stride_block is None else stride_block
        self.kv_dtype = kv_dtype

    @classmethod
    def from_geom(cls, g):
        return cls(g.num_blocks, g.block_size, g.num_kv_heads, g.row_dim, g.head_dim_k, g.head_dim_v,
                   g.v_offset, g.stride_block, g.stride_slot, g.stride_head, g.kv_dtype)

    def row_offset(self, slot: int, head: int) -> int:
        blk, pos = divmod(int(slot), self.block_size)
        return blk * self.stride_block + pos * self.stride_slot + head * self.stride_head


def _scale_for(scale, head):
    if scale is None:
        return np.float32(1.0)
    s = np.asarray(scale, dtype=np.float32).reshape(-1)
    return s[0] if s.size == 1 else s[head]


def cache_write(cache_flat: np.ndarray, spec: CacheSpec, key_bits: np.ndarray,
                value_bits: Optional[np.ndarray], slot_mapping: np.ndarray,
                k_scale=None, v_scale=None) -> np.ndarray:
    """Return a copy of ``cache_flat`` after writing every token with slot >= 0.

    bf16 caches get the bf16 bit patterns unchanged; fp8 caches get
    E4M3FN(fp32(x) / fp32(scale)) with K and V scales separate, each per tensor
    ([1]) or per KV head ([Hkv]).
    """
    out = np.array(cache_flat, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]                           # slot -1: padding token, skipped
    blk, pos = slots[live] // spec.block_size, slots[live] % spec.block_size
    for h in range(spec.num_kv_heads):
        base = blk * spec.stride_block + pos * spec.stride_slot + h * spec.stride_head   # [n]
        k = np.asarray(key_bits)[live, h, : spec.dk]
        if spec.kv_dtype == "fp8":
            k = e4m3fn.quantize(k, _scale_for(k_scale, h))
        out[base[:, None] + np.arange(spec.dk)[None, :]] = k
        if value_bits is not None:
            v = np.asarray(value_bits)[live, h, : spec.dv]
            if spec.kv_dtype == "fp8":
                v = e4m3fn.quantize(v, _scale_for(v_scale, h))
            out[base[:, None] + spec.v_off + np.arange(spec.dv)[None, :]] = v
    return out


def decode_cache(cache_flat: np.ndarray, spec: CacheSpec) -> np.ndarray:
    """Values of raw cache elements as float64 (no scale applied)."""
    if spec.kv_dtype == "fp8":
        return e4m3fn.decode(np.asarray(cache_flat, dtype=np.uint8))
    return bf16_to_f64(np.asarray(cache_flat).view(np.uint16))


def gather_kv(cache_flat: np.ndarray, spec: CacheSpec, block_table_row: np.ndarray, seq_len: int,
              k_scale=None, v_scale=None):
    """Dense K [S, Hkv, Dk] and V [S, Hkv, Dv] of one sequence through its block table.

    ``cache_flat`` holds the raw cache elements (bf16 bit patterns or E4M3FN bytes);
    only the gathered elements are decoded, then multiplied by the K / V scale.
    """
    S, H = int(seq_len), spec.num_kv_heads
    K = np.empty((S, H, spec.dk), dtype=np.float64)
    V = np.empty((S, H, spec.dv), dtype=np.float64)
    if S == 0:
        return K, V
    j = np.arange(S)
    blocks = np.asarray(block_table_row, dtype=np.int64)[j // spec.block_size]
    slot_base = blocks * spec.stride_block + (j % spec.block_size) * spec.stride_slot
    for h in range(H):
        base = slot_base + h * spec.stride_head
        k_raw = cache_flat[base[:, None] + np.arange(spec.dk)[None, :]]
        v_raw = cache_flat[base[:, None] + spec.v_off + np.arange(spec.dv)[None, :]]
        K[:, h, :] = decode_cache(k_raw, spec) * float(_scale_for(k_scale, h))
        V[:, h, :] = decode_cache(v_raw, spec) * float(_scale_for(v_scale, h))
    return K, V


def attention_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions: np.ndarray, scale: float,
                   key_range=None, sinks=None):
    """Softmax attention of query rows of ONE sequence.

    q [L, Hq, Dk] float64, K [S, Hkv, Dk], V [S, Hkv, Dv]; query l sits at absolute
    position positions[l] and sees keys j <= positions[l] (restricted to
    ``key_range`` = [lo, hi) when given, for split-KV partials).
    Returns out [L, Hq, Dv] (0 for rows without visible keys) and lse [L, Hq]
    (natural log, -inf for those rows).  sinks [Hq] (or None): each head's sink logit
    is one more score column with a zero value row.
    """
    L, Hq, _ = q.shape
    S, Hkv, Dv = V.shape
    G = Hq // Hkv
    lo, hi = (0, S) if key_range is None else key_range
    out = np.zeros((L, Hq, Dv), dtype=np.float64)
    lse = np.full((L, Hq), -np.inf, dtype=np.float64)
    keys = np.arange(lo, hi)
    for h in range(Hq):
        g = h // G                                             # GQA: consecutive q-heads share a KV head
        s = scale * (q[:, h, :] @ K[lo:hi, g, :].T)            # [L, hi-lo]
        visible = keys[None, :] <= np.asarray(positions)[:, None]
        s = np.where(visible, s, -np.inf)
        if sinks is not None and np.isfinite(sinks[h]):
            # the sink: one more column, always visible, value row zero
            s_all = np.concatenate([s, np.full((L, 1), float(sinks[h]))], axis=1)
            m = s_all.max(axis=1)
            w = np.exp(s_all - m[:, None])
            den = w.sum(axis=1)
            out[:, h, :] = (w[:, :-1] @ V[lo:hi, g, :]) / den[:, None]
            lse[:, h] = m + np.log(den)
            continue
        m = s.max(axis=1, initial=-np.inf)
        has = np.isfinite(m)
        w = np.where(visible & has[:, None], np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
        l = w.sum(axis=1)
        out[has, h, :] = (w[has] @ V[lo:hi, g, :]) / l[has, None]
        lse[has, h] = m[has] + np.log(l[has])
    return out, lse


def paged_attention(q_bits: np.ndarray, query_start_loc, seq_lens, block_tables, cache_flat: np.ndarray,
                    spec: CacheSpec, scale: float, k_scale=None, v_scale=None, rows: Optional[Sequence[int]] = None,
                    sinks=None):
    """Attention of every query token (or of the token ids in ``rows``) over the paged cache.

    Query i of sequence b (i < L_b = qsl[b+1] - qsl[b]) sits at position S_b - L_b + i:
    seq_lens count the step's new tokens, which are in the cache before attention.
    Returns (out [T or len(rows), Hq, Dv], lse [.., Hq]).
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q = bf16_to_f64(np.asarray(q_bits).view(np.uint16))
    T, Hq = q.shape[0], q.shape[1]
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(want), Hq, spec.dv), dtype=np.float64)
    lse = np.full((len(want), Hq), -np.inf, dtype=np.float64)
    for b in range(len(seq_lens)):
        t0, t1 = int(qsl[b]), int(qsl[b + 1])
        sel = np.nonzero((want >= t0) & (want < t1))[0]
        if sel.size == 0:
            continue
        S, L = int(seq_lens[b]), t1 - t0
        K, V = gather_kv(cache_flat, spec, block_tables[b], S, k_scale, v_scale)
        pos = S - L + (want[sel] - t0)
        o, l = attention_rows(q[want[sel]], K, V, pos, scale, sinks=sinks)
        out[sel], lse[sel] = o, l
    return out, lse


# Split-KV partitions are cut in whole 16-key tiles: the library's documented rule (each
# of P ranges holds ceil(S / P) keys rounded up to 16), whatever the cache block size.
PARTITION_TILE = 16


def partition_ranges(seq_len: int, num_partitions: int, tile: int = PARTITION_TILE):
    """Key ranges of split-KV partitions (vLLM PR #50371, review thread: a runtime split count
    over a sequence's keys): partition p covers [p*C, min((p+1)*C, S)) with C = ceil(S / P)
    rounded up to a multiple of ``tile``; trailing partitions may be empty."""
    if seq_len == 0:
        return [(0, 0)] * num_partitions
    chunk = math.ceil(math.ceil(seq_len / num_partitions) / tile) * tile
    return [(min(p * chunk, seq_len), min((p + 1) * chunk, seq_len)) for p in range(num_partitions)]


def active_splits(seq_len: int, num_partitions: int, policy=None) -> int:
    """A sequence's active split count under a context-bucket policy (vLLM PR #50371, review
    thread: the split count chosen per runtime sequence length by context buckets, one table
    for both stages): policy = [(max_seq_len, splits), ...] ascending; the first bucket whose
    bound holds seq_len decides (the last one for longer sequences), capped at num_partitions."""
    if not policy:
        return num_partitions
    k = policy[-1][1]
    for bound, splits in policy:
        if seq_len <= bound:
            k = splits
            break
    return max(1, min(k, num_partitions))


def paged_attention_partials(q_bits, query_start_loc, seq_lens, block_tables, cache_flat, spec, scale,
                             num_partitions, k_scale=None, v_scale=None, policy=None):
    """Per-partition normalised outputs [T, Hq, P, Dv] and lse [T, Hq, P] (empty -> 0, -inf).
    With a policy, a sequence splits its keys over its first active_splits(...) partitions
    only; the rest stay empty."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    q = bf16_to_f64(np.asarray(q_bits).view(np.uint16))
    T, Hq = q.shape[0], q.shape[1]
    P = num_partitions
    po = np.zeros((T, Hq, P, spec.dv), dtype=np.float64)
    pl = np.full((T, Hq, P), -np.inf, dtype=np.float64)
    for b in range(len(seq_lens)):
        t0, t1 = int(qsl[b]), int(qsl[b + 1])
        S, L = int(seq_lens[b]), t1 - t0
        K, V = gather_kv(cache_flat, spec, block_tables[b], S, k_scale, v_scale)
        pos = S - L + np.arange(L)
        for p, rng in enumerate(partition_ranges(S, active_splits(S, P, policy))):
            if rng[1] <= rng[0]:
                continue
            o, l = attention_rows(q[t0:t1], K, V, pos, scale, key_range=rng)
            po[t0:t1, :, p, :], pl[t0:t1, :, p] = o, l
    return po, pl


def merge_lse(part_out: np.ndarray, part_lse: np.ndarray, sinks=None):
    """Combine split-KV partials: out = sum_p w_p o_p / sum_p w_p, w_p = exp(lse_p - max lse).

    A row whose partials are all empty (max lse = -inf) gives out = 0, lse = -inf, never NaN.
    sinks [Hq] (or None; part_lse is [rows, Hq, P]): each head's sink joins as one more
    partial whose lse is the sink and whose output is zero.
    """
    po = np.asarray(part_out, dtype=np.float64)
    pl = np.asarray(part_lse, dtype=np.float64)
    if sinks is not None:
        sk = np.broadcast_to(np.asarray(sinks, dtype=np.float64)[None, :, None], pl.shape[:-1] + (1,))
        pl = np.concatenate([pl, sk], axis=-1)
        po = np.concatenate([po, np.zeros(po.shape[:-2] + (1,) + po.shape[-1:])], axis=-2)
    M = pl.max(axis=-1)
    has = np.isfinite(M)
    Msafe = np.where(has, M, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - Msafe[..., None]), 0.0)
    den = w.sum(axis=-1)
    out = np.zeros(po.shape[:-2] + po.shape[-1:], dtype=np.float64)
    num = (w[..., None] * po).sum(axis=-2)
    out[has] = num[has] / den[has][..., None]
    lse = np.where(has, Msafe + np.log(np.where(has, den, 1.0)), -np.inf)
    return out, lse
