"""Seeded synthetic inputs for the paged-KV attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, no quantisation, no addressing of the cache
other than choosing which block ids a sequence owns).  Both the fp64 CPU oracle
and the HIP library consume what it returns, so they see identical bits.

All tensors are produced on the CPU with ``torch.Generator().manual_seed(seed)``
and a fixed draw order: Q, K, V, scales, block permutation.  Floating inputs are
drawn in fp32 and cast to bf16 (round-to-nearest-even, done by torch).

Workload shapes follow the pages:
  * MiMo-V2.6 asymmetric K/V rows (K 192 / V 128 packed per KV head, 4 KV heads,
    block sizes 16 and 64): vLLM PR #64064, sections "Overview", "Tests" and
    "Details".
  * 12 query heads over one 576-wide latent head whose output is 512 wide, 100K
    context: vLLM PR #50371, sections "Purpose" and "Test Plan".
  * fp8 E4M3 KV cache with per-tensor / per-head scales, 46K-token agent
    contexts, 3 draft tokens + 1 verified (4 query tokens), padded rows with no
    visible keys, 4096-token prefill chunks: the diffbot MiMo-V2.6-Flash model
    card, sections "Benchmarks", "Update 2026-10-01" and "What the kernels do".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F
# Finite poison for slots past a sequence's end inside its last page: large enough
# that an unmasked read changes the result, finite so that weight 0 times it is 0.
BF16_TAIL_POISON = 1024.0
FP8_TAIL_POISON_CODE = 0x7E  # +448, the largest finite E4M3FN value


@dataclass
class CacheGeom:
    """Geometry of one paged KV cache ``[num_blocks, block_size, num_kv_heads, row_dim]``.

    ``v_offset`` is the column where V starts inside a row.  For the packed
    DiffKV row it is ``head_dim_k``; for the shared MLA latent row it is 0 and V
    is the row's first ``head_dim_v`` columns.
    """
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    v_offset: int
    row_dim: int
    kv_dtype: str = "bf16"          # "bf16" or "fp8"
    slack_elems: int = 4096         # guard slack past the cache end
    # "NHD": [block][slot][head][row] (default); "HND": [block][head][slot][row].  row_pad
    # widens the pitch between consecutive rows, block_pad the pitch between blocks
    # (elements; the padding is never read or written).
    layout: str = "NHD"
    row_pad: int = 0
    block_pad: int = 0

    @property
    def elem_bytes(self) -> int:
        return 1 if self.kv_dtype == "fp8" else 2

    @property
    def row_pitch(self) -> int:
        return self.row_dim + self.row_pad

    @property
    def stride_head(self) -> int:
        return self.row_pitch if self.layout == "NHD" else self.block_size * self.row_pitch

    @property
    def stride_slot(self) -> int:
        return self.num_kv_heads * self.row_pitch if self.layout == "NHD" else self.row_pitch

    @property
    def stride_block(self) -> int:
        return self.block_size * self.num_kv_heads * self.row_pitch + self.block_pad

    def rows_view(self, flat: torch.Tensor) -> torch.Tensor:
        """[num_blocks, block_size, num_kv_heads, row_dim] view of a flat cache image."""
        return flat.as_strided((self.num_blocks, self.block_size, self.num_kv_heads, self.row_dim),
                               (self.stride_block, self.stride_slot, self.stride_head, 1))

    @property
    def cache_elems(self) -> int:
        return self.num_blocks * self.stride_block

    @property
    def total_elems(self) -> int:
        return self.cache_elems + self.slack_elems


def diffkv_geom(num_blocks, block_size, kv_dtype="bf16", num_kv_heads=4, slack_elems=4096, layout="NHD",
                row_pad=0, block_pad=0):
    return CacheGeom(num_blocks, block_size, num_kv_heads, 192, 128, 192, 320, kv_dtype, slack_elems, layout, row_pad,
                     block_pad)


def mla_geom(num_blocks, block_size=64, slack_elems=4096, layout="NHD", row_pad=0, block_pad=0):
    return CacheGeom(num_blocks, block_size, 1, 576, 512, 0, 576, "bf16", slack_elems, layout, row_pad, block_pad)


@dataclass
class Workload:
    """One synthetic batch.  All tensors live on the CPU.

    q            [num_tokens, Hq, Dk] bf16
    key          [num_new, Hkv, Dk] bf16   tokens written by the cache write
    value        [num_new, Hkv, Dv] bf16 or None (MLA: V is part of the K row)
    slot_mapping [num_new] int64           slot of each written token, -1 = skip
    cache_init   [total_elems] uint8/int16 cache contents before the write
    block_tables [num_seqs, bt_stride] int32
    seq_lens     [num_seqs] int32 (keys visible to the last query, new tokens included)
    query_start_loc [num_seqs + 1] int32
    """
    name: str
    geom: CacheGeom
    num_q_heads: int
    softmax_scale: float
    q: torch.Tensor
    key: torch.Tensor
    value: Optional[torch.Tensor]
    slot_mapping: torch.Tensor
    cache_init: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    query_start_loc: torch.Tensor
    scale_mode: str = "none"           # "none", "tensor", "head"
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_query_len(self) -> int:
        qsl = self.query_start_loc
        return int((qsl[1:] - qsl[:-1]).max().item()) if qsl.numel() > 1 else 0


def _normal_bf16(gen, shape, std=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)


def _poisoned_cache(geom: CacheGeom, used_blocks, seq_lens_list, tables) -> torch.Tensor:
    """Initial cache image: unused blocks NaN, page tails finite poison, slack NaN.

    Slots that the workload's cache write fills are overwritten later; anything an
    attention kernel should never touch is poisoned so that a touch shows.
    """
    if geom.kv_dtype == "fp8":
        img = torch.full((geom.total_elems,), FP8_NAN_CODE, dtype=torch.uint8)
        poison = FP8_TAIL_POISON_CODE
    else:
        img = torch.full((geom.total_elems,), BF16_NAN_BITS, dtype=torch.int16)
        poison = int(torch.tensor([BF16_TAIL_POISON], dtype=torch.bfloat16).view(torch.int16).item())
    view = geom.rows_view(img)
    # every mapped page starts as finite poison (its padding stays NaN); the write fills
    # the live slots
    if len(used_blocks):
        view[torch.as_tensor(used_blocks, dtype=torch.int64)] = poison
    return img


def _tables(gen, num_blocks_total, blocks_per_seq, bt_stride, spare_block):
    """Random block permutation sliced per sequence; unused entries point at a spare."""
    perm = torch.randperm(num_blocks_total, generator=gen)
    perm = perm[perm != spare_block]
    tables = torch.full((len(blocks_per_seq), bt_stride), spare_block, dtype=torch.int32)
    pos = 0
    for b, nb in enumerate(blocks_per_seq):
        tables[b, :nb] = perm[pos: pos + nb].to(torch.int32)
        pos += nb
    return tables, pos


def _slots_for(tables, seq, positions, block_size):
    pos = torch.as_tensor(positions, dtype=torch.int64)
    blk = tables[seq].to(torch.int64)[pos // block_size]
    return blk * block_size + pos % block_size


def paged_workload(name, geom: CacheGeom, seq_lens, query_lens, num_q_heads, softmax_scale,
                   seed=0, std=1.0, write_all=True, scale_mode="none", scale_range=(0.01, 0.1),
                   num_blocks=None, extra_empty_rows=0, bt_stride=None, q_std=None):
    """General builder.

    Every sequence b has ``seq_lens[b]`` keys; its last ``query_lens[b]`` positions are
    queries.  With ``write_all`` every key of every sequence is a new token written
    by the cache write (the tiny and chunk configs); otherwise only the query
    positions are written and the older context is placed directly in the cache image
    (the long-context configs, whose setup is not what is measured).
    ``extra_empty_rows`` appends sequences with seq_len 0 and one query row each.
    """
    gen = torch.Generator().manual_seed(seed)
    seq_lens = list(seq_lens) + [0] * extra_empty_rows
    query_lens = list(query_lens) + [1] * extra_empty_rows
    bs = geom.block_size
    blocks_per_seq = [math.ceil(s / bs) for s in seq_lens]
    need = sum(blocks_per_seq)
    if num_blocks is None:
        num_blocks = need + 1
    assert num_blocks >= need + 1, "need one spare block for unused table entries"
    geom.num_blocks = num_blocks
    if bt_stride is None:
        bt_stride = max(1, max(blocks_per_seq))
    hq, hkv, dk, dv = num_q_heads, geom.num_kv_heads, geom.head_dim_k, geom.head_dim_v
    num_tokens = sum(query_lens)
    total_keys = sum(seq_lens)
    qstd = std if q_std is None else q_std

    # draw order: Q, K, V, scales, block permutation
    q = _normal_bf16(gen, (num_tokens, hq, dk), qstd)
    k_all = _normal_bf16(gen, (total_keys, hkv, dk), std)
    has_v = geom.v_offset != 0 or dv > dk
    v_all = _normal_bf16(gen, (total_keys, hkv, dv), std) if has_v else None
    k_scale = v_scale = None
    if scale_mode != "none":
        n = 1 if scale_mode == "tensor" else hkv
        lo, hi = scale_range
        k_scale = torch.rand((n,), generator=gen, dtype=torch.float32) * (hi - lo) + lo
        v_scale = torch.rand((n,), generator=gen, dtype=torch.float32) * (hi - lo) + lo
    spare = num_blocks - 1
    tables, _ = _tables(gen, num_blocks, blocks_per_seq, bt_stride, spare)
    used = tables[tables != spare].tolist()
    cache = _poisoned_cache(geom, used, seq_lens, tables)

    # which keys the cache write handles
    qsl = [0]
    for L in query_lens:
        qsl.append(qsl[-1] + L)
    write_idx, slots, pre_idx, pre_slots = [], [], [], []
    off = 0
    for b, (s, L) in enumerate(zip(seq_lens, query_lens)):
        if s:
            sl = _slots_for(tables, b, torch.arange(s), bs)
            idx = torch.arange(off, off + s)
            first_new = 0 if write_all else max(0, s - L)
            write_idx.append(idx[first_new:])
            slots.append(sl[first_new:])
            pre_idx.append(idx[:first_new])
            pre_slots.append(sl[:first_new])
        off += s
    cat = lambda xs: torch.cat(xs) if xs else torch.zeros(0, dtype=torch.int64)
    write_idx, slots, pre_idx, pre_slots = cat(write_idx), cat(slots), cat(pre_idx), cat(pre_slots)
    key = k_all[write_idx]
    value = v_all[write_idx] if v_all is not None else None
    slot_mapping = slots.clone()
    extra = {}
    if pre_idx.numel():
        extra["pre_slots"] = pre_slots
        extra["pre_key"] = k_all[pre_idx]
        extra["pre_value"] = v_all[pre_idx] if v_all is not None else None
    return Workload(name=name, geom=geom, num_q_heads=hq, softmax_scale=softmax_scale, q=q, key=key,
                    value=value, slot_mapping=slot_mapping, cache_init=cache, block_tables=tables,
                    seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                    query_start_loc=torch.tensor(qsl, dtype=torch.int32), scale_mode=scale_mode,
                    k_scale=k_scale, v_scale=v_scale, extra=extra)


def place_bf16_rows(cache_img: torch.Tensor, geom: CacheGeom, slots, key, value):
    """Copy bf16 K/V bits into the cache image at ``slots`` (setup of long contexts).

    This is plain placement of already-drawn bits, used to build a cache image whose
    context predates the measured step; it is not the cache write under test.
    """
    assert geom.kv_dtype == "bf16"
    view = geom.rows_view(cache_img)
    s = torch.as_tensor(slots, dtype=torch.int64)
    blk, pos = s // geom.block_size, s % geom.block_size
    view[blk, pos, :, 0: geom.head_dim_k] = key.view(torch.int16)
    if value is not None:
        view[blk, pos, :, geom.v_offset: geom.v_offset + geom.head_dim_v] = value.view(torch.int16)


# ---------------------------------------------------------------------------------
# The five synthetic configurations (seed 0).
# ---------------------------------------------------------------------------------

def tiny(seed=0):
    """2 seqs (37 and 100 keys), 8 q heads / 4 KV heads, K192/V128, BS16, 16 shuffled blocks."""
    g = diffkv_geom(16, 16)
    return paged_workload("tiny", g, [37, 100], [1, 1], 8, 1.0 / math.sqrt(192), seed=seed,
                          num_blocks=16, write_all=True)


def long_decode(batch, ctx, block_size, seed=0):
    """Decode over a long context: Hq 32 / Hkv 4, K192/V128 bf16; 1 new token per seq."""
    g = diffkv_geom(0, block_size)
    return paged_workload(f"decode_b{batch}_s{ctx}_bs{block_size}", g, [ctx] * batch, [1] * batch, 32,
                          1.0 / math.sqrt(192), seed=seed, write_all=False)


def prefill_chunks(total=32768, chunk=4096, block_size=16, seed=0):
    """One seq of ``total`` new tokens written and attended in ``chunk``-token chunks."""
    g = diffkv_geom(0, block_size)
    w = paged_workload(f"prefill_{total}_c{chunk}", g, [total], [total], 32, 1.0 / math.sqrt(192),
                       seed=seed, write_all=True)
    w.extra["chunk"] = chunk
    return w


def fp8_verify(batch=4, ctx=46080, qlen=4, scale_mode="tensor", empty_rows=4, block_size=16, seed=0):
    """fp8 E4M3FN cache, spec-verify with ``qlen`` query tokens per seq plus empty rows."""
    g = diffkv_geom(0, block_size, kv_dtype="fp8")
    return paged_workload(f"verify_b{batch}_s{ctx}_l{qlen}_{scale_mode}", g, [ctx] * batch, [qlen] * batch, 32,
                          1.0 / math.sqrt(192), seed=seed, write_all=True, scale_mode=scale_mode,
                          extra_empty_rows=empty_rows)


def mla_verify(batch, ctx, qlen=4, num_q_heads=12, seed=0, block_size=64):
    """The MLA decode shape with ``qlen`` query tokens per sequence (drafts + 1), causal
    among themselves; the older context is placed in the cache image."""
    g = mla_geom(0, block_size)
    return paged_workload(f"mla_verify_b{batch}_s{ctx}_l{qlen}_h{num_q_heads}", g, [ctx] * batch, [qlen] * batch,
                          num_q_heads, 1.0 / math.sqrt(576), seed=seed, std=0.1, write_all=False)


def mla_decode(batch, ctx, num_q_heads=12, seed=0, block_size=64):
    """12 q heads on one 576-wide latent head, V = first 512 columns; Q/KV ~ N(0,1)*0.1."""
    g = mla_geom(0, block_size)
    return paged_workload(f"mla_b{batch}_s{ctx}_h{num_q_heads}", g, [ctx] * batch, [1] * batch, num_q_heads,
                          1.0 / math.sqrt(576), seed=seed, std=0.1, write_all=False)
