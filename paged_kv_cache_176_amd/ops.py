"""ctypes binding of the C ABI in ``include/pagedattn.h`` (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpagedattn.so")
_lib = None

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_HIP = 0, 1, 2, 3
_STATUS = {1: "ATTN_E_INVALID", 2: "ATTN_E_UNSUPPORTED", 3: "ATTN_E_HIP"}
KV_BF16, KV_FP8 = 0, 1
SCALE_NONE, SCALE_TENSOR, SCALE_HEAD = 0, 1, 2
EXPORTS = ("attn_cache_write", "attn_splitkv_workspace_bytes", "attn_decode_splitkv", "attn_decode_splitkv_append",
           "attn_decode_splitkv_noalloc", "attn_merge_lse",
           "attn_prefill_causal", "attn_verify", "attn_last_error", "attn_version")


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _CacheDescC(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("row_dim", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("v_offset", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("stride_block", ctypes.c_int64),
        ("stride_slot", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("dtype", ctypes.c_int),
        ("scale_mode", ctypes.c_int),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


def library_path() -> str:
    return _LIB_PATH


def use_library(path: str):
    """Make `path` (a build of the same sources, e.g. the phase-stamped diagnostics library)
    the library every entry point calls; must precede the first call."""
    global _LIB_PATH, _lib
    if _lib is not None:
        raise RuntimeError("use_library: a library is already loaded")
    _LIB_PATH = path
    return load_library()


def load_library(path: Optional[str] = None):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with paged_kv_cache_176_amd/build.py (no fallback exists)")
    lib = ctypes.CDLL(p)
    i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(_CacheDescC)
    lib.attn_cache_write.argtypes = [vp, i64, i64, vp, i64, i64, vp, i32, dp, vp]
    lib.attn_splitkv_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_splitkv_workspace_bytes.restype = sz
    pp = ctypes.POINTER(_SplitPolicyC)
    lib.attn_decode_splitkv.argtypes = [vp, i64, i64, i32, i32, dp, vp, i32, vp, f32, i32, pp, vp, sz, vp, vp, vp, vp]
    lib.attn_decode_splitkv_append.argtypes = [vp, i64, i64, i32, i32, dp, vp, i32, vp, f32, i32, pp,
                                               vp, i64, i64, vp, i64, i64, vp, vp, sz, vp, vp, vp, vp]
    lib.attn_decode_splitkv_noalloc.argtypes = [vp, i64, i64, i32, i32, dp, vp, i32, vp, f32, i32, pp, vp, vp, vp,
                                                vp]
    lib.attn_merge_lse.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.attn_prefill_causal.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, dp, vp, i32, vp, f32, vp, vp, vp, vp]
    lib.attn_verify.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, dp, vp, i32, vp, f32, i32, pp, vp, sz, vp, vp,
                                vp, vp]
    for name in ("attn_cache_write", "attn_decode_splitkv", "attn_decode_splitkv_append",
                 "attn_decode_splitkv_noalloc", "attn_merge_lse",
                 "attn_prefill_causal", "attn_verify"):
        getattr(lib, name).restype = ctypes.c_int
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(st: int):
    if st != ATTN_OK:
        raise AttnError(st, _lib.attn_last_error().decode())


class PreparedCall:
    """One library call whose argument checks and marshalling are done: calling it enqueues
    the same call again (same tensors, same stream) at the cost of one ctypes call.  For loops
    that replay a step on unchanged buffers (their contents may change, their storage may
    not); the tensors it was built from are kept alive.  Its results live in ``out``,
    ``out_lse`` and ``workspace``."""

    __slots__ = ("_fn", "_args", "_keep", "out", "out_lse", "workspace")

    def __init__(self, fn, args, keep, out=None, out_lse=None, workspace=None):
        self._fn, self._args, self._keep = fn, args, keep
        self.out, self.out_lse, self.workspace = out, out_lse, workspace

    def __call__(self):
        st = self._fn(*self._args)
        if st != ATTN_OK:
            raise AttnError(st, _lib.attn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    """The given stream, or the current stream of the tensors' GPU (not of the current device,
    which may be another GPU)."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class CacheDesc:
    """A paged KV cache living in ``storage`` (any dtype; addressed by element strides).

    Element (block, slot, head, col) is at storage_base + block*stride_block +
    slot*stride_slot + head*stride_head + col, in cache elements (2 bytes for
    bf16, 1 byte for fp8).  The checked C descriptor is built on first use and kept
    until a field is assigned again.
    """
    storage: torch.Tensor
    num_blocks: int
    block_size: int
    num_kv_heads: int
    row_dim: int
    head_dim_k: int
    head_dim_v: int
    v_offset: int
    kv_dtype: str = "bf16"
    stride_block: Optional[int] = None
    stride_slot: Optional[int] = None
    stride_head: Optional[int] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    scale_mode: str = "none"

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        object.__setattr__(self, "_c", None)            # any change: check and rebuild on next use

    def __post_init__(self):
        if self.stride_head is None:
            self.stride_head = self.row_dim
        if self.stride_slot is None:
            self.stride_slot = self.num_kv_heads * self.stride_head
        if self.stride_block is None:
            self.stride_block = self.block_size * self.stride_slot

    @classmethod
    def from_geom(cls, storage, geom, k_scale=None, v_scale=None, scale_mode="none"):
        return cls(storage, geom.num_blocks, geom.block_size, geom.num_kv_heads, geom.row_dim, geom.head_dim_k,
                   geom.head_dim_v, geom.v_offset, geom.kv_dtype, geom.stride_block, geom.stride_slot,
                   geom.stride_head, k_scale, v_scale, scale_mode)

    def extent_bytes(self) -> int:
        """Bytes from the storage's first element to the end of the last row the strides address."""
        esize = 1 if self.kv_dtype == "fp8" else 2
        last = ((self.num_blocks - 1) * self.stride_block + (self.block_size - 1) * self.stride_slot +
                (self.num_kv_heads - 1) * self.stride_head + self.row_dim)
        return last * esize

    def c_struct(self) -> _CacheDescC:
        if self._c is None:
            object.__setattr__(self, "_c", self._build())
        return self._c

    def _build(self) -> _CacheDescC:
        mode = {"none": SCALE_NONE, "tensor": SCALE_TENSOR, "head": SCALE_HEAD}[self.scale_mode]
        if self.storage.device.type != "cuda":
            raise TypeError("the cache storage must be on the GPU")
        if self.storage.is_contiguous():              # the storage tensor's own bytes
            avail = self.storage.numel() * self.storage.element_size()
        else:                                         # else the allocation past its first element
            st = self.storage.untyped_storage()
            avail = st.nbytes() - (self.storage.data_ptr() - st.data_ptr())
        if self.extent_bytes() > avail:
            raise ValueError(f"the cache strides address {self.extent_bytes()} bytes but the storage holds {avail}")
        if self.kv_dtype == "fp8":
            n = {"tensor": 1, "head": self.num_kv_heads}.get(self.scale_mode)
            for name, sc in (("k_scale", self.k_scale), ("v_scale", self.v_scale)):
                if n is None or sc is None:
                    raise ValueError("an fp8 cache needs k_scale and v_scale, per tensor or per head")
                _need(sc, torch.float32, name)
                if sc.numel() != n or not sc.is_contiguous():
                    raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} values")
        return _CacheDescC(
            self.storage.data_ptr(), self.num_blocks, self.block_size, self.num_kv_heads, self.row_dim,
            self.head_dim_k, self.head_dim_v, self.v_offset, 0, self.stride_block, self.stride_slot,
            self.stride_head, KV_FP8 if self.kv_dtype == "fp8" else KV_BF16, mode,
            None if self.k_scale is None else self.k_scale.data_ptr(),
            None if self.v_scale is None else self.v_scale.data_ptr())


def _need(t: torch.Tensor, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be on the GPU")


def _need_rows(t: Optional[torch.Tensor], dtype, name, shape):
    """An output or partials buffer: given dtype, on the GPU, contiguous, exactly `shape`."""
    if t is None:
        return
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {list(shape)} tensor, got {list(t.shape)}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _need_query(q: torch.Tensor, cache: "CacheDesc", name="q"):
    """[tokens, Hq, head_dim_k] bf16 with a contiguous last dim (token and head strides are free)."""
    _need(q, torch.bfloat16, name)
    if q.dim() != 3 or q.shape[2] != cache.head_dim_k or q.stride(2) != 1:
        raise ValueError(f"{name} must be [tokens, heads, {cache.head_dim_k}] with a contiguous last dim")


def _need_index(t: torch.Tensor, name, numel=None, dtype=torch.int32):
    _need(t, dtype, name)
    if t.dim() != 1 or not t.is_contiguous() or (numel is not None and t.numel() != numel):
        raise ValueError(f"{name} must be a contiguous 1-D {dtype} tensor" +
                         ("" if numel is None else f" of {numel} entries"))


def _need_table(bt: torch.Tensor, num_seqs: int):
    _need(bt, torch.int32, "block_tables")
    if bt.dim() != 2 or bt.shape[0] < num_seqs or bt.stride(1) != 1:
        raise ValueError(f"block_tables must be [>= {num_seqs}, max_blocks] int32 with contiguous rows")


def _need_kv(key, value, cache: "CacheDesc", tokens: int):
    _need(key, torch.bfloat16, "key")
    if key.dim() != 3 or tuple(key.shape) != (tokens, cache.num_kv_heads, cache.head_dim_k) or key.stride(2) != 1:
        raise ValueError(f"key must be [{tokens}, {cache.num_kv_heads}, {cache.head_dim_k}] bf16 with a contiguous "
                         "last dim")
    if value is not None:
        if cache.v_offset < cache.head_dim_k:
            raise ValueError(f"value columns [{cache.v_offset}, {cache.v_offset + cache.head_dim_v}) overlap the key's "
                             f"[0, {cache.head_dim_k}): pass value=None when V is part of the K row")
        _need(value, torch.bfloat16, "value")
        if (value.dim() != 3 or tuple(value.shape) != (tokens, cache.num_kv_heads, cache.head_dim_v)
                or value.stride(2) != 1):
            raise ValueError(f"value must be [{tokens}, {cache.num_kv_heads}, {cache.head_dim_v}] bf16 with a "
                             "contiguous last dim")


def cache_write(key: torch.Tensor, value: Optional[torch.Tensor], slot_mapping: torch.Tensor, cache: CacheDesc,
                stream=None) -> None:
    """Write key [T, Hkv, Dk] / value [T, Hkv, Dv] (bf16, any token/head strides) into ``cache``."""
    load_library()
    _need_kv(key, value, cache, key.shape[0])
    _need_index(slot_mapping, "slot_mapping", key.shape[0], torch.int64)
    d = cache.c_struct()
    _check(_lib.attn_cache_write(
        _ptr(key), key.stride(0), key.stride(1),
        _ptr(value), value.stride(0) if value is not None else 0, value.stride(1) if value is not None else 0,
        _ptr(slot_mapping), key.shape[0], ctypes.byref(d), _stream(stream, key.device)))


def splitkv_workspace_bytes(rows: int, num_q_heads: int, head_dim_v: int, num_partitions: int) -> int:
    load_library()
    return int(_lib.attn_splitkv_workspace_bytes(rows, num_q_heads, head_dim_v, num_partitions))


def new_workspace(rows: int, num_q_heads: int, head_dim_v: int, num_partitions: int, device="cuda") -> torch.Tensor:
    """A split-KV workspace of the size attn_splitkv_workspace_bytes gives (contents undefined)."""
    return torch.empty(splitkv_workspace_bytes(rows, num_q_heads, head_dim_v, num_partitions), dtype=torch.uint8,
                       device=device)


def workspace_views(ws: torch.Tensor, rows, num_q_heads, head_dim_v, P):
    """(part_out [rows, Hq, P, Dv], part_lse [rows, Hq, P]) fp32 views of a split-KV workspace."""
    n_out = rows * num_q_heads * P * head_dim_v
    part_bytes = (n_out * 4 + 255) // 256 * 256
    f = ws.view(torch.float32)
    po = f[:n_out].view(rows, num_q_heads, P, head_dim_v)
    pl = f[part_bytes // 4: part_bytes // 4 + rows * num_q_heads * P].view(rows, num_q_heads, P)
    return po, pl


MAX_SPLIT_BUCKETS = 8


class _SplitPolicyC(ctypes.Structure):
    _fields_ = [("num_buckets", ctypes.c_int32), ("max_seq_len", ctypes.c_int32 * MAX_SPLIT_BUCKETS),
                ("splits", ctypes.c_int32 * MAX_SPLIT_BUCKETS)]


def _policy(split_policy):
    """[(max_seq_len, splits), ...] ascending (the last bucket also takes longer sequences) -> C table."""
    if split_policy is None:
        return None
    if not 0 < len(split_policy) <= MAX_SPLIT_BUCKETS:
        raise ValueError(f"a split policy has 1..{MAX_SPLIT_BUCKETS} buckets")
    c = _SplitPolicyC()
    c.num_buckets = len(split_policy)
    for i, (bound, k) in enumerate(split_policy):
        c.max_seq_len[i], c.splits[i] = int(bound), int(k)
    return ctypes.byref(c)


def _sinks(sinks: Optional[torch.Tensor], num_q_heads: int):
    """Device fp32 [num_q_heads] sink logits (or None) -> pointer."""
    if sinks is None:
        return None
    _need(sinks, torch.float32, "sinks")
    if sinks.numel() != num_q_heads or not sinks.is_contiguous():
        raise ValueError(f"sinks must be a contiguous [{num_q_heads}] fp32 tensor")
    return _ptr(sinks)


def _need_batch(query_start_loc, seq_lens, block_tables):
    """The per-sequence arrays of a multi-token call (prefill, verify)."""
    _need_index(seq_lens, "seq_lens")
    _need_index(query_start_loc, "query_start_loc", seq_lens.numel() + 1)
    _need_table(block_tables, seq_lens.numel())


def _workspace(rows, hq, dv, P, device, ws):
    """The caller's workspace (checked) or a new one."""
    need = splitkv_workspace_bytes(rows, hq, dv, P)
    if ws is None:
        return new_workspace(rows, hq, dv, P, device)
    if ws.device.type != "cuda" or not ws.is_contiguous() or ws.numel() * ws.element_size() < need:
        raise ValueError(f"the workspace must be a contiguous GPU buffer of >= {need} bytes")
    return ws


def decode_splitkv(q: torch.Tensor, cache: CacheDesc, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                   softmax_scale: float, num_partitions: int, out: Optional[torch.Tensor] = None,
                   out_lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   partials_only: bool = False, with_lse: bool = True, sinks: Optional[torch.Tensor] = None,
                   split_policy=None, stream=None):
    """One query per sequence: q [B, Hq, Dk] bf16 -> (out [B, Hq, Dv] bf16, lse [B, Hq] fp32, workspace).
    sinks: optional [Hq] fp32 logits joining each row's softmax denominator (applied by the merge).
    split_policy: optional [(max_seq_len, splits), ...] context buckets choosing each sequence's active
    partitions on the device (num_partitions is then the launch's maximum)."""
    load_library()
    _need_query(q, cache)
    B, Hq = q.shape[0], q.shape[1]
    _need_table(block_tables, B)
    _need_index(seq_lens, "seq_lens", B)
    _need_rows(out, torch.bfloat16, "out", (B, Hq, cache.head_dim_v))
    _need_rows(out_lse, torch.float32, "out_lse", (B, Hq))
    ws = _workspace(B, Hq, cache.head_dim_v, num_partitions, q.device, workspace)
    if not partials_only and out is None:
        out = torch.empty(B, Hq, cache.head_dim_v, dtype=torch.bfloat16, device=q.device)
    if not partials_only and with_lse and out_lse is None:
        out_lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    d = cache.c_struct()
    _check(_lib.attn_decode_splitkv(
        _ptr(q), q.stride(0), q.stride(1), B, Hq, ctypes.byref(d), _ptr(block_tables), block_tables.stride(0),
        _ptr(seq_lens), float(softmax_scale), num_partitions, _policy(split_policy), _ptr(ws),
        ws.numel() * ws.element_size(),
        None if partials_only else _ptr(out), None if partials_only else _ptr(out_lse), _sinks(sinks, Hq),
        _stream(stream, q.device)))
    return out, out_lse, ws


NOALLOC_WORKSPACE_BYTES = 16 << 20


def decode_splitkv_noalloc(q: torch.Tensor, cache: CacheDesc, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                           softmax_scale: float, num_partitions: int, out: torch.Tensor,
                           out_lse: Optional[torch.Tensor] = None, sinks: Optional[torch.Tensor] = None,
                           split_policy=None, stream=None):
    """decode_splitkv into caller-given outputs with the library's own fixed workspace: the call
    allocates nothing (out [B, Hq, Dv] bf16 is required; out_lse [B, Hq] fp32 optional)."""
    load_library()
    _need_query(q, cache)
    B, Hq = q.shape[0], q.shape[1]
    _need_table(block_tables, B)
    _need_index(seq_lens, "seq_lens", B)
    if out is None:
        raise ValueError("out is required")
    _need_rows(out, torch.bfloat16, "out", (B, Hq, cache.head_dim_v))
    _need_rows(out_lse, torch.float32, "out_lse", (B, Hq))
    d = cache.c_struct()
    _check(_lib.attn_decode_splitkv_noalloc(
        _ptr(q), q.stride(0), q.stride(1), B, Hq, ctypes.byref(d), _ptr(block_tables), block_tables.stride(0),
        _ptr(seq_lens), float(softmax_scale), num_partitions, _policy(split_policy), _ptr(out), _ptr(out_lse),
        _sinks(sinks, Hq), _stream(stream, q.device)))
    return out, out_lse


def decode_splitkv_append(q: torch.Tensor, key: torch.Tensor, value: Optional[torch.Tensor],
                          slot_mapping: torch.Tensor, cache: CacheDesc, block_tables: torch.Tensor,
                          seq_lens: torch.Tensor, softmax_scale: float, num_partitions: int,
                          out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, partials_only: bool = False,
                          with_lse: bool = True, sinks: Optional[torch.Tensor] = None, split_policy=None,
                          stream=None, prepare: bool = False):
    """cache_write(key [B, Hkv, Dk], value [B, Hkv, Dv] or None, slot_mapping [B]) followed by
    decode_splitkv, as one call (the write rides in the decode kernel where it can).
    prepare=True checks and marshals without calling, and returns a PreparedCall."""
    load_library()
    _need_query(q, cache)
    B, Hq = q.shape[0], q.shape[1]
    _need_kv(key, value, cache, B)                  # one new token per sequence
    _need_index(slot_mapping, "slot_mapping", B, torch.int64)
    _need_table(block_tables, B)
    _need_index(seq_lens, "seq_lens", B)
    _need_rows(out, torch.bfloat16, "out", (B, Hq, cache.head_dim_v))
    _need_rows(out_lse, torch.float32, "out_lse", (B, Hq))
    ws = _workspace(B, Hq, cache.head_dim_v, num_partitions, q.device, workspace)
    if not partials_only and out is None:
        out = torch.empty(B, Hq, cache.head_dim_v, dtype=torch.bfloat16, device=q.device)
    if not partials_only and with_lse and out_lse is None:
        out_lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    d = cache.c_struct()
    args = (
        _ptr(q), q.stride(0), q.stride(1), B, Hq, ctypes.byref(d), _ptr(block_tables), block_tables.stride(0),
        _ptr(seq_lens), ctypes.c_float(softmax_scale), num_partitions, _policy(split_policy),
        _ptr(key), key.stride(0), key.stride(1),
        _ptr(value), value.stride(0) if value is not None else 0, value.stride(1) if value is not None else 0,
        _ptr(slot_mapping), _ptr(ws), ws.numel() * ws.element_size(),
        None if partials_only else _ptr(out), None if partials_only else _ptr(out_lse), _sinks(sinks, Hq),
        _stream(stream, q.device))
    if prepare:
        return PreparedCall(_lib.attn_decode_splitkv_append, args,
                            (q, key, value, slot_mapping, block_tables, seq_lens, sinks, d), out, out_lse, ws)
    _check(_lib.attn_decode_splitkv_append(*args))
    return out, out_lse, ws


def merge_lse(part_out: torch.Tensor, part_lse: torch.Tensor, out: Optional[torch.Tensor] = None,
              out_lse: Optional[torch.Tensor] = None, with_lse: bool = True, sinks: Optional[torch.Tensor] = None,
              stream=None):
    """part_out [rows, Hq, P, Dv] fp32, part_lse [rows, Hq, P] fp32 -> (out bf16, lse fp32)."""
    load_library()
    _need(part_out, torch.float32, "part_out")
    _need(part_lse, torch.float32, "part_lse")
    if not (part_out.is_contiguous() and part_lse.is_contiguous()):
        raise ValueError("partials must be contiguous")
    rows, Hq, P, Dv = part_out.shape
    _need_rows(part_lse, torch.float32, "part_lse", (rows, Hq, P))
    _need_rows(out, torch.bfloat16, "out", (rows, Hq, Dv))
    _need_rows(out_lse, torch.float32, "out_lse", (rows, Hq))
    if out is None:
        out = torch.empty(rows, Hq, Dv, dtype=torch.bfloat16, device=part_out.device)
    if with_lse and out_lse is None:
        out_lse = torch.empty(rows, Hq, dtype=torch.float32, device=part_out.device)
    _check(_lib.attn_merge_lse(_ptr(part_out), _ptr(part_lse), rows, Hq, Dv, P, _ptr(out), _ptr(out_lse),
                               _sinks(sinks, Hq), _stream(stream, part_out.device)))
    return out, out_lse


def prefill_causal(q: torch.Tensor, query_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                   block_tables: torch.Tensor, cache: CacheDesc, softmax_scale: float, max_query_len: int,
                   out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                   with_lse: bool = True, sinks: Optional[torch.Tensor] = None, stream=None):
    load_library()
    _need_query(q, cache)
    T, Hq = q.shape[0], q.shape[1]
    _need_batch(query_start_loc, seq_lens, block_tables)
    _need_rows(out, torch.bfloat16, "out", (T, Hq, cache.head_dim_v))
    _need_rows(out_lse, torch.float32, "out_lse", (T, Hq))
    if out is None:
        out = torch.empty(T, Hq, cache.head_dim_v, dtype=torch.bfloat16, device=q.device)
    if with_lse and out_lse is None:
        out_lse = torch.empty(T, Hq, dtype=torch.float32, device=q.device)
    d = cache.c_struct()
    _check(_lib.attn_prefill_causal(
        _ptr(q), q.stride(0), q.stride(1), _ptr(query_start_loc), seq_lens.numel(), T, max_query_len, Hq,
        ctypes.byref(d), _ptr(block_tables), block_tables.stride(0), _ptr(seq_lens), float(softmax_scale),
        _ptr(out), _ptr(out_lse), _sinks(sinks, Hq), _stream(stream, q.device)))
    return out, out_lse


def verify(q: torch.Tensor, query_start_loc: torch.Tensor, seq_lens: torch.Tensor, block_tables: torch.Tensor,
           cache: CacheDesc, softmax_scale: float, max_query_len: int, num_partitions: int,
           out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, partials_only: bool = False, with_lse: bool = True,
           sinks: Optional[torch.Tensor] = None, split_policy=None, stream=None, prepare: bool = False):
    """Multi-token verify (split-KV): q [T, Hq, Dk] -> (out [T, Hq, Dv] bf16, lse [T, Hq], workspace).
    prepare=True checks and marshals without calling, and returns a PreparedCall."""
    load_library()
    _need_query(q, cache)
    T, Hq = q.shape[0], q.shape[1]
    _need_batch(query_start_loc, seq_lens, block_tables)
    _need_rows(out, torch.bfloat16, "out", (T, Hq, cache.head_dim_v))
    _need_rows(out_lse, torch.float32, "out_lse", (T, Hq))
    ws = _workspace(T, Hq, cache.head_dim_v, num_partitions, q.device, workspace)
    if not partials_only and out is None:
        out = torch.empty(T, Hq, cache.head_dim_v, dtype=torch.bfloat16, device=q.device)
    if not partials_only and with_lse and out_lse is None:
        out_lse = torch.empty(T, Hq, dtype=torch.float32, device=q.device)
    d = cache.c_struct()
    args = (
        _ptr(q), q.stride(0), q.stride(1), _ptr(query_start_loc), seq_lens.numel(), T, max_query_len, Hq,
        ctypes.byref(d), _ptr(block_tables), block_tables.stride(0), _ptr(seq_lens), ctypes.c_float(softmax_scale),
        num_partitions, _policy(split_policy), _ptr(ws), ws.numel() * ws.element_size(),
        None if partials_only else _ptr(out), None if partials_only else _ptr(out_lse), _sinks(sinks, Hq),
        _stream(stream, q.device))
    if prepare:
        return PreparedCall(_lib.attn_verify, args, (q, query_start_loc, seq_lens, block_tables, sinks, d), out,
                            out_lse, ws)
    _check(_lib.attn_verify(*args))
    return out, out_lse, ws
