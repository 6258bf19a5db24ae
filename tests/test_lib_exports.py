"""The C-ABI library loads, exports every entry point the header declares, and
rejects bad host-side arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_cache_176_amd as pk
from paged_kv_cache_176_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pk.library_path()):
        pytest.fail("libpagedattn.so is not built (run __graft_entry__.build())")
    return pk.load_library()


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("attn_cache_write", "attn_decode_splitkv", "attn_merge_lse", "attn_prefill_causal", "attn_verify"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pk.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(ops.EXPORTS) == set(declared_functions())


def test_phase_stamped_twin_exports_the_same_calls_plus_the_stamp_reader():
    """The diagnostics library (decode, fp8-verify and MLA-verify kernels with phase stamps) is a
    drop-in twin: every declared call, plus the stamp readers, which the product library does not carry."""
    from paged_kv_cache_176_amd import build as pkb
    assert os.path.exists(pkb.STAMPS_LIB), "libpagedattn_stamps.so is not built"
    nm = lambda p: set(re.findall(r"\sT\s(\w+)$", subprocess.run(["nm", "-D", "--defined-only", p],
                                                                  capture_output=True, text=True).stdout, flags=re.M))
    twin, product = nm(pkb.STAMPS_LIB), nm(pk.library_path())
    assert set(declared_functions()) <= twin
    readers = {"attn_phase_stamps_read", "attn_phase_stamps_read_wide", "attn_phase_stamps_read_tokens"}
    assert readers <= twin and not readers & product
    assert {n for n in product if n.startswith("attn_")} == {n for n in twin if n.startswith("attn_")} - readers


def test_mfma_probe_library_is_separate_and_lists_its_configurations():
    """The matrix-core issue probe (bench.py --mfma-probe) lives in its own library: it exports
    only its three calls, none of the attention entry points, and names its configurations
    without a GPU."""
    from paged_kv_cache_176_amd import build as pkb
    assert os.path.exists(pkb.PROBE_LIB), "libmfma_probe.so is not built"
    out = subprocess.run(["nm", "-D", "--defined-only", pkb.PROBE_LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert {"mfma_probe_count", "mfma_probe_label", "mfma_probe_run"} <= exported
    assert not {n for n in exported if n.startswith("attn_")}
    probe = ctypes.CDLL(pkb.PROBE_LIB)
    probe.mfma_probe_label.restype = ctypes.c_char_p
    n = probe.mfma_probe_count()
    labels = [probe.mfma_probe_label(i) for i in range(n)]
    assert n >= 10 and all(labels) and len(set(labels)) == n
    assert probe.mfma_probe_label(n) is None and probe.mfma_probe_label(-1) is None
    res = (ctypes.c_double * 3)()
    assert probe.mfma_probe_run(n, res) == -1          # a bad index is rejected before the GPU


def test_struct_layout_matches_header(lib):
    # data(8) + 8 x int32(32) + 3 x int64(24) + 2 x enum(8) + 2 pointers(16)
    assert ctypes.sizeof(ops._CacheDescC) == 88
    assert ops._CacheDescC.stride_block.offset == 40
    assert ops._CacheDescC.k_scale.offset == 72


def _desc(**kw):
    base = dict(data=0x1000, num_blocks=4, block_size=16, num_kv_heads=4, row_dim=320, head_dim_k=192,
                head_dim_v=128, v_offset=192, reserved0=0, stride_block=16 * 4 * 320, stride_slot=4 * 320,
                stride_head=320, dtype=0, scale_mode=0, k_scale=None, v_scale=None)
    base.update(kw)
    return ops._CacheDescC(**base)


@pytest.mark.parametrize("bad,msg", [
    (dict(data=None), "data is NULL"),
    (dict(num_blocks=0), "must be positive"),
    (dict(v_offset=200), "does not fit"),
    (dict(head_dim_k=400), "does not fit"),
    (dict(stride_head=100), "strides"),
    (dict(dtype=1, scale_mode=0), "fp8 caches need"),
    (dict(dtype=7), "unknown cache dtype"),
])
def test_cache_write_rejects_bad_descriptors(lib, bad, msg):
    d = _desc(**bad)
    st = lib.attn_cache_write(ctypes.c_void_p(0x2000), 768, 192, None, 0, 0, ctypes.c_void_p(0x3000), 3,
                              ctypes.byref(d), None)
    assert st == ops.ATTN_E_INVALID
    assert msg in lib.attn_last_error().decode()


@pytest.mark.parametrize("v_offset,dv", [(0, 512), (64, 128), (191, 8)])
def test_value_overlapping_key_is_invalid(lib, v_offset, dv):
    """A value whose columns share bytes with K's (the MLA row, V = K's first columns) would make
    two threads store one element in no fixed order: rejected, also on the fused decode path."""
    d = _desc(num_kv_heads=1, row_dim=576, head_dim_k=576 if v_offset == 0 else 192, head_dim_v=dv,
              v_offset=v_offset, stride_block=16 * 576, stride_slot=576, stride_head=576)
    st = lib.attn_cache_write(ctypes.c_void_p(0x2000), 576, 576, ctypes.c_void_p(0x4000), dv, dv,
                              ctypes.c_void_p(0x3000), 3, ctypes.byref(d), None)
    assert st == ops.ATTN_E_INVALID and "overlap K columns" in lib.attn_last_error().decode()
    # the same row without a value is accepted up to the launch (no GPU here: checked via a 0-token call)
    assert lib.attn_cache_write(None, 0, 0, None, 0, 0, None, 0, ctypes.byref(d), None) == ops.ATTN_OK
    ws = ctypes.c_void_p(0x10000)
    st = lib.attn_decode_splitkv_append(ctypes.c_void_p(0x2000), 576, 576, 1, 12, ctypes.byref(d),
                                        ctypes.c_void_p(0x5000), 4, ctypes.c_void_p(0x6000), ctypes.c_float(0.04),
                                        4, None, ctypes.c_void_p(0x2000), 576, 576, ctypes.c_void_p(0x4000), dv, dv,
                                        ctypes.c_void_p(0x3000), ws, 1 << 30, None, None, None, None)
    assert st == ops.ATTN_E_INVALID and "overlap K columns" in lib.attn_last_error().decode()


def test_value_after_key_is_accepted_by_the_column_check(lib):
    """V starting exactly where K ends (the DiffKV row) passes the overlap check: the call gets as
    far as the 0-token no-op."""
    d = _desc()
    assert lib.attn_cache_write(None, 0, 0, ctypes.c_void_p(0x4000), 0, 0, None, 0, ctypes.byref(d), None) == ops.ATTN_OK


def test_zero_tokens_is_a_noop_and_null_desc_is_invalid(lib):
    d = _desc()
    assert lib.attn_cache_write(None, 0, 0, None, 0, 0, None, 0, ctypes.byref(d), None) == ops.ATTN_OK
    assert lib.attn_cache_write(None, 0, 0, None, 0, 0, None, 1, None, None) == ops.ATTN_E_INVALID


def test_splitkv_argument_checks(lib):
    d = _desc()
    ws_need = lib.attn_splitkv_workspace_bytes(2, 8, 128, 4)
    assert ws_need >= 2 * 8 * 4 * 129 * 4
    assert lib.attn_splitkv_workspace_bytes(-1, 8, 128, 4) == 0
    args = lambda P, ws_bytes, hq=8, pol=None: (ctypes.c_void_p(0x10000), 8 * 192, 192, 2, hq, ctypes.byref(d),
                                                ctypes.c_void_p(0x20000), 8, ctypes.c_void_p(0x30000), 0.07, P, pol,
                                                ctypes.c_void_p(0x40000), ws_bytes, ctypes.c_void_p(0x50000), None, None,
                                      None)
    assert lib.attn_decode_splitkv(*args(0, ws_need)) == ops.ATTN_E_INVALID
    assert lib.attn_decode_splitkv(*args(5000, ws_need)) == ops.ATTN_E_INVALID
    assert lib.attn_decode_splitkv(*args(4, ws_need - 1)) == ops.ATTN_E_INVALID
    assert "workspace" in lib.attn_last_error().decode()
    assert lib.attn_decode_splitkv(*args(4, ws_need, hq=6)) == ops.ATTN_E_INVALID   # 6 % 4 != 0
    # a head-dim pair without a kernel is UNSUPPORTED, not INVALID
    d2 = _desc(head_dim_k=64, head_dim_v=64, v_offset=64, row_dim=128, stride_head=128,
               stride_slot=512, stride_block=16 * 512)
    a = list(args(4, ws_need))
    a[5] = ctypes.byref(d2)
    assert lib.attn_decode_splitkv(*a) == ops.ATTN_E_UNSUPPORTED
    # split policies: bucket count, ascending bounds and splits >= 1 are checked on the host
    bad = ops._SplitPolicyC()
    bad.num_buckets = 9
    assert lib.attn_decode_splitkv(*args(4, ws_need, pol=ctypes.byref(bad))) == ops.ATTN_E_INVALID
    bad.num_buckets = 2
    bad.max_seq_len[0], bad.max_seq_len[1], bad.splits[0], bad.splits[1] = 4096, 4096, 8, 16
    assert lib.attn_decode_splitkv(*args(4, ws_need, pol=ctypes.byref(bad))) == ops.ATTN_E_INVALID
    assert "ascending" in lib.attn_last_error().decode()
    bad.max_seq_len[1], bad.splits[1] = 65536, 0
    assert lib.attn_decode_splitkv(*args(4, ws_need, pol=ctypes.byref(bad))) == ops.ATTN_E_INVALID


def test_append_decode_argument_checks(lib):
    """The write-then-decode call validates its own arguments and the decode's before
    enqueueing anything (a failing call launches no cache write)."""
    d = _desc()
    ws_need = lib.attn_splitkv_workspace_bytes(2, 8, 128, 4)
    key, slots = ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000)
    args = lambda key, slots, P=4, ks=768: (ctypes.c_void_p(0x10000), 8 * 192, 192, 2, 8, ctypes.byref(d),
                                            ctypes.c_void_p(0x20000), 8, ctypes.c_void_p(0x30000), 0.07, P, None,
                                            key, ks, 192, ctypes.c_void_p(0x80000), 512, 128, slots,
                                            ctypes.c_void_p(0x40000), ws_need, ctypes.c_void_p(0x50000), None, None,
                                            None)
    assert lib.attn_decode_splitkv_append(*args(None, slots)) == ops.ATTN_E_INVALID
    assert "NULL key or slot_mapping" in lib.attn_last_error().decode()
    assert lib.attn_decode_splitkv_append(*args(key, None)) == ops.ATTN_E_INVALID
    assert lib.attn_decode_splitkv_append(*args(key, slots, ks=-1)) == ops.ATTN_E_INVALID
    assert lib.attn_decode_splitkv_append(*args(key, slots, P=0)) == ops.ATTN_E_INVALID
    assert "num_partitions" in lib.attn_last_error().decode()


def test_merge_and_prefill_argument_checks(lib):
    assert lib.attn_merge_lse(None, None, 1, 8, 128, 4, None, None, None, None) == ops.ATTN_E_INVALID
    assert lib.attn_merge_lse(None, None, 0, 8, 128, 4, None, None, None, None) == ops.ATTN_OK
    assert lib.attn_merge_lse(ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), 1, 8, 128, 5000,
                              ctypes.c_void_p(1 << 22), None, None, None) == ops.ATTN_E_UNSUPPORTED
    d = _desc()
    st = lib.attn_prefill_causal(None, 0, 0, None, 1, 4, 4, 8, ctypes.byref(d), None, 1, None, 0.1, None, None, None,
                                 None)
    assert st == ops.ATTN_E_INVALID
    st = lib.attn_prefill_causal(ctypes.c_void_p(0x1000), 8 * 192, 192, ctypes.c_void_p(0x2000), 1, 4, 4, 8,
                                 ctypes.byref(d), ctypes.c_void_p(0x3000), 1, ctypes.c_void_p(0x4000),
                                 float("nan"), ctypes.c_void_p(0x5000), None, None, None)
    assert st == ops.ATTN_E_INVALID and "not finite" in lib.attn_last_error().decode()


def test_version_string(lib):
    assert lib.attn_version().decode().startswith("pagedattn")


@pytest.mark.parametrize("bad", [
    dict(stride_slot=640),                              # NHD slots of 2 heads: slot 1 head 0 == slot 0 head 2
    dict(stride_head=320, stride_slot=320),             # slot and head dims alias
    dict(stride_block=15 * 4 * 320),                    # a block one slot too short
    dict(stride_head=16 * 320, stride_slot=300),        # HND order with a row pitch below row_dim
])
def test_overlapping_strides_are_invalid(lib, bad):
    d = _desc(**bad)
    st = lib.attn_cache_write(ctypes.c_void_p(0x2000), 768, 192, None, 0, 0, ctypes.c_void_p(0x3000), 3,
                              ctypes.byref(d), None)
    assert st == ops.ATTN_E_INVALID
    assert "overlapping cache strides" in lib.attn_last_error().decode()


def test_alignment_and_size_checks(lib):
    big = 1 << 20
    # merge: part_out read as float4, out written 4 bf16 at a time
    assert lib.attn_merge_lse(ctypes.c_void_p(big + 4), ctypes.c_void_p(2 * big), 1, 8, 128, 4,
                              ctypes.c_void_p(3 * big), None, None, None) == ops.ATTN_E_UNSUPPORTED
    assert "part_out" in lib.attn_last_error().decode()
    assert lib.attn_merge_lse(ctypes.c_void_p(big), ctypes.c_void_p(2 * big), 1, 8, 128, 4,
                              ctypes.c_void_p(3 * big + 2), None, None, None) == ops.ATTN_E_UNSUPPORTED
    assert "out must be 8-byte aligned" in lib.attn_last_error().decode()
    # verify: tokens with max_query_len 0, and a misaligned output
    d = _desc()
    ws_need = lib.attn_splitkv_workspace_bytes(4, 8, 128, 4)
    vargs = lambda max_q, out: (ctypes.c_void_p(big), 8 * 192, 192, ctypes.c_void_p(2 * big), 2, 4, max_q, 8,
                                ctypes.byref(d), ctypes.c_void_p(3 * big), 8, ctypes.c_void_p(4 * big), 0.07, 4, None,
                                ctypes.c_void_p(5 * big), ws_need, out, None, None, None)
    assert lib.attn_verify(*vargs(0, ctypes.c_void_p(6 * big))) == ops.ATTN_E_INVALID
    assert "max_query_len 0" in lib.attn_last_error().decode()
    assert lib.attn_verify(*vargs(2, ctypes.c_void_p(6 * big + 6))) == ops.ATTN_E_UNSUPPORTED
    # a workspace size past 62 bits is reported as 0 (invalid), not wrapped
    assert lib.attn_splitkv_workspace_bytes(2 ** 31 - 1, 2 ** 31 - 1, 2 ** 20, 4096) == 0


def test_noalloc_rejects_sizes_over_its_workspace_before_the_gpu(lib):
    """attn_decode_splitkv_noalloc checks the partials' size against its fixed 16 MiB workspace
    before any HIP call (this machine has no GPU): B1 x 32 heads x 1024 partitions x 129 floats
    = 16.9 MB is refused; a NULL output is refused too."""
    d = _desc()
    args = lambda B, P, out: (ctypes.c_void_p(0x2000), 32 * 192, 192, B, 32, ctypes.byref(d), ctypes.c_void_p(0x5000),
                              64, ctypes.c_void_p(0x6000), ctypes.c_float(0.07), P, None, out, None, None, None)
    st = lib.attn_decode_splitkv_noalloc(*args(1, 1024, ctypes.c_void_p(0x7000)))
    assert st == ops.ATTN_E_INVALID and "over the fixed workspace" in lib.attn_last_error().decode()
    assert lib.attn_splitkv_workspace_bytes(1, 32, 128, 1024) > ops.NOALLOC_WORKSPACE_BYTES
    assert lib.attn_splitkv_workspace_bytes(1, 32, 128, 1000) <= ops.NOALLOC_WORKSPACE_BYTES
    st = lib.attn_decode_splitkv_noalloc(*args(1, 64, None))
    assert st == ops.ATTN_E_INVALID and "out is required" in lib.attn_last_error().decode()
    assert lib.attn_decode_splitkv_noalloc(*args(0, 64, None)) == ops.ATTN_OK      # nothing to do
