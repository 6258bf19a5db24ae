"""Caches past 4 GB: the same small workload placed in the top blocks of a cache whose
byte offsets exceed 2^32 (block ids shifted up by 60K-220K blocks) must give bit-identical
outputs, log-sum-exps and written rows as in a compact cache, for every entry point and
kernel family (LDS-streamed, 32-row wide and register-prefetch split-KV, fused write-and-
decode, fast and generic prefill, cache write).  A 288 GB part holds caches far larger than
4 GB, so any 32-bit byte offset in a kernel would show here.  The compact run is itself
checked against the oracle."""
import copy
import math

import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention, split_last_keys

pytestmark = pytest.mark.gpu


class Lifted:
    """The workload's cache, block tables and slots with every block id raised by `shift`."""

    def __init__(self, u: Uploaded, shift: int):
        g = copy.copy(u.w.geom)
        g.num_blocks = u.w.geom.num_blocks + shift
        self.geom, self.shift = g, shift
        esz = u.storage.element_size()
        self.storage = torch.empty(g.total_elems, dtype=u.storage.dtype, device=DEV)
        self.base = shift * g.stride_block
        log(f"lifted cache: {g.total_elems * esz / 2**30:.2f} GiB, first used byte at {self.base * esz / 2**30:.2f} GiB")
        self.storage[self.base: self.base + u.storage.numel()] = u.storage
        self.bt = u.bt + shift
        self.slots = torch.where(u.slots >= 0, u.slots + shift * g.block_size, u.slots)
        self.desc = pk.CacheDesc.from_geom(self.storage, g, u.k_scale, u.v_scale, u.w.scale_mode)

    def region(self, n):
        return self.storage[self.base: self.base + n]


@pytest.mark.parametrize("kv,bs,shift", [("bf16", 16, 110_000), ("bf16", 24, 75_000), ("fp8", 16, 220_000)])
def test_split_kv_and_write_above_4gb(gpu_lib, kv, bs, shift):
    scales = "none" if kv == "bf16" else "head"
    g = workloads.diffkv_geom(0, bs, kv_dtype=kv)
    lens, qlens = [900, 37, 0, 400], [1, 1, 1, 1]
    w = workloads.paged_workload("big", g, lens, qlens, 32, 1 / math.sqrt(192), seed=81, scale_mode=scales)
    small = Uploaded(w)
    big = Lifted(small, shift)
    n = small.storage.numel()
    # cache write of every key, then decode with 7 partitions
    pk.cache_write(small.key, small.value, small.slots, small.desc)
    pk.cache_write(small.key, small.value, big.slots, big.desc)
    torch.cuda.synchronize()
    assert torch.equal(big.region(n), small.storage), "written rows differ above 4 GB"
    o1, l1, _ = pk.decode_splitkv(small.q, small.desc, small.bt, small.seq_lens, w.softmax_scale, 7)
    o2, l2, _ = pk.decode_splitkv(small.q, big.desc, big.bt, small.seq_lens, w.softmax_scale, 7)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "decode differs above 4 GB"
    ref, ref_lse = oracle_attention(w, small.cache_bytes())
    compare(o1, ref, fp8=kv == "fp8", lse_gpu=l1, lse_ref=ref_lse, what=f"compact decode {kv} bs {bs}")
    # the fused write-and-decode rewrites each sequence's last key in both caches
    _, (key, value, slots) = split_last_keys(w, small)
    lifted_slots = torch.where(slots >= 0, slots + shift * g.block_size, slots)
    o3, l3, _ = pk.decode_splitkv_append(small.q, key, value, slots, small.desc, small.bt, small.seq_lens,
                                         w.softmax_scale, 5)
    o4, l4, _ = pk.decode_splitkv_append(small.q, key, value, lifted_slots, big.desc, big.bt, small.seq_lens,
                                         w.softmax_scale, 5)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4) and torch.equal(big.region(n), small.storage)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_verify_and_prefill_above_4gb(gpu_lib, kv):
    scales = "none" if kv == "bf16" else "tensor"
    g = workloads.diffkv_geom(0, 16, kv_dtype=kv)
    shift = 110_000 if kv == "bf16" else 220_000
    # verify: 4 tokens x 8 heads = 32 rows per KV head (the wide kernel for fp8)
    w = workloads.paged_workload("bigv", g, [700, 129], [4, 4], 32, 1 / math.sqrt(192), seed=82, scale_mode=scales)
    small = Uploaded(w)
    small.write()
    big = Lifted(small, shift)
    o1, l1, _ = pk.verify(small.q, small.qsl, small.seq_lens, small.bt, small.desc, w.softmax_scale, 4, 6)
    o2, l2, _ = pk.verify(small.q, small.qsl, small.seq_lens, big.bt, big.desc, w.softmax_scale, 4, 6)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "verify differs above 4 GB"
    ref, ref_lse = oracle_attention(w, small.cache_bytes())
    compare(o1, ref, fp8=kv == "fp8", lse_gpu=l1, lse_ref=ref_lse, what=f"compact verify {kv}")
    # prefill (fast kernel for bf16, generic for fp8)
    w = workloads.paged_workload("bigp", g, [300, 129], [300, 65], 32, 1 / math.sqrt(192), seed=83,
                                 scale_mode=scales)
    small = Uploaded(w)
    small.write()
    big = Lifted(small, shift)
    o1, l1 = pk.prefill_causal(small.q, small.qsl, small.seq_lens, small.bt, small.desc, w.softmax_scale, 300)
    o2, l2 = pk.prefill_causal(small.q, small.qsl, small.seq_lens, big.bt, big.desc, w.softmax_scale, 300)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "prefill differs above 4 GB"


def test_mla_above_4gb(gpu_lib):
    w = workloads.paged_workload("bigm", workloads.mla_geom(0, 64), [2000, 65], [1, 1], 12, 1 / math.sqrt(576),
                                 seed=84, std=0.1)
    small = Uploaded(w)
    small.write()
    big = Lifted(small, 60_000)
    o1, l1, _ = pk.decode_splitkv(small.q, small.desc, small.bt, small.seq_lens, w.softmax_scale, 9)
    o2, l2, _ = pk.decode_splitkv(small.q, big.desc, big.bt, small.seq_lens, w.softmax_scale, 9)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "MLA decode differs above 4 GB"
    # the multi-token MLA verify (shared-ring token kernel)
    w = workloads.paged_workload("bigmv", workloads.mla_geom(0, 16), [1500, 70], [4, 3], 12, 1 / math.sqrt(576),
                                 seed=85, std=0.1)
    small = Uploaded(w)
    small.write()
    big = Lifted(small, 240_000)
    o1, l1, _ = pk.verify(small.q, small.qsl, small.seq_lens, small.bt, small.desc, w.softmax_scale, 4, 7)
    o2, l2, _ = pk.verify(small.q, small.qsl, small.seq_lens, big.bt, big.desc, w.softmax_scale, 4, 7)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "MLA verify differs above 4 GB"
    ref, ref_lse = oracle_attention(w, small.cache_bytes())
    compare(o1, ref, lse_gpu=l1, lse_ref=ref_lse, what="compact MLA verify")
