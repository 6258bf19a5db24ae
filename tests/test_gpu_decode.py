"""GPU parity of attn_decode_splitkv (+ attn_merge_lse) against the fp64 oracle.

Split-KV decode with runtime partition ranges (vLLM PR #50371, review thread) and
GQA-grouped K/V reads; empty rows give 0 (diffbot model card, "Update 2026-10-01").
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention

pytestmark = pytest.mark.gpu


def run_decode(u, P, **kw):
    w = u.w
    return pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, **kw)


@pytest.mark.parametrize("P", [1, 2, 7, 16, 64])
def test_tiny_config(gpu_lib, P):
    w = workloads.tiny()
    u = Uploaded(w)
    u.write()
    out, lse, _ = run_decode(u, P)
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"tiny P={P}", strict=True)


@pytest.mark.parametrize("lens", [[1], [15, 16, 17], [0, 5, 0], [300, 1, 33], [1000]])
@pytest.mark.parametrize("bs", [16, 64])
def test_ragged_lengths_and_empty_rows(gpu_lib, lens, bs):
    g = workloads.diffkv_geom(0, bs)
    w = workloads.paged_workload("dec", g, lens, [1] * len(lens), 32, 1 / math.sqrt(192), seed=21)
    u = Uploaded(w)
    u.write()
    for P in (1, 5, 32):
        out, lse, _ = run_decode(u, P)
        ref, ref_lse = oracle_attention(w, u.cache_bytes())
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"lens={lens} bs={bs} P={P}")
        for b, s in enumerate(lens):
            if s == 0:
                o = out[b].float().cpu()
                assert torch.all(o == 0) and not torch.any(torch.signbit(o))
                assert torch.all(torch.isneginf(lse[b].cpu()))


def test_split_invariance_and_partials_path(gpu_lib):
    g = workloads.diffkv_geom(0, 16)
    w = workloads.paged_workload("dec", g, [2000, 777], [1, 1], 32, 1 / math.sqrt(192), seed=22)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    outs = []
    for P in (1, 3, 16, 64, 125):
        out, lse, ws = run_decode(u, P)
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"P={P}")
        outs.append(out.float())
        # partials only, then the separate merge call: identical to the one-call result
        _, _, ws2 = run_decode(u, P, partials_only=True)
        from paged_kv_cache_176_amd.ops import workspace_views
        po, pl = workspace_views(ws2, 2, 32, 128, P)
        out2, lse2 = pk.merge_lse(po.contiguous(), pl.contiguous())
        # same partials, merged in a different summation order: within one bf16 ulp
        assert torch.all((out2.float() - out.float()).abs() <= out.float().abs() * 2.0 ** -7 + 1e-6)
        assert torch.allclose(lse2, lse, rtol=0, atol=1e-5)
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) < 4e-3


def test_block_permutation_is_bit_exact(gpu_lib):
    w = workloads.tiny()
    u = Uploaded(w)
    u.write()
    out, lse, _ = run_decode(u, 3)
    # move the physical blocks and rewrite the tables: results must not change at all
    g = w.geom
    perm = torch.randperm(g.num_blocks, generator=torch.Generator().manual_seed(9))
    view = u.storage[: g.cache_elems].view(g.num_blocks, -1)
    moved = u.storage.clone()
    moved[: g.cache_elems].view(g.num_blocks, -1)[perm.to(DEV)] = view
    u.storage = moved
    u.desc.storage = moved
    u.bt = perm.to(DEV)[u.bt.long()].to(torch.int32)
    out2, lse2, _ = run_decode(u, 3)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_gqa_equals_mha_with_repeated_kv(gpu_lib):
    """32 q heads over 4 KV heads == 32 q heads over 32 KV heads holding repeated rows."""
    w = workloads.paged_workload("gqa", workloads.diffkv_geom(0, 16), [333], [1], 32, 1 / math.sqrt(192), seed=23)
    u = Uploaded(w)
    u.write()
    out, lse, _ = run_decode(u, 4)
    g2 = workloads.diffkv_geom(0, 16, num_kv_heads=32)
    w2 = workloads.paged_workload("mha", g2, [333], [1], 32, 1 / math.sqrt(192), seed=23)
    w2.q = w.q
    w2.key = w.key.repeat_interleave(8, dim=1)
    w2.value = w.value.repeat_interleave(8, dim=1)
    w2.slot_mapping = w.slot_mapping
    w2.block_tables = w.block_tables
    g2.num_blocks = w.geom.num_blocks
    w2.cache_init = torch.zeros(g2.total_elems, dtype=torch.int16)
    u2 = Uploaded(w2)
    u2.write()
    out2, lse2, _ = run_decode(u2, 4)
    assert float((out.float() - out2.float()).abs().max()) <= 1e-2 / 4
    assert float((lse - lse2).abs().max()) <= 1e-4


# the first split of each shape is the one bench.py times (two workgroups per CU), the
# second another one; both against the same oracle result
@pytest.mark.parametrize("shape", [(1, 131072, 16, (128, 64)), (1, 131072, 64, (128, 16)), (8, 8192, 16, (16, 8)),
                                   (8, 8192, 64, (16, 32))])
def test_long_context_config(gpu_lib, shape):
    B, S, bs, Ps = shape
    log(f"long decode B={B} S={S} bs={bs} P={Ps}: generating")
    w = workloads.long_decode(B, S, bs)
    u = Uploaded(w)
    u.write()
    outs = [run_decode(u, P)[:2] for P in Ps]
    log("oracle")
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P, (out, lse) in zip(Ps, outs):
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"decode B{B} S{S} bs{bs} P{P}", strict=True)
