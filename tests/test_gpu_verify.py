"""GPU parity of attn_verify: several query tokens per sequence, causal among themselves,
split-KV, bf16 or fp8 (E4M3FN) caches with per-tensor or per-head scales, and padded
rows with seq_len 0 that must output exact zeros (diffbot MiMo-V2.6-Flash model card,
"What the kernels do", "Benchmarks", "Update 2026-10-01")."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention

pytestmark = pytest.mark.gpu


def run_verify(u, P, **kw):
    w = u.w
    return pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P, **kw)


@pytest.mark.parametrize("kv", ["bf16", "fp8_tensor", "fp8_head"])
@pytest.mark.parametrize("qlens", [[1, 1], [4, 4], [2, 3, 1], [4, 1, 4]])
def test_small_verify(gpu_lib, kv, qlens):
    mode = {"bf16": "none", "fp8_tensor": "tensor", "fp8_head": "head"}[kv]
    g = workloads.diffkv_geom(0, 16, kv_dtype="bf16" if kv == "bf16" else "fp8")
    lens = [300, 47, 1000][: len(qlens)]
    w = workloads.paged_workload("ver", g, lens, qlens, 32, 1 / math.sqrt(192), seed=31, scale_mode=mode,
                                 extra_empty_rows=2)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P in (1, 4, 33):
        out, lse, _ = run_verify(u, P)
        compare(out, ref, fp8=kv != "bf16", lse_gpu=lse, lse_ref=ref_lse, what=f"{kv} L={qlens} P={P}")
        tail = out[-2:].float().cpu()
        assert torch.all(tail == 0) and not torch.any(torch.signbit(tail))


def test_verify_row_equals_decode_at_its_position(gpu_lib):
    """Verify query i of L sees exactly what a decode at S - L + i + 1 keys sees."""
    g = workloads.diffkv_geom(0, 16)
    w = workloads.paged_workload("ver", g, [500], [4], 32, 1 / math.sqrt(192), seed=32)
    u = Uploaded(w)
    u.write()
    out, lse, _ = run_verify(u, 8)
    for i in range(4):
        sl = torch.tensor([500 - 4 + i + 1], dtype=torch.int32, device=DEV)
        o, l, _ = pk.decode_splitkv(u.q[i: i + 1], u.desc, u.bt, sl, w.softmax_scale, 8)
        assert float((o.float() - out[i: i + 1].float()).abs().max()) <= 4e-3
        assert float((l - lse[i: i + 1]).abs().max()) <= 1e-4


@pytest.mark.parametrize("mode", ["tensor", "head"])
def test_fp8_verify_config(gpu_lib, mode):
    """4 seqs x 46080 keys, 4 query tokens each, fp8 cache, plus 4 rows with seq_len 0."""
    log(f"fp8 verify config ({mode} scales): generating")
    w = workloads.fp8_verify(scale_mode=mode)
    u = Uploaded(w)
    u.write()
    outs = {P: run_verify(u, P)[:2] for P in (16, 64)}      # 16: the split bench.py times
    log("oracle")
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P, (out, lse) in outs.items():
        compare(out, ref, fp8=True, lse_gpu=lse, lse_ref=ref_lse, what=f"fp8 verify {mode} P{P}", strict=True)
        tail = out[16:].float().cpu()
        assert torch.all(tail == 0) and not torch.any(torch.signbit(tail))
        assert torch.all(torch.isneginf(lse[16:].cpu()))
