"""GPU parity of the exported split-KV partials: with out = NULL the partial kernels leave each
partition's normalised output and log-sum-exp in the workspace for attn_merge_lse -- the first
stage of the two-stage decode (vLLM PR #50371, review thread) and the split-KV reducer's segments
(diffbot model card, "Update 2026-10-01: three correctness fixes").  Each partition is compared
element by element with the oracle's partials over the same 16-key-rounded key range (the header's
num_partitions rule, whatever the block size); empty partitions must hold exactly 0 and -inf."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import Uploaded, compare, log
from oracle import paged_ref as R

pytestmark = pytest.mark.gpu


def oracle_partials(w, cache_np, P):
    qb = w.q.view(torch.int16).numpy().view(np.uint16)
    ks = w.k_scale.numpy() if w.k_scale is not None else None
    vs = w.v_scale.numpy() if w.v_scale is not None else None
    return R.paged_attention_partials(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(),
                                      cache_np, R.CacheSpec.from_geom(w.geom), w.softmax_scale, P, ks, vs)


def check_partials(ws, w, cache_np, P, fp8, what):
    rows, Hq, Dv = w.num_tokens, w.num_q_heads, w.geom.head_dim_v
    po, pl = pk.ops.workspace_views(ws, rows, Hq, Dv, P)
    po, pl = po.cpu(), pl.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle_partials(w, cache_np, P)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(pl), empty), f"{what}: empty-partition pattern"
    assert torch.all(po[torch.from_numpy(empty)] == 0), f"{what}: empty partials not 0"
    live = ~empty
    log(f"{what}: {int(live.sum())} live (row, head, partition) partials of {live.size}")
    if live.any():
        compare(po[torch.from_numpy(live)], ref_o[live], fp8=fp8, what=what, strict=True)
        d = float(np.abs(pl[live] - ref_l[live]).max())
        assert d <= 1e-3, f"{what}: lse err {d}"


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("P", [1, 7, 128])
def test_decode_partials(gpu_lib, bs, P):
    g = workloads.diffkv_geom(0, bs)
    w = workloads.paged_workload("parts", g, [3000, 1000, 37, 0], [1, 1, 1, 1], 32, 1 / math.sqrt(192), seed=71)
    u = Uploaded(w)
    u.write()
    _, _, ws = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, partials_only=True)
    check_partials(ws, w, u.cache_bytes(), P, False, f"decode partials bs={bs} P={P}")


@pytest.mark.parametrize("P", [1, 7, 128])
def test_mla_decode_partials(gpu_lib, P):
    w = workloads.paged_workload("parts_mla", workloads.mla_geom(0, 64), [5000, 300, 0], [1, 1, 1], 12,
                                 1 / math.sqrt(576), seed=72, std=0.1, q_std=0.8)
    u = Uploaded(w)
    u.write()
    _, _, ws = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, partials_only=True)
    check_partials(ws, w, u.cache_bytes(), P, False, f"mla decode partials P={P}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [1, 7, 33])
def test_verify_partials(gpu_lib, kv, P):
    """Verify rows (4 tokens x 8 heads per KV head): the bf16 LDS-streamed kernel, the fp8 32-row
    kernel; rows whose keys all lie past a partition's range are empty there."""
    g = workloads.diffkv_geom(0, 16, kv_dtype=kv)
    w = workloads.paged_workload("parts_v", g, [2000, 45, 3], [4, 4, 2], 32, 1 / math.sqrt(192), seed=73,
                                 scale_mode="head" if kv == "fp8" else "none", extra_empty_rows=1)
    u = Uploaded(w)
    u.write()
    _, _, ws = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P,
                         partials_only=True)
    check_partials(ws, w, u.cache_bytes(), P, kv == "fp8", f"{kv} verify partials P={P}")


def test_mla_verify_partials(gpu_lib):
    w = workloads.paged_workload("parts_mv", workloads.mla_geom(0, 64), [3000, 70], [4, 3], 12,
                                 1 / math.sqrt(576), seed=74, std=0.1, q_std=0.8)
    u = Uploaded(w)
    u.write()
    _, _, ws = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, 9,
                         partials_only=True)
    check_partials(ws, w, u.cache_bytes(), 9, False, "mla verify partials P=9")
