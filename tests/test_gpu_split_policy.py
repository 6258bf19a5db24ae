"""GPU parity of the device-side split policy (vLLM PR #50371, review thread: active splits
chosen in both stages from device-side sequence lengths by context buckets, launch shape
graph-stable, one table for both stages).  Each sequence of a mixed batch uses only its
bucket's partitions (the rest come out empty), the merge reads only those, and the result
matches the oracle; a captured decode replayed after the sequence lengths change on the
device picks the new buckets and equals the eager call bit for bit."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention
from oracle import paged_ref as R

pytestmark = pytest.mark.gpu

POLICY = [(512, 2), (4096, 8), (16384, 24), (1 << 30, 48)]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mixed_batch_uses_each_bucket(gpu_lib, kv):
    g = workloads.diffkv_geom(0, 16, kv_dtype=kv)
    lens = [40, 1000, 6000, 20000, 0]
    w = workloads.paged_workload("policy", g, lens, [1] * len(lens), 32, 1 / math.sqrt(192), seed=102,
                                 scale_mode="none" if kv == "bf16" else "head")
    u = Uploaded(w)
    u.write()
    P = 64
    out, lse, ws = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, split_policy=POLICY)
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    compare(out, ref, fp8=kv == "fp8", lse_gpu=lse, lse_ref=ref_lse, what=f"{kv} decode with a split policy")
    # the partials: empty past each sequence's active count, and the merge of all P equals the call's
    _, _, ws2 = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, partials_only=True,
                                  split_policy=POLICY)
    po, pl = pk.ops.workspace_views(ws2, len(lens), 32, 128, P)
    pl_c, po_c = pl.cpu(), po.cpu()
    for b, S in enumerate(lens):
        k = R.active_splits(S, P, POLICY)
        log(f"seq {b}: {S} keys -> {k} active splits")
        assert torch.all(pl_c[b, :, k:] == -math.inf) and torch.all(po_c[b, :, k:] == 0)
        for p, (lo, hi) in enumerate(R.partition_ranges(S, k, 16)):    # 16-key rounding, as the kernels
            assert bool(torch.all(torch.isfinite(pl_c[b, :, p]))) == (hi > lo), f"seq {b} split {p}"
    o2, l2 = pk.merge_lse(po, pl)
    assert torch.equal(o2, out) and torch.equal(l2, lse), "reading only the active partials changed the merge"


def test_verify_with_a_split_policy(gpu_lib):
    """Verify rows (DiffKV fp8 32-row kernel, bf16 and the MLA token kernel) under a policy."""
    for geom, hq, scale, std, qlens in [(workloads.diffkv_geom(0, 16, kv_dtype="fp8"), 32, 1 / math.sqrt(192), 1.0,
                                         [4, 2, 1]),
                                        (workloads.diffkv_geom(0, 16), 32, 1 / math.sqrt(192), 1.0, [3, 3, 1]),
                                        (workloads.mla_geom(0, 64), 12, 1 / math.sqrt(576), 0.1, [4, 2, 3])]:
        w = workloads.paged_workload("policy_v", geom, [9000, 300, 2000], qlens, hq, scale, seed=103, std=std,
                                     scale_mode="tensor" if geom.kv_dtype == "fp8" else "none")
        u = Uploaded(w)
        u.write()
        out, lse, _ = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, 32,
                                split_policy=POLICY)
        ref, ref_lse = oracle_attention(w, u.cache_bytes())
        compare(out, ref, fp8=geom.kv_dtype == "fp8", lse_gpu=lse, lse_ref=ref_lse,
                what=f"verify {geom.kv_dtype} rows {geom.row_dim} with a policy")


def test_graph_replay_follows_device_lengths(gpu_lib):
    """One capture, three replays: seq_lens rewritten on the device between them (every
    length stays within the keys written) move sequences between buckets."""
    g = workloads.diffkv_geom(0, 16)
    full = [20000, 3000, 400]
    w = workloads.paged_workload("policy_g", g, full, [1, 1, 1], 32, 1 / math.sqrt(192), seed=104)
    u = Uploaded(w)
    u.write()
    P = 48
    sl = u.seq_lens.clone()
    ws = pk.new_workspace(3, 32, 128, P, DEV)
    out = torch.empty(3, 32, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(3, 32, dtype=torch.float32, device=DEV)

    def step():
        pk.decode_splitkv(u.q, u.desc, u.bt, sl, w.softmax_scale, P, out=out, out_lse=lse, workspace=ws,
                          split_policy=POLICY)

    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for lens in ([20000, 3000, 400], [5000, 600, 250], [300, 2999, 16], [16385, 512, 1]):
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el, _ = pk.decode_splitkv(u.q, u.desc, u.bt, sl, w.softmax_scale, P, split_policy=POLICY)
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"replay at {lens} differs from the eager call"
        # the oracle over the first `lens` keys of each sequence, the query unchanged
        wl = workloads.Workload(**{**w.__dict__, "seq_lens": torch.tensor(lens, dtype=torch.int32)})
        ref, ref_lse = oracle_attention(wl, u.cache_bytes())
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"graph replay at lengths {lens}")
