"""A decode step (cache write of the new token, split-KV partials, merge) captured in a
HIP graph must reproduce the eagerly launched step on every replay, with eager work and
synchronisations between the replays: the entry points enqueue kernels only (no memset
nodes, no host synchronisation), so capture records exactly the eager launches.  The
"one_call" step is attn_decode_splitkv_append with an output buffer: the library
enqueues the partial kernel (new-token write inside) and the merge itself."""
import math

import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["separate", "append", "one_call"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_decode_step_graph_replays(gpu_lib, kv, mode):
    g = workloads.diffkv_geom(0, 16, kv_dtype=kv)
    w = workloads.paged_workload("graph", g, [3000, 517], [1, 1], 32, 1 / math.sqrt(192), seed=41,
                                 scale_mode="none" if kv == "bf16" else "head")
    u = Uploaded(w)
    u.write()
    P = 12
    B, Hq = w.q.shape[0], w.q.shape[1]
    key, value, slots = w.key.to(DEV), w.value.to(DEV), w.slot_mapping.to(DEV)
    if mode != "separate":                           # one token per sequence: its last key
        last = torch.cumsum(w.seq_lens.to(torch.int64), 0) - 1
        key, value, slots = key[last.to(DEV)], value[last.to(DEV)], slots[last.to(DEV)]
    ws = pk.new_workspace(B, Hq, g.head_dim_v, P, DEV)
    po, pl = pk.ops.workspace_views(ws, B, Hq, g.head_dim_v, P)
    out = torch.empty(B, Hq, g.head_dim_v, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)

    def step():
        if mode == "one_call":                       # write + partials, then the merge: one call
            pk.decode_splitkv_append(u.q, key, value, slots, u.desc, u.bt, u.seq_lens, w.softmax_scale, P,
                                     out=out, out_lse=lse, workspace=ws)
            return
        if mode == "append":                         # the write rides in the partial kernel
            pk.decode_splitkv_append(u.q, key, value, slots, u.desc, u.bt, u.seq_lens, w.softmax_scale, P,
                                     workspace=ws, partials_only=True)
        else:
            pk.cache_write(key, value, slots, u.desc)
            pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, workspace=ws, partials_only=True)
        pk.merge_lse(po, pl, out=out, out_lse=lse)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()

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

    for r in range(4):
        out.zero_()
        lse.fill_(float("nan"))
        po.fill_(float("nan"))                       # the replay must rewrite every partial it reads
        pl.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: output differs from the eager step"
        assert torch.equal(lse, ref_lse), f"replay {r}: lse differs from the eager step"
        # eager work between replays: a different decode into separate buffers
        o2, l2, _ = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, 3)
        torch.cuda.synchronize()
        assert torch.isfinite(o2.float()).all()
