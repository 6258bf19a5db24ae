"""Verify and prefill calls captured in a HIP graph reproduce the eager calls on every replay:
the fp8 32-row verify kernel, the bf16 DiffKV verify, the multi-token MLA verify (token
kernel) and the chunked-prefill kernel.  Before each replay the query is rewritten in place
with new values and every output is poisoned, so a replay must recompute everything; between
replays runs eager work of its own, with synchronisations.  Each replay equals an eager call
on the same inputs bit for bit, and the eager call equals the oracle."""
import math

import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention

pytestmark = pytest.mark.gpu

CASES = {
    # name: (geometry, q heads, scale, value std, seq lens, query lens, fp8 scale mode)
    "fp8_verify": (lambda: workloads.diffkv_geom(0, 16, kv_dtype="fp8"), 32, 1 / math.sqrt(192), 1.0,
                   [700, 300, 0], [4, 4, 1], "tensor"),
    "bf16_verify": (lambda: workloads.diffkv_geom(0, 16), 32, 1 / math.sqrt(192), 1.0, [500, 90], [3, 2], "none"),
    "mla_verify": (lambda: workloads.mla_geom(0, 64), 12, 1 / math.sqrt(576), 0.1, [900, 130], [4, 3], "none"),
    "prefill": (lambda: workloads.diffkv_geom(0, 16), 32, 1 / math.sqrt(192), 1.0, [300, 96], [160, 96], "none"),
}


def _capture(step):
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
    return graph


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_recompute(gpu_lib, name):
    geom, hq, scale, std, lens, qlens, mode = CASES[name]
    g = geom()
    w = workloads.paged_workload("graph_v", g, lens, qlens, hq, scale, seed=130, std=std, scale_mode=mode)
    u = Uploaded(w)
    u.write()
    T, P = w.q.shape[0], 8
    q = u.q.clone()
    out = torch.empty(T, hq, g.head_dim_v, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, hq, dtype=torch.float32, device=DEV)
    ws = pk.new_workspace(T, hq, g.head_dim_v, P, DEV)

    def call(q_, out_=None, lse_=None, ws_=None):
        if name == "prefill":
            return pk.prefill_causal(q_, u.qsl, u.seq_lens, u.bt, u.desc, scale, w.max_query_len, out=out_,
                                     out_lse=lse_)[:2]
        return pk.verify(q_, u.qsl, u.seq_lens, u.bt, u.desc, scale, w.max_query_len, P, out=out_, out_lse=lse_,
                         workspace=ws_)[:2]

    graph = _capture(lambda: call(q, out, lse, ws))
    gen = torch.Generator().manual_seed(131)
    for r in range(3):
        log(f"{name}: replay {r}")
        q.copy_((torch.randn(tuple(q.shape), generator=gen) * std).to(torch.bfloat16))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el = call(q.clone())                      # eager, its own buffers
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"{name} replay {r} differs from the eager call"
        wq = workloads.Workload(**{**w.__dict__, "q": q.cpu()})
        ref, ref_lse = oracle_attention(wq, u.cache_bytes())
        compare(eo, ref, fp8=g.kv_dtype == "fp8", lse_gpu=el, lse_ref=ref_lse, what=f"{name} replay {r}")
