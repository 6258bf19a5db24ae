"""GPU parity across cache layouts: NHD [block][slot][head][row], HND [block][head][slot][row]
(the two layouts the attention backend hands the asymmetric write, vLLM PR #64064, "Tests")
and padded row and block pitches.  The same logical workload in every layout must give the
same logical cache rows after attn_cache_write (bit for bit, padding untouched) and
bit-identical outputs and log-sum-exps from every attention entry point, against the NHD run
-- which is itself checked against the oracle, as is each HND run."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention, split_last_keys

pytestmark = pytest.mark.gpu

LAYOUTS = [("NHD", 0, 0), ("HND", 0, 0), ("NHD", 64, 128), ("HND", 32, 80)]


def rows_of(u):
    return u.w.geom.rows_view(u.storage)


def padding_untouched(u):
    g = u.w.geom
    covered = torch.zeros(g.total_elems, dtype=torch.bool)
    covered[g.rows_view(torch.arange(g.total_elems, dtype=torch.int64)).reshape(-1)] = True
    got = u.storage.cpu()
    return torch.equal(got[~covered], u.w.cache_init[~covered])


def run_all(w, kv):
    """cache write of every key but each sequence's last, then (a) the fused write-and-
    decode of the last keys, (b) decode, (c) verify, (d) prefill; returns the results."""
    u = Uploaded(w)
    setup, (key, value, slots) = split_last_keys(w, u)
    pk.cache_write(*setup, u.desc)
    res = {"append": pk.decode_splitkv_append(u.q[w.query_start_loc[1:].to(DEV) - 1], key, value, slots, u.desc,
                                              u.bt, u.seq_lens, w.softmax_scale, 5)[:2]}
    res["decode"] = pk.decode_splitkv(u.q[w.query_start_loc[1:].to(DEV) - 1], u.desc, u.bt, u.seq_lens,
                                      w.softmax_scale, 7)[:2]
    res["verify"] = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, 6)[:2]
    res["prefill"] = pk.prefill_causal(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len)
    torch.cuda.synchronize()
    return u, res


@pytest.mark.parametrize("kv,scales,bs", [("bf16", "none", 16), ("fp8", "head", 16), ("bf16", "none", 64),
                                          ("fp8", "tensor", 32)])
def test_diffkv_layouts(gpu_lib, kv, scales, bs):
    base = None
    for layout, row_pad, block_pad in LAYOUTS:
        log(f"{kv}/{scales} bs {bs}: {layout} row pad {row_pad} block pad {block_pad}")
        g = workloads.diffkv_geom(0, bs, kv_dtype=kv, layout=layout, row_pad=row_pad, block_pad=block_pad)
        w = workloads.paged_workload("layouts", g, [900, 37, 260, 4], [4, 1, 3, 2], 32, 1 / math.sqrt(192),
                                     seed=95, scale_mode=scales)
        u, res = run_all(w, kv)
        assert padding_untouched(u), f"{layout}: a write touched padding or slack"
        if base is None:
            base = (rows_of(u).cpu(), res)
            ref, ref_lse = oracle_attention(w, u.cache_bytes())
            compare(res["verify"][0], ref, fp8=kv == "fp8", lse_gpu=res["verify"][1], lse_ref=ref_lse,
                    what=f"{layout} verify vs oracle")
            continue
        assert torch.equal(rows_of(u).cpu(), base[0]), f"{layout}: cache rows differ from NHD"
        for name, (o, l) in res.items():
            assert torch.equal(o, base[1][name][0]), f"{layout}: {name} output differs from NHD"
            if l is not None:
                assert torch.equal(l, base[1][name][1]), f"{layout}: {name} lse differs from NHD"
        if layout == "HND" and row_pad == 0:
            ref, ref_lse = oracle_attention(w, u.cache_bytes())
            compare(res["prefill"][0], ref, fp8=kv == "fp8", lse_gpu=res["prefill"][1], lse_ref=ref_lse,
                    what=f"{layout} prefill vs oracle")


def test_mla_layouts(gpu_lib):
    """The latent row (one KV head, so NHD and HND differ only by padding) in decode and verify."""
    base = None
    for layout, row_pad, block_pad in [("NHD", 0, 0), ("HND", 64, 0), ("NHD", 0, 256)]:
        g = workloads.mla_geom(0, 64, layout=layout, row_pad=row_pad, block_pad=block_pad)
        w = workloads.paged_workload("mla_layouts", g, [3000, 65, 7], [3, 1, 2], 12, 1 / math.sqrt(576), seed=96,
                                     std=0.1)
        u = Uploaded(w)
        u.write()
        dec = pk.decode_splitkv(u.q[w.query_start_loc[1:].to(DEV) - 1], u.desc, u.bt, u.seq_lens,
                                w.softmax_scale, 9)[:2]
        ver = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, 9)[:2]
        torch.cuda.synchronize()
        assert padding_untouched(u)
        if base is None:
            base = (rows_of(u).cpu(), dec, ver)
            ref, ref_lse = oracle_attention(w, u.cache_bytes())
            compare(ver[0], ref, lse_gpu=ver[1], lse_ref=ref_lse, what="MLA verify vs oracle")
            continue
        assert torch.equal(rows_of(u).cpu(), base[0])
        assert torch.equal(dec[0], base[1][0]) and torch.equal(dec[1], base[1][1]), f"{layout}: MLA decode"
        assert torch.equal(ver[0], base[2][0]) and torch.equal(ver[1], base[2][1]), f"{layout}: MLA verify"
