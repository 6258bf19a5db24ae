"""GPU parity of the native 12-head MLA decode: 12 query heads over one 576-wide latent
KV head, V = the row's first 512 columns, no padding to 16 heads (vLLM PR #50371:
"Purpose", "Test Plan"; the test there must stay valid once a native 12-head kernel
replaces the zero-padding).  The padded 16-head run through the same entry point must
leave heads 0-11 unchanged."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention

pytestmark = pytest.mark.gpu


def run(u, P, q=None):
    return pk.decode_splitkv(u.q if q is None else q, u.desc, u.bt, u.seq_lens, u.w.softmax_scale, P)


def padded16(q12):
    return torch.cat([q12, torch.zeros(q12.shape[0], 4, q12.shape[2], dtype=q12.dtype, device=q12.device)], dim=1)


@pytest.mark.parametrize("lens", [[4096], [300, 1, 0, 77]])
def test_small_mla(gpu_lib, lens):
    w = workloads.paged_workload("mla", workloads.mla_geom(0, 64), lens, [1] * len(lens), 12,
                                 1 / math.sqrt(576), seed=51, std=0.1)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P in (1, 8, 96):
        out, lse, _ = run(u, P)
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"mla lens={lens} P={P}")
        out16, lse16, _ = run(u, P, q=padded16(u.q))
        assert torch.equal(out16[:, :12], out) and torch.equal(lse16[:, :12], lse)


def test_peaked_mla(gpu_lib):
    """Scores with std 0.01 make softmax nearly uniform; scale Q by 8 and plant needles."""
    w = workloads.paged_workload("mla", workloads.mla_geom(0, 64), [5000, 2000], [1, 1], 12,
                                 1 / math.sqrt(576), seed=52, std=0.1)
    w.q = (w.q.float() * 8).to(torch.bfloat16)
    # needle: key 1234 of seq 0 and key 17 of seq 1 aligned with the heads' queries
    for b, j in ((0, 1234), (1, 17)):
        t = int((w.query_start_loc[b]).item())
        base = sum(w.seq_lens[:b].tolist())
        w.key[base + j, 0] = (w.q[t].float().mean(0) * 4).to(torch.bfloat16)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    out, lse, _ = run(u, 32)
    compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what="mla peaked")
    assert float(np.abs(ref).max()) > 0.05


# the first split of each batch is the one bench.py times
@pytest.mark.parametrize("B,Ps", [(1, (224, 256, 96)), (16, (16, 32))])
def test_mla_config(gpu_lib, B, Ps):
    log(f"MLA config B={B}: generating")
    w = workloads.mla_decode(B, 100000)
    u = Uploaded(w)
    u.write()
    outs = {}
    for P in Ps:
        out, lse, _ = run(u, P)
        out16, lse16, _ = run(u, P, q=padded16(u.q))
        assert torch.equal(out16[:, :12], out) and torch.equal(lse16[:, :12], lse)
        outs[P] = (out, lse)
    seqs = list(range(B)) if B <= 2 else [0, B // 2, B - 1]
    log(f"oracle on seqs {seqs}")
    ref, ref_lse = oracle_attention(w, u.cache_bytes(), rows=seqs)
    idx = torch.tensor(seqs, device=DEV)
    for P, (out, lse) in outs.items():
        compare(out[idx], ref, lse_gpu=lse[idx], lse_ref=ref_lse, what=f"mla B{B} P{P}", strict=True)
