"""GPU parity of the multi-token MLA verify: 2 or more query tokens per sequence over the
576-wide latent KV head (V = the row's first 512 columns), each token seeing the keys up
to its own position -- the verify case the single-token MLA path leaves open (vLLM PR
#50371, review thread).  attn_verify serves it with one wave per token over a shared LDS
ring.  Each case is checked against the oracle on the same cache bytes; the 16-head call
with heads 12-15 zero must leave heads 0-11 bit-identical."""
import math

import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention


pytestmark = pytest.mark.gpu


def run(u, w, P, q=None):
    return pk.verify(u.q if q is None else q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P)


def padded16(q12):
    return torch.cat([q12, torch.zeros(q12.shape[0], 4, q12.shape[2], dtype=q12.dtype, device=q12.device)], dim=1)


@pytest.mark.parametrize("bs,lens,qlens", [
    (64, [3000, 700, 5, 2], [4, 2, 3, 2]),          # ragged drafts, one token group
    (16, [2000, 300, 9], [7, 5, 8]),                # 5-8 tokens: two token groups
    (32, [1500, 0, 40, 1], [3, 1, 4, 1]),           # an empty sequence and single-token rows
])
def test_mla_verify_small(gpu_lib, bs, lens, qlens):
    w = workloads.paged_workload("mla_verify", workloads.mla_geom(0, bs), lens, qlens, 12, 1 / math.sqrt(576),
                                 seed=61, std=0.1)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P in (1, 5, 33):
        log(f"MLA verify bs {bs} lens {lens} L {qlens} P {P}")
        out, lse, _ = run(u, w, P)
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"mla verify bs={bs} L={qlens} P={P}")
        out16, lse16, _ = run(u, w, P, q=padded16(u.q))
        assert torch.equal(out16[:, :12], out) and torch.equal(lse16[:, :12], lse)


@pytest.mark.parametrize("G", [8, 16])
def test_mla_verify_heads(gpu_lib, G):
    """Other group sizes that the kernel takes (up to 16 query heads per KV head)."""
    w = workloads.paged_workload("mla_verify_g", workloads.mla_geom(0, 64), [1000, 77], [3, 4], G,
                                 1 / math.sqrt(576), seed=62, std=0.1)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    out, lse, _ = run(u, w, 6)
    compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"mla verify G={G}")


def test_mla_verify_peaked(gpu_lib):
    """Near-uniform scores hide a wrong causal limit; a needle at each token's last visible
    key (and one key past it) tells the tokens apart."""
    lens, L = [2500, 600], 4
    w = workloads.paged_workload("mla_verify_peak", workloads.mla_geom(0, 64), lens, [L, L], 12,
                                 1 / math.sqrt(576), seed=63, std=0.1)
    w.q = (w.q.float() * 8).to(torch.bfloat16)
    for b, S in enumerate(lens):
        t0 = int(w.query_start_loc[b].item())
        base = sum(lens[:b])
        for i in range(L):                        # key S-L+i lines up with token i's heads
            w.key[base + S - L + i, 0] = (w.q[t0 + i].float().mean(0) * 4).to(torch.bfloat16)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    out, lse, _ = run(u, w, 16)
    compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what="mla verify peaked")


# the split count is the one bench.py times
@pytest.mark.parametrize("B,P", [(1, 224), (4, 64)])
def test_mla_verify_config(gpu_lib, B, P):
    log(f"MLA verify B={B} x 100000, 4 tokens: generating")
    w = workloads.mla_verify(B, 100000, qlen=4)
    u = Uploaded(w)
    u.write()
    out, lse, _ = run(u, w, P)
    seqs = [0] if B == 1 else [0, B - 1]
    qsl = w.query_start_loc.tolist()
    toks = [r for b in seqs for r in range(qsl[b], qsl[b + 1])]
    log(f"oracle on seqs {seqs} (tokens {toks})")
    ref, ref_lse = oracle_attention(w, u.cache_bytes(), rows=toks)
    idx = torch.tensor(toks, device=DEV)
    compare(out[idx], ref, lse_gpu=lse[idx], lse_ref=ref_lse, what=f"mla verify B{B} P{P}", strict=True)
