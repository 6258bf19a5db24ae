"""GPU parity of the split-KV shapes served by the register-prefetch fallback kernel:
block sizes that are not a power of two >= 16 (a 16-key tile then straddles blocks and
each lane looks up its own key's block) and 33-64 query rows per KV head (verify with
up to 8 tokens x 8 GQA heads).  Same contract and oracle as the fast paths (vLLM PR
#64064, "Tests": several block sizes; diffbot model card, "What the kernels do")."""
import math

import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import Uploaded, compare, oracle_attention

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [8, 24, 48])
def test_decode_other_block_sizes(gpu_lib, kv, bs):
    g = workloads.diffkv_geom(0, bs, kv_dtype=kv)
    lens = [700, 23, 0, 161]
    w = workloads.paged_workload("fb", g, lens, [1] * len(lens), 32, 1 / math.sqrt(192), seed=61,
                                 scale_mode="none" if kv == "bf16" else "head")
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P in (1, 5, 19):
        out, lse, _ = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P)
        compare(out, ref, fp8=kv == "fp8", lse_gpu=lse, lse_ref=ref_lse, what=f"{kv} bs={bs} P={P}")
        o = out[2].float().cpu()
        assert torch.all(o == 0) and not torch.any(torch.signbit(o))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("qlens,bs", [([8, 5, 1], 16), ([6, 8], 64), ([4, 4], 8)])
def test_verify_many_rows_and_small_blocks(gpu_lib, kv, qlens, bs):
    g = workloads.diffkv_geom(0, bs, kv_dtype=kv)
    lens = [900, 333, 64][: len(qlens)]
    w = workloads.paged_workload("fbv", g, lens, qlens, 32, 1 / math.sqrt(192), seed=62,
                                 scale_mode="none" if kv == "bf16" else "tensor", extra_empty_rows=2)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    for P in (1, 6):
        out, lse, _ = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P)
        compare(out, ref, fp8=kv == "fp8", lse_gpu=lse, lse_ref=ref_lse, what=f"{kv} L={qlens} bs={bs} P={P}")
        tail = out[-2:].float().cpu()
        assert torch.all(tail == 0) and not torch.any(torch.signbit(tail))
