"""GPU parity of attn_prefill_causal: chunked causal prefill over the paged cache
(4096-token chunks, GQA; diffbot MiMo-V2.6-Flash model card, "What the kernels do")."""
import copy
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention

pytestmark = pytest.mark.gpu


def run_prefill(u, **kw):
    w = u.w
    return pk.prefill_causal(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, **kw)


@pytest.mark.parametrize("kv", ["bf16", "fp8_head"])
@pytest.mark.parametrize("case", ["single", "ragged", "context"])
def test_small_prefill(gpu_lib, kv, case):
    mode = "none" if kv == "bf16" else "head"
    g = workloads.diffkv_geom(0, 16, kv_dtype="bf16" if kv == "bf16" else "fp8")
    if case == "single":
        lens, qlens = [256], [256]
    elif case == "ragged":
        lens, qlens = [37, 100, 1, 65], [37, 100, 1, 65]
    else:  # queries are the tail of a longer context (chunk c > 0)
        lens, qlens = [300, 129], [77, 33]
    w = workloads.paged_workload("pf", g, lens, qlens, 32, 1 / math.sqrt(192), seed=41, scale_mode=mode)
    u = Uploaded(w)
    u.write()
    out, lse = run_prefill(u)
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    compare(out, ref, fp8=kv != "bf16", lse_gpu=lse, lse_ref=ref_lse, what=f"prefill {case} {kv}")


@pytest.mark.parametrize("bs", [8, 64])
def test_block_sizes_and_batches(gpu_lib, bs):
    """Block size 8 takes the generic kernel, 64 the LDS-streamed one; several sequences,
    some queries in the tail of a longer context, one sequence shorter than a tile."""
    g = workloads.diffkv_geom(0, bs)
    w = workloads.paged_workload("pf", g, [700, 5, 333, 64], [100, 5, 333, 31], 32, 1 / math.sqrt(192),
                                 seed=43)
    u = Uploaded(w)
    u.write()
    out, lse = run_prefill(u)
    ref, ref_lse = oracle_attention(w, u.cache_bytes())
    compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"prefill bs={bs}")


def test_chunked_equals_one_shot(gpu_lib):
    """Prefill in 64-token chunks == one 256-token prefill (bitwise on the shared rows is
    not required: the key tiling differs only by where chunks end)."""
    g = workloads.diffkv_geom(0, 16)
    w = workloads.paged_workload("pf", g, [256], [256], 32, 1 / math.sqrt(192), seed=42)
    u = Uploaded(w)
    u.write()
    full, _ = run_prefill(u)
    for c in range(4):
        qsl = torch.tensor([0, 64], dtype=torch.int32, device=DEV)
        sl = torch.tensor([64 * (c + 1)], dtype=torch.int32, device=DEV)
        part, _ = pk.prefill_causal(u.q[64 * c: 64 * (c + 1)], qsl, sl, u.bt, u.desc, w.softmax_scale, 64)
        assert float((part.float() - full[64 * c: 64 * (c + 1)].float()).abs().max()) <= 4e-3


def test_chunked_prefill_config(gpu_lib):
    """32768 tokens written and attended in 8 chunks of 4096 (block size 16).  Checked rows: all
    4096 of chunk 0; in every chunk its first and last row, one random row of every 32-token
    query tile (the fast kernel's workgroup tile, so every tile rank of the XCD-aware mapping
    is sampled) and 256 more random rows."""
    log("prefill config: generating")
    w = workloads.prefill_chunks()
    u = Uploaded(w)
    C = w.extra["chunk"]
    T = w.q.shape[0]
    out = torch.empty(T, 32, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, 32, dtype=torch.float32, device=DEV)
    for c in range(T // C):
        sl = slice(c * C, (c + 1) * C)
        pk.cache_write(u.key[sl], u.value[sl], u.slots[sl], u.desc)
        qsl = torch.tensor([0, C], dtype=torch.int32, device=DEV)
        seq = torch.tensor([(c + 1) * C], dtype=torch.int32, device=DEV)
        pk.prefill_causal(u.q[sl], qsl, seq, u.bt, u.desc, w.softmax_scale, C, out=out[sl], out_lse=lse[sl])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    cache = u.cache_bytes()
    refs, ref_lses, rows = [], [], []
    for c in range(T // C):
        if c == 0:
            local = np.arange(C)
        else:
            local = np.unique(np.concatenate([[0, C - 1], np.arange(0, C, 32) + rng.integers(0, 32, C // 32),
                                              rng.choice(C, 256, replace=False)]))
        # the oracle on chunk c alone: its C queries at positions cC..cC+C-1 over keys 0..(c+1)C-1
        wc = copy.copy(w)
        wc.q = w.q[c * C: (c + 1) * C]
        wc.seq_lens = torch.tensor([(c + 1) * C], dtype=torch.int32)
        wc.query_start_loc = torch.tensor([0, C], dtype=torch.int32)
        log(f"oracle on {len(local)} rows of chunk {c}")
        r, rl = oracle_attention(wc, cache, rows=local)
        refs.append(r)
        ref_lses.append(rl)
        rows.append(c * C + local)
    rows = np.concatenate(rows)
    idx = torch.from_numpy(rows).to(DEV)
    compare(out[idx], np.concatenate(refs), lse_gpu=lse[idx], lse_ref=np.concatenate(ref_lses),
            what=f"chunked prefill 32768 ({len(rows)} rows)", strict=True)
