"""Randomised GPU parity sweep: seeded small cases over the shape space each entry point
serves -- cache dtype and scale granularity, block size (powers of two and not), batch,
ragged and empty sequences, GQA ratio, query tokens per sequence, split count, cache layout
(NHD, HND, padded pitches), sink logits and a split policy, and the MLA decode and verify
over random shapes -- each against the oracle on the same cache bytes.  The seeds are
fixed; a failing case prints its parameters.  Kernel selection differs across these shapes
(LDS-streamed, 32-row wide, MLA token and register-prefetch split-KV kernels; fast and
generic prefill), so the sweep crosses paths the hand-picked tests visit one at a time."""
import math
import random

import pytest
import torch

import numpy as np

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, split_last_keys
from oracle import paged_ref as R

pytestmark = pytest.mark.gpu

BLOCK_SIZES = (8, 16, 24, 32, 64)


def draw_common(rng):
    kv = rng.choice(["bf16", "bf16", "fp8"])
    scales = "none" if kv == "bf16" else rng.choice(["tensor", "head"])
    bs = rng.choice(BLOCK_SIZES)
    hkv = rng.choice([1, 2, 4])
    return kv, scales, bs, hkv


def draw_extras(rng, hq, kv):
    """Cache layout, sink logits (or none) and a split policy (or none)."""
    layout = rng.choice(["NHD", "NHD", "HND"])
    pad = rng.choice([0, 0, 16 if kv == "fp8" else 8, 64])
    sinks = None
    if rng.random() < 0.35:
        sinks = torch.tensor([rng.uniform(-4, 4) if rng.random() < 0.8 else -math.inf for _ in range(hq)],
                             dtype=torch.float32)
    policy = None
    if rng.random() < 0.35:
        policy = [(64, 1), (400, rng.randint(1, 4)), (1 << 30, rng.randint(2, 40))]
    return layout, pad, sinks, policy


def oracle(w, u, sinks):
    qb = w.q.view(torch.int16).numpy().view(np.uint16)
    ks = w.k_scale.numpy() if w.k_scale is not None else None
    vs = w.v_scale.numpy() if w.v_scale is not None else None
    return R.paged_attention(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(),
                             u.cache_bytes(), R.CacheSpec.from_geom(w.geom), w.softmax_scale, ks, vs,
                             sinks=None if sinks is None else sinks.double().numpy())


@pytest.mark.parametrize("seed", range(48))
def test_random_split_kv(gpu_lib, seed):
    rng = random.Random(1000 + seed)
    kv, scales, bs, hkv = draw_common(rng)
    G = rng.choice([1, 2, 4, 8, 12, 16])
    verify = rng.random() < 0.5
    max_l = max(1, min(8, 64 // G)) if verify else 1
    B = rng.randint(1, 5)
    qlens = [rng.randint(1, max_l) for _ in range(B)]
    lens = [0 if rng.random() < 0.15 else rng.randint(L, 600) for L in qlens]
    qlens = [L if s else 1 for s, L in zip(lens, qlens)]        # an empty sequence keeps one query row
    P = rng.choice([1, 2, 3, 7, 16, 33])
    what = (f"seed {seed}: {'verify' if verify else 'decode'} {kv}/{scales} bs {bs} Hkv {hkv} G {G} "
            f"lens {lens} L {qlens} P {P}")
    append = not verify and rng.random() < 0.5     # the decode step's write inside the decode call
    what += " (append)" if append else ""
    layout, pad, sinks, policy = draw_extras(rng, hkv * G, kv)
    what += f" {layout} pad {pad}" + (" sinks" if sinks is not None else "") + (f" policy {policy}" if policy else "")
    log(what)
    g = workloads.diffkv_geom(0, bs, kv_dtype=kv, num_kv_heads=hkv, layout=layout, row_pad=pad)
    w = workloads.paged_workload("rand", g, lens, qlens, hkv * G, 1 / math.sqrt(192), seed=seed,
                                 scale_mode=scales)
    u = Uploaded(w)
    skd = None if sinks is None else sinks.to(DEV)
    if append:
        setup, (key, value, slots) = split_last_keys(w, u)
        pk.cache_write(*setup, u.desc)
        out, lse, _ = pk.decode_splitkv_append(u.q, key, value, slots, u.desc, u.bt, u.seq_lens, w.softmax_scale,
                                               P, sinks=skd, split_policy=policy)
        torch.cuda.synchronize()
    else:
        u.write()
        if verify:
            out, lse, _ = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P,
                                    sinks=skd, split_policy=policy)
        else:
            out, lse, _ = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, sinks=skd,
                                            split_policy=policy)
    ref, ref_lse = oracle(w, u, sinks)
    compare(out, ref, fp8=kv == "fp8", lse_gpu=lse, lse_ref=ref_lse, what=what)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(gpu_lib, seed):
    rng = random.Random(2000 + seed)
    kv, scales, bs, hkv = draw_common(rng)
    G = rng.choice([1, 2, 4, 8, 16])
    B = rng.randint(1, 3)
    qlens = [rng.randint(1, 200) for _ in range(B)]
    lens = [L + rng.choice([0, 0, rng.randint(1, 300)]) for L in qlens]   # some chunks follow a context
    layout, pad, sinks, _ = draw_extras(rng, hkv * G, kv)
    what = (f"seed {seed}: prefill {kv}/{scales} bs {bs} Hkv {hkv} G {G} lens {lens} L {qlens} {layout} pad {pad}"
            + (" sinks" if sinks is not None else ""))
    log(what)
    g = workloads.diffkv_geom(0, bs, kv_dtype=kv, num_kv_heads=hkv, layout=layout, row_pad=pad)
    w = workloads.paged_workload("randpf", g, lens, qlens, hkv * G, 1 / math.sqrt(192), seed=seed,
                                 scale_mode=scales)
    u = Uploaded(w)
    u.write()
    ref, ref_lse = oracle(w, u, sinks)
    out, lse = pk.prefill_causal(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len,
                                 sinks=None if sinks is None else sinks.to(DEV))
    compare(out, ref, fp8=kv == "fp8", lse_gpu=lse, lse_ref=ref_lse, what=what)


@pytest.mark.parametrize("seed", range(24))
def test_random_mla(gpu_lib, seed):
    """MLA decode and multi-token verify (one 576-wide latent KV head, V = its first 512 columns)
    over random batches, lengths, query-head counts, draft lengths, block sizes, split counts,
    layouts and sink logits; half the cases with queries 80x larger than the latent rows, so
    the scores are peaked and a wrong causal limit or merge weight shows."""
    rng = random.Random(5000 + seed)
    bs = rng.choice([16, 32, 64])
    G = rng.choice([8, 12, 12, 16])
    B = rng.randint(1, 5)
    verify = rng.random() < 0.6
    qlens = [rng.randint(2, 8) if verify else 1 for _ in range(B)]
    lens = [0 if rng.random() < 0.1 else rng.randint(L, 3000) for L in qlens]
    qlens = [L if s else 1 for s, L in zip(lens, qlens)]
    P = rng.choice([1, 2, 5, 16, 33, 64])
    layout = rng.choice(["NHD", "NHD", "HND"])
    pad = rng.choice([0, 0, 8, 64])
    peaked = rng.random() < 0.5
    sinks = None
    if rng.random() < 0.3:
        sinks = torch.tensor([rng.uniform(-4, 4) for _ in range(G)], dtype=torch.float32)
    what = (f"seed {seed}: MLA {'verify' if verify else 'decode'} bs {bs} G {G} lens {lens} L {qlens} P {P} "
            f"{layout} pad {pad}" + (" peaked" if peaked else "") + (" sinks" if sinks is not None else ""))
    log(what)
    g = workloads.mla_geom(0, bs, layout=layout, row_pad=pad)
    w = workloads.paged_workload("mla_rand", g, lens, qlens, G, 1 / math.sqrt(576), seed=seed, std=0.1,
                                 q_std=8.0 if peaked else None)
    u = Uploaded(w)
    u.write()
    skd = None if sinks is None else sinks.to(DEV)
    if verify:
        out, lse, _ = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P, sinks=skd)
    else:
        out, lse, _ = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P, sinks=skd)
    ref, ref_lse = oracle(w, u, sinks)
    compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=what)
