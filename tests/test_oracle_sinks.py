"""Pins of the oracle's attention sink: a per-query-head logit that joins the softmax
denominator as one more term with no value (diffbot model card, "Update 2026-10-01: three
correctness fixes", the item on the vision encoder's sink, read as an extra
softmax-denominator logit).
  * a -inf sink is no sink, bit for bit;
  * one visible key k against a sink c is a two-way softmax: out = v * sigmoid(s - c) and
    lse = logaddexp(s, c), with s = scale * q.k computed here from the bf16 values;
  * a row that sees no key outputs 0 with lse = c;
  * split-KV partials merged with the sink equal the unsplit attention with the sink."""
import math

import numpy as np
import torch

import workloads
from oracle import paged_ref as R


def _att(w, sinks=None, rows=None):
    spec = R.CacheSpec.from_geom(w.geom)
    img = w.cache_init.numpy().view(np.uint16)
    cache = R.cache_write(img, spec, w.key.view(torch.int16).numpy().view(np.uint16),
                          w.value.view(torch.int16).numpy().view(np.uint16), w.slot_mapping.numpy())
    q = w.q.view(torch.int16).numpy().view(np.uint16)
    return cache, q, R.paged_attention(q, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(),
                                       cache, spec, w.softmax_scale, rows=rows, sinks=sinks)


def _work(lens, qlens, seed):
    g = workloads.diffkv_geom(0, 16)
    return workloads.paged_workload("sink", g, lens, qlens, 8, 1 / math.sqrt(192), seed=seed)


def test_minus_inf_sink_is_no_sink():
    w = _work([37, 100, 0], [1, 4, 1], 11)
    _, _, (o0, l0) = _att(w)
    _, _, (o1, l1) = _att(w, sinks=np.full(8, -np.inf))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_one_key_is_a_two_way_softmax():
    w = _work([1], [1], 12)
    c = np.linspace(-3.0, 2.5, 8)                   # one sink per query head
    _, _, (out, lse) = _att(w, sinks=c)
    q = w.q[0].float().double().numpy()             # [8, 192]
    k = w.key[0].float().double().numpy()           # [4, 192]
    v = w.value[0].float().double().numpy()         # [4, 128]
    for h in range(8):
        s = w.softmax_scale * float(q[h] @ k[h // 2])
        sig = 1.0 / (1.0 + math.exp(c[h] - s))
        np.testing.assert_allclose(out[0, h], v[h // 2] * sig, rtol=1e-12, atol=1e-15)
        assert abs(lse[0, h] - np.logaddexp(s, c[h])) < 1e-12


def test_row_without_keys_gives_the_sink():
    w = _work([0, 20], [1, 1], 13)
    c = np.arange(8, dtype=np.float64) - 4.0
    _, _, (out, lse) = _att(w, sinks=c)
    assert np.all(out[0] == 0) and np.array_equal(lse[0], c)
    assert np.all(np.isfinite(out[1])) and np.all(lse[1] > c)    # the real keys only add to the denominator


def test_merged_partials_with_sink_equal_the_whole():
    w = _work([300, 45, 7], [1, 3, 2], 14)
    c = np.array([0.5, -1.0, 2.0, -np.inf, 0.0, 1.5, -2.5, 3.0])
    cache, q, (out, lse) = _att(w, sinks=c)
    spec = R.CacheSpec.from_geom(w.geom)
    po, pl = R.paged_attention_partials(q, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(),
                                        cache, spec, w.softmax_scale, 5)
    mo, ml = R.merge_lse(po, pl, sinks=c)
    np.testing.assert_allclose(mo, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=1e-12, atol=1e-12)
