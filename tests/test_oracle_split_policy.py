"""Pins of the oracle's split policy (vLLM PR #50371, review thread: each sequence's active
split count comes from its runtime length by context buckets -- a 100K context selecting 96
splits -- with one table shared by the partial and merge stages).
  * the bucket lookup at and around every bound, the last bucket for longer contexts, and
    the cap at the launch's partition count;
  * partitions past a sequence's active count are empty;
  * whatever the policy, the merged partials equal the unsplit attention."""
import math

import numpy as np
import torch

import workloads
from oracle import paged_ref as R

POLICY = [(512, 2), (4096, 8), (65536, 32), (131072, 96)]


def test_bucket_lookup():
    f = lambda s, P=128: R.active_splits(s, P, POLICY)
    assert [f(0), f(1), f(512), f(513), f(4096), f(4097), f(65536), f(65537), f(100000), f(10 ** 6)] == \
        [2, 2, 2, 8, 8, 32, 32, 96, 96, 96]
    assert f(100000, P=64) == 64 and f(100, P=1) == 1
    assert R.active_splits(100000, 48, None) == 48


def test_policy_partials_merge_to_the_whole():
    g = workloads.diffkv_geom(0, 16)
    lens = [30, 700, 5000, 0]
    w = workloads.paged_workload("pol", g, lens, [1, 1, 1, 1], 8, 1 / math.sqrt(192), seed=21)
    spec = R.CacheSpec.from_geom(g)
    cache = R.cache_write(w.cache_init.numpy().view(np.uint16), spec, w.key.view(torch.int16).numpy().view(np.uint16),
                          w.value.view(torch.int16).numpy().view(np.uint16), w.slot_mapping.numpy())
    q = w.q.view(torch.int16).numpy().view(np.uint16)
    args = (q, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(), cache, spec, w.softmax_scale)
    full, full_lse = R.paged_attention(*args)
    P = 40
    po, pl = R.paged_attention_partials(*args, P, policy=POLICY)
    for b, S in enumerate(lens):
        k = R.active_splits(S, P, POLICY)
        assert np.all(pl[b, :, k:] == -np.inf) and np.all(po[b, :, k:] == 0), f"seq {b}: past the active splits"
        for p, (lo, hi) in enumerate(R.partition_ranges(S, k, 16)):
            assert np.all(np.isfinite(pl[b, :, p])) == (hi > lo), f"seq {b} split {p}"
    mo, ml = R.merge_lse(po, pl)
    np.testing.assert_allclose(mo, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, full_lse, rtol=1e-12, atol=1e-12)
