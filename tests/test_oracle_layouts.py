"""Pins of the oracle's stride handling: the cache write and attention read a slot's row of a
KV head at block*stride_block + pos*stride_slot + head*stride_head, whatever those strides
are.  The page tests the asymmetric write in both layouts the attention backend hands the
kernel (vLLM PR #64064, "Tests"): NHD [block][slot][head][row] and HND [block][head][slot][row];
padded row and block pitches stand for any other stride set.  Pins: the same logical
workload in every layout gives the same logical cache rows (read through torch's strided
views, not the oracle's offsets), leaves every padding element and the slack untouched, and
gives bit-identical attention outputs and log-sum-exps."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import paged_ref as R

LAYOUTS = [("NHD", 0, 0), ("HND", 0, 0), ("NHD", 64, 128), ("HND", 32, 80)]


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _build(kv, layout, row_pad, block_pad, scales):
    g = workloads.diffkv_geom(0, 16, kv_dtype=kv, layout=layout, row_pad=row_pad, block_pad=block_pad)
    return workloads.paged_workload("lay", g, [37, 100, 5], [1, 3, 2], 8, 1 / math.sqrt(192), seed=4,
                                    scale_mode=scales)


def _write(w):
    spec = R.CacheSpec.from_geom(w.geom)
    img = w.cache_init.numpy()
    if spec.kv_dtype == "bf16":
        img = img.view(np.uint16)
    return R.cache_write(img, spec, _bits(w.key), _bits(w.value), w.slot_mapping.numpy(), w.k_scale, w.v_scale)


def _rows(w, flat):
    t = torch.from_numpy(np.ascontiguousarray(flat))
    return w.geom.rows_view(t.view(torch.int16) if t.dtype == torch.uint16 else t).clone()


@pytest.mark.parametrize("kv,scales", [("bf16", "none"), ("fp8", "head")])
def test_layouts_hold_the_same_rows_and_results(kv, scales):
    ref_rows = ref_att = None
    for layout, row_pad, block_pad in LAYOUTS:
        w = _build(kv, layout, row_pad, block_pad, scales)
        out = _write(w)
        rows = _rows(w, out)
        # padding and slack: every element outside the rows keeps its initial value
        g = w.geom
        init = w.cache_init.numpy().view(out.dtype)
        covered = np.zeros(g.total_elems, dtype=bool)
        idx = g.rows_view(torch.arange(g.total_elems, dtype=torch.int64)).reshape(-1).numpy()
        covered[idx] = True
        assert np.array_equal(out[~covered], init[~covered]), f"{layout}: padding or slack changed"
        spec = R.CacheSpec.from_geom(g)
        qb = _bits(w.q)
        ks = w.k_scale.numpy() if w.k_scale is not None else None
        vs = w.v_scale.numpy() if w.v_scale is not None else None
        att = R.paged_attention(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(), out,
                                spec, w.softmax_scale, ks, vs)
        if ref_rows is None:
            ref_rows, ref_att = rows, att
            continue
        assert torch.equal(rows, ref_rows), f"{layout} pad {row_pad}/{block_pad}: rows differ from NHD"
        assert np.array_equal(att[0], ref_att[0]) and np.array_equal(att[1], ref_att[1]), f"{layout}: attention"


def test_hnd_strides_are_the_transposed_order():
    """HND puts a KV head's slots of one block next to each other: slot pos+1 of head h is
    one row pitch after slot pos, head h+1 is block_size row pitches after head h."""
    g = workloads.diffkv_geom(3, 16, layout="HND", row_pad=8)
    v = g.rows_view(torch.arange(g.total_elems, dtype=torch.int64))
    assert int(v[1, 5, 2, 0] - v[1, 4, 2, 0]) == 320 + 8
    assert int(v[1, 4, 3, 0] - v[1, 4, 2, 0]) == 16 * (320 + 8)
    assert int(v[2, 0, 0, 0] - v[1, 0, 0, 0]) == 4 * 16 * (320 + 8)
