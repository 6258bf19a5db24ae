"""Pins of the oracle's cache write (vLLM PR #64064, sections "Tests" and "Details").

The write must put K in the first head_dim columns of each slot's row and V in
its own head_dim_v columns at V's own offset, leave every other byte alone
(including slack past the cache end), skip slot -1, and for fp8 caches store
E4M3FN(fp32(x) / fp32(scale)) per tensor or per KV head.  The checks index the
cache through torch views (not the oracle's offset arithmetic) and compare fp8
codes with torch's own float8_e4m3fn cast.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import e4m3fn
from oracle import paged_ref as R


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _write(w, value=True, slots=None, planted=None):
    spec = R.CacheSpec.from_geom(w.geom)
    img = w.cache_init.numpy()
    if spec.kv_dtype == "bf16":
        img = img.view(np.uint16)
    fn = R.cache_write if planted is None else planted
    return fn(img, spec, _bits(w.key), _bits(w.value) if (value and w.value is not None) else None,
              (w.slot_mapping if slots is None else slots).numpy(), w.k_scale, w.v_scale)


def _view(w, flat):
    g = w.geom
    return torch.from_numpy(np.ascontiguousarray(flat[: g.cache_elems])).view(
        g.num_blocks, g.block_size, g.num_kv_heads, g.row_dim)


@pytest.mark.parametrize("bs", [16, 64])
def test_bf16_rows_hold_k_then_v_and_nothing_else_changes(bs):
    g = workloads.diffkv_geom(0, bs)
    w = workloads.paged_workload("cw", g, [37, 100, 5], [37, 100, 5], 8, 0.1, seed=2)
    out = _write(w)
    view = _view(w, out.view(np.int16))
    init = _view(w, w.cache_init.numpy())
    touched = torch.zeros_like(init, dtype=torch.bool)
    for t, s in enumerate(w.slot_mapping.tolist()):
        blk, pos = divmod(s, bs)
        assert torch.equal(view[blk, pos, :, :192], w.key[t].view(torch.int16))
        assert torch.equal(view[blk, pos, :, 192:320], w.value[t].view(torch.int16))
        touched[blk, pos] = True
    assert torch.equal(view[~touched], init[~touched])
    slack = out.view(np.int16)[g.cache_elems:]
    assert np.array_equal(slack, w.cache_init.numpy()[g.cache_elems:])


def test_skipped_slots_and_missing_value():
    g = workloads.diffkv_geom(0, 16)
    w = workloads.paged_workload("cw", g, [40], [40], 8, 0.1, seed=4)
    slots = w.slot_mapping.clone()
    slots[::3] = -1
    out = _write(w, slots=slots)
    view, init = _view(w, out.view(np.int16)), _view(w, w.cache_init.numpy())
    for t, s in enumerate(w.slot_mapping.tolist()):
        blk, pos = divmod(s, 16)
        if t % 3 == 0:
            assert torch.equal(view[blk, pos], init[blk, pos])
        else:
            assert torch.equal(view[blk, pos, :, :192], w.key[t].view(torch.int16))
    # value omitted (MLA-style latent row): only the K columns are written
    out = _write(w, value=False)
    view = _view(w, out.view(np.int16))
    for t, s in enumerate(w.slot_mapping.tolist()):
        blk, pos = divmod(s, 16)
        assert torch.equal(view[blk, pos, :, 192:], init[blk, pos, :, 192:])


@pytest.mark.parametrize("mode", ["tensor", "head"])
def test_fp8_codes_are_torch_cast_of_fp32_quotient(mode):
    g = workloads.diffkv_geom(0, 16, kv_dtype="fp8")
    w = workloads.paged_workload("cw8", g, [33, 64], [33, 64], 8, 0.1, seed=5, scale_mode=mode)
    out = _write(w)
    view = _view(w, out)
    ks = w.k_scale.expand(4) if mode == "tensor" else w.k_scale
    vs = w.v_scale.expand(4) if mode == "tensor" else w.v_scale
    k32, v32 = w.key.to(torch.float32), w.value.to(torch.float32)
    for t, s in enumerate(w.slot_mapping.tolist()):
        blk, pos = divmod(s, 16)
        qk = k32[t] / ks[:, None]
        qv = v32[t] / vs[:, None]
        assert float(qk.abs().max()) < 448 and float(qv.abs().max()) < 448
        assert torch.equal(view[blk, pos, :, :192], qk.to(torch.float8_e4m3fn).view(torch.uint8))
        assert torch.equal(view[blk, pos, :, 192:], qv.to(torch.float8_e4m3fn).view(torch.uint8))


def test_fp8_saturates_large_values_keeping_sign():
    g = workloads.diffkv_geom(0, 16, kv_dtype="fp8")
    w = workloads.paged_workload("cw8", g, [4], [4], 8, 0.1, seed=6, scale_mode="tensor")
    w.key = (w.key.to(torch.float32) * 1000).to(torch.bfloat16)
    out = _view(w, _write(w))
    q = w.key.to(torch.float32) / w.k_scale
    for t, s in enumerate(w.slot_mapping.tolist()):
        blk, pos = divmod(s, 16)
        codes = out[blk, pos, :, :192]
        big = q[t].abs() >= 448
        assert big.any()
        assert torch.all(codes[big] & 0x7F == 0x7E)
        assert torch.equal((codes[big] & 0x80) != 0, q[t][big] < 0)


def test_planted_symmetric_write_bug_is_caught():
    """The bug the page describes: V addressed with K's offset and copied at K's width.

    A write that reuses K's per-head offset and element count for V overruns into the
    next head and, on the last slot, past the cache; the pins above must catch it.
    """
    def buggy(cache_flat, spec, key_bits, value_bits, slot_mapping, k_scale=None, v_scale=None):
        out = np.array(cache_flat, copy=True)
        for t, s in enumerate(slot_mapping):
            for h in range(spec.num_kv_heads):
                base = R.CacheSpec.row_offset(spec, int(s), h)
                out[base: base + spec.dk] = key_bits[t, h, : spec.dk]
                vsrc = np.asarray(value_bits).reshape(len(slot_mapping), -1)[t, h * spec.dk: h * spec.dk + spec.dk]
                n = min(spec.dk, len(out) - (base + spec.v_off))
                out[base + spec.v_off: base + spec.v_off + n] = np.resize(vsrc, n)
        return out

    g = workloads.diffkv_geom(0, 16)
    w = workloads.paged_workload("cw", g, [37], [37], 8, 0.1, seed=2)
    good = _write(w)
    bad = _write(w, planted=buggy)
    assert not np.array_equal(good, bad)
    gv, bv = _view(w, good.view(np.int16)), _view(w, bad.view(np.int16))
    t, s = 3, int(w.slot_mapping[3])
    blk, pos = divmod(s, 16)
    assert torch.equal(gv[blk, pos, :, 192:], w.value[t].view(torch.int16))
    assert not torch.equal(bv[blk, pos, :, 192:], w.value[t].view(torch.int16))


def test_workload_generators_are_deterministic():
    a, b = workloads.tiny(), workloads.tiny()
    for x, y in [(a.q, b.q), (a.key, b.key), (a.value, b.value), (a.block_tables, b.block_tables),
                 (a.slot_mapping, b.slot_mapping), (a.cache_init, b.cache_init)]:
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
    assert a.block_tables.shape == (2, 7) and sorted(a.block_tables[a.block_tables != 15].tolist()) == \
        sorted(set(a.block_tables[a.block_tables != 15].tolist()))
