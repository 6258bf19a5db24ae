"""Host-side pins of the binding (no GPU): the byte extent a cache descriptor's strides address
(the bound the binding checks the storage tensor against) is exactly one past the last element of
the last row, read through torch's strided view of the rows, for NHD, HND and padded pitches, bf16
and fp8, DiffKV and MLA rows."""
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads


@pytest.mark.parametrize("geom", [
    lambda: workloads.diffkv_geom(6, 16),
    lambda: workloads.diffkv_geom(6, 16, layout="HND"),
    lambda: workloads.diffkv_geom(5, 32, layout="NHD", row_pad=64, block_pad=128),
    lambda: workloads.diffkv_geom(5, 16, layout="HND", row_pad=32, block_pad=80),
    lambda: workloads.diffkv_geom(4, 16, kv_dtype="fp8", layout="HND", row_pad=16),
    lambda: workloads.mla_geom(3, 64, layout="HND", row_pad=64),
    lambda: workloads.mla_geom(3, 64, block_pad=256),
])
def test_extent_is_one_past_the_last_row_element(geom):
    g = geom()
    esize = 1 if g.kv_dtype == "fp8" else 2
    d = pk.CacheDesc.from_geom(torch.empty(g.total_elems, dtype=torch.uint8 if esize == 1 else torch.int16), g)
    last = int(g.rows_view(torch.arange(g.total_elems, dtype=torch.int64)).max())
    assert d.extent_bytes() == (last + 1) * esize
    assert d.extent_bytes() <= g.total_elems * esize          # the geometry's storage covers it (slack past it)


def test_assigning_a_field_drops_the_checked_descriptor():
    g = workloads.diffkv_geom(2, 16)
    d = pk.CacheDesc.from_geom(torch.empty(g.total_elems, dtype=torch.int16), g)
    object.__setattr__(d, "_c", "built")
    d.num_blocks = 1
    assert d._c is None
