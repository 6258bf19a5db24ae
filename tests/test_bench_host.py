"""Host-side logic of bench.py (no GPU): the split counts it launches the measured workloads
with and the partition sizes the kernels cut from them (ceil(S / P) rounded up to 16 keys);
where a workgroup's 4 waves would otherwise hold few tiles each, that size is a whole number of
64-key rounds, so every wave gets the same count of 16-key tiles; at any size the split count
leaves no partition empty; and the one-GPU refusal."""
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("args,kw,P,chunk", [
    ((1, 4, 131072), dict(wgs_per_cu=2), 128, 1024),   # decode B1: two resident workgroups per CU
    ((8, 4, 8192), dict(wgs_per_cu=2), 16, 512),       # decode B8
    ((1, 1, 100000), {}, 224, 448),                    # MLA B1: 7 tiles for every wave
    ((16, 1, 100000), {}, 16, 6256),                   # MLA B16: 391 tiles, waves hold 98 or 97
    ((4, 4, 46080), {}, 16, 2880),                     # fp8 verify: one working workgroup per CU
])
def test_auto_partitions(args, kw, P, chunk):
    assert bench.auto_partitions(*args, **kw) == P
    assert math.ceil(math.ceil(args[2] / P) / 16) * 16 == chunk


@pytest.mark.parametrize("ctx", [1, 63, 64, 1000, 8192, 46080, 100000, 131072, 10 ** 6])
@pytest.mark.parametrize("batch,heads,wpc", [(1, 1, 1), (1, 4, 2), (8, 4, 2), (16, 1, 1), (64, 8, 1)])
def test_no_partition_is_empty(ctx, batch, heads, wpc):
    P = bench.auto_partitions(batch, heads, ctx, wgs_per_cu=wpc)
    assert 1 <= P <= 4096
    chunk = math.ceil(math.ceil(ctx / P) / 16) * 16
    assert (P - 1) * chunk < ctx <= P * chunk                 # every partition has keys, all keys covered


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_spinup_flag_is_accepted():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 0 and "--spinup-ms" in r.stdout


def test_parse_clocks_reads_every_xcd_and_the_memory_clock():
    import json
    import bench
    doc = {"gpu_data": [{"gpu": 0, "clock": {
        **{f"gfx_{i}": {"clk": {"value": 2100 + i, "unit": "MHz"}, "max_clk": {"value": 2400, "unit": "MHz"}}
           for i in range(8)},
        "mem_0": {"clk": {"value": 2000, "unit": "MHz"}}, "vclk_0": {"clk": {"value": 29, "unit": "MHz"}}}}]}
    c = bench.parse_clocks(json.dumps(doc))
    assert c["gfx_mhz_per_xcd"] == [2100 + i for i in range(8)] and c["mem_mhz"] == 2000
    assert c["gfx_mhz_mean"] == 2103.5
    assert bench.parse_clocks(None) is None and bench.parse_clocks("not json") is None


def test_oracle_timing_helpers_on_the_tiny_workload():
    import bench
    import workloads
    w = workloads.tiny()
    sec, n = bench.oracle_seconds(w, 0.01, with_write=True)
    assert sec > 0 and n >= 1
    line = bench.cpu_line(sec, n, 1e9, "GB/s", "tiny", scale=2.0)
    assert line["s_per_call"] == round(2 * sec, 3) and line["unit"] == "GB/s"
    info = bench.host_info()
    assert info["affinity_cores"] >= 1 and info["blas_threads"] >= 1
    p = bench.pcts([1e-6, 2e-6, 3e-6])
    assert p["p50"] == 2.0 and p["p10"] < p["p50"] < p["p90"]
