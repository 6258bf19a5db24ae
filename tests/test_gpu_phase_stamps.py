"""The phase-stamped diagnostics build of the split-KV partial kernels runs and gives a consistent
per-wave timeline (bench.py --phase-stamps, in a process of its own since it loads the
stamped twin of the library)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# tiles per wave: B8 512 keys per partition / 16-key tiles / 4 waves; MLA B1 448 keys per
# partition (7 per wave), the last partition 100000 - 223 x 448 = 96 keys (2, 2, 1, 1)
# fp8 verify: 46080 keys / 16 partitions = 2880 keys = 90 tiles of 32 keys over 4 waves (23, 23, 22, 22);
# MLA verify B1 (steps of two 32-key tiles): 448 keys = 7 steps, the last partition's 96 keys 2 steps
@pytest.mark.parametrize("name,tiles", [("decode_b8", [8]), ("mla_b1", [1, 2, 7]), ("fp8_verify", [22, 23]),
                                        ("mla_verify_b1", [2, 7])])
def test_phase_timeline(name, tiles):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--phase-stamps", name],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads([x for x in r.stdout.splitlines() if x.startswith("{")][-1])
    assert res["tiles_per_wave"] == tiles
    ph = res["us_from_first_entry"]
    # Q's landing and the prologue's issue come in either order (the kernel's choice); both
    # follow the entry and precede the first tile, the rest is in sequence
    pairs = [("entry", "prologue_issued"), ("entry", "q_landed"), ("prologue_issued", "first_tile_ready"),
             ("q_landed", "first_tile_ready"), ("first_tile_ready", "loop_end"), ("loop_end", "epilogue_barrier"),
             ("epilogue_barrier", "end")]
    for a, b in pairs:
        assert ph[a]["min"] <= ph[b]["min"] and ph[a]["max"] <= ph[b]["max"], (a, b, ph[a], ph[b])
    assert 0 < ph["end"]["max"] < 1000                 # one launch, in microseconds
    assert len(res["tiles"]) == max(tiles)
    assert res["tiles"][0]["waves"] == res["waves"]
    assert all(t["compute_us"]["min"] >= 0 and t["wait_us"]["min"] >= 0 for t in res["tiles"])
    assert len(res["end_us_by_xcc"]) == 8
