"""The matrix-core issue probe (libmfma_probe.so, `bench.py --mfma-probe`) runs on the GPU and
gives the figures its table is read for: a v_mfma_f32_32x32x16_bf16 occupies a SIMD's matrix
core ~32 cycles, and a single dependent accumulation chain issues slower than independent ones.
The bounds are loose (cycle counts, not a clock): they only catch a probe that measures nothing."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe(gpu_lib):
    from paged_kv_cache_176_amd import build as pkb
    if not os.path.exists(pkb.PROBE_LIB):
        pytest.fail("libmfma_probe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(pkb.PROBE_LIB)
    lib.mfma_probe_label.restype = ctypes.c_char_p
    lib.mfma_probe_run.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    return lib


def run(lib, label):
    for i in range(lib.mfma_probe_count()):
        if lib.mfma_probe_label(i).decode() == label:
            res = (ctypes.c_double * 3)()
            assert lib.mfma_probe_run(i, res) == 0
            return res[0], res[1]
    raise AssertionError(f"no probe configuration {label!r}")


def test_mfma_issue_rates(probe):
    dep, _ = run(probe, "1 wave/SIMD: 1 dependent chain")
    two, _ = run(probe, "1 wave/SIMD: 2 independent chains")
    pair, _ = run(probe, "2 waves/SIMD: 1 dependent chain each")
    print(f"cycles per MFMA per SIMD: dependent chain {dep:.1f}, two chains {two:.1f}, two waves {pair:.1f}")
    assert 28.0 <= two <= 48.0 and 28.0 <= pair <= 48.0
    assert dep > 1.2 * two


def test_split_roles_report_both_waves(probe):
    m, v = run(probe, "MFMA-only wave beside a wave of 6 FMA + 2 exp2 per MFMA")
    print(f"MFMA wave {m:.1f} cycles per MFMA, VALU wave {v:.2f} cycles per instruction")
    assert 28.0 <= m <= 80.0 and 1.0 <= v <= 40.0
