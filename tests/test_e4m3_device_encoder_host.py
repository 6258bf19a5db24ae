"""The library's E4M3FN encoder (the one the fp8 cache write and the fused decode write run on the
GPU) checked on EVERY binary32 bit pattern against the oracle's encoder: the function is built for
the host from the same source (tests/native/e4m3_host.hip includes the kernels' common header), so
all 2^32 inputs -- normals, subnormals, ties, the saturation edge, infinities and every NaN payload --
run in a few tens of seconds on the CPU.  The oracle's encoder (a nearest-value search over the
format's codes) is itself pinned against torch's fp8 cast in test_oracle_e4m3fn.py.  The pages ask
for an fp8 E4M3 KV cache with per-tensor and per-head scales (vLLM PR #64064, "Tests"); the device
division fp32(x)/fp32(scale) ahead of the encoder is covered on the GPU (every bf16 pattern x 5
scales in test_gpu_cache_write.py)."""
import ctypes
import multiprocessing as mp
import os
import subprocess

import numpy as np
import pytest

from oracle import e4m3fn

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "e4m3_host.hip")
LIB = os.path.join(HERE, "native", "libe4m3host.so")
CHUNK = 1 << 24


def build_host_lib() -> str:
    """Compile the host build of the encoder (also done by __graft_entry__.build())."""
    hipcc = "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "-O2", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-x", "hip", SRC, "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {LIB} failed:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _lib():
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(SRC), os.path.getmtime(
            os.path.join(HERE, "..", "paged_kv_cache_176_amd", "csrc", "common.hpp"))):
        build_host_lib()
    lib = ctypes.CDLL(LIB)
    lib.e4m3fn_encode_patterns.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    return lib


def _check_range(first: int, n_chunks: int):
    """Compare the two encoders on patterns [first, first + n_chunks*CHUNK); returns mismatches."""
    lib = _lib()
    out = np.empty(CHUNK, dtype=np.uint8)
    bad = []
    for c in range(n_chunks):
        base = first + c * CHUNK
        lib.e4m3fn_encode_patterns(base, CHUNK, out.ctypes.data)
        pats = np.arange(base, base + CHUNK, dtype=np.uint64).astype(np.uint32)
        with np.errstate(invalid="ignore", over="ignore"):
            ref = e4m3fn.encode(pats.view(np.float32))
        diff = np.nonzero(out != ref)[0]
        bad += [(int(pats[i]), int(out[i]), int(ref[i])) for i in diff[:8]]
    return bad


def test_host_build_matches_on_landmarks():
    """A few patterns whose codes are fixed by the format: 448 and beyond saturate, 480 too, the
    smallest subnormal 2^-9 and half of it (a tie to 0), 1.5 x 2^-9 (a tie to 2 x 2^-9), 1.0, NaN -> 0x7F, -0 -> 0x80."""
    lib = _lib()
    vals = np.array([448.0, 480.0, 1e30, np.inf, 2.0 ** -9, 2.0 ** -10, 1.0, -1.0, -0.0, np.nan, 3 * 2.0 ** -10],
                    dtype=np.float32)
    pats = vals.view(np.uint32)
    got = []
    out = np.empty(1, dtype=np.uint8)
    for p in pats:
        lib.e4m3fn_encode_patterns(int(p), 1, out.ctypes.data)
        got.append(int(out[0]))
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x01, 0x00, 0x38, 0xB8, 0x80, 0x7F, 0x02]


def test_every_fp32_pattern():
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    total = (1 << 32) // CHUNK
    per = -(-total // workers)
    jobs = [(w * per * CHUNK, min(per, total - w * per)) for w in range(workers) if w * per < total]
    _lib()                                          # build once before forking
    with mp.get_context("fork").Pool(len(jobs)) as pool:
        results = pool.starmap(_check_range, jobs)
    bad = [x for r in results for x in r]
    assert not bad, "device encoder != oracle for (pattern, device, oracle): " + ", ".join(
        f"(0x{p:08x}, 0x{d:02x}, 0x{o:02x})" for p, d, o in bad[:16])
