"""Build ``libpagedattn.so`` in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``) and without fast-math, so
that fp32 division stays correctly rounded (the fp8 quantiser relies on it).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpagedattn.so")
# the same library with the decode, fp8-verify and MLA-verify kernels' per-wave phase stamps compiled in
# (diagnostics only: bench.py --phase-stamps loads it; the entry points' library never
# carries them)
STAMPS_LIB = os.path.join(HERE, "libpagedattn_stamps.so")
STAMPED_SOURCES = ("splitkv_dma.hip", "splitkv_wide.hip", "splitkv_tokens.hip")
# the matrix-core issue probe (a measurement tool, bench.py --mfma-probe), its own library
PROBE_LIB = os.path.join(HERE, "libmfma_probe.so")
PROBE_SOURCE = "mfma_probe.hip"
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "cache_write.hip", "splitkv.hip", "splitkv_dma.hip", "splitkv_wide.hip", "splitkv_tokens.hip",
           "prefill.hip"]
ARCH = os.environ.get("PAGEDATTN_ARCH", "gfx950")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + tag + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x and x.strip())
    if warn and os.environ.get("PAGEDATTN_VERBOSE"):
        print(warn, file=sys.stderr)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library (and its phase-stamped twin, and
    the matrix-core probe); returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = ([(src, (), "") for src in SOURCES] + [(src, ("-DPA_PHASE_STAMPS",), ".stamps") for src in STAMPED_SOURCES]
            + [(PROBE_SOURCE, (), "")])
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n, ns = len(SOURCES), len(STAMPED_SOURCES)
    _link(objs[:n], LIB)
    stamped_obj = dict(zip(STAMPED_SOURCES, objs[n:n + ns]))
    _link([stamped_obj.get(src, o) for src, o in zip(SOURCES, objs)], STAMPS_LIB)
    _link(objs[n + ns:], PROBE_LIB)
    if verbose:
        print(f"built {LIB}, {os.path.basename(STAMPS_LIB)} and {os.path.basename(PROBE_LIB)}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
