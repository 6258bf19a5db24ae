"""The LDS ring layouts against the bank rule measured on gfx950 (64 banks of 4 bytes; a 64-bit read
served 32 lanes at a time): every transposing V^T read of the bf16 decode, MLA, MLA-verify and prefill
kernels must cover the 64 banks exactly once per 32-lane half.  The swizzles are the kernels' own
(lds_layout.hpp built for the host); the lane patterns restate each kernel's V^T operand addressing.
The same rule flags the layouts the kernels used before (2-way), which the bank-conflict counter had
measured at 25-32% of LDS cycles.  128-bit K-operand reads follow no rule this simple: their layouts
are covered by the kernels' measured counters instead (0.0-0.1% conflict cycles in the profiles)."""
import ctypes
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "lds_layout_host.hip")
HDR = os.path.join(HERE, "..", "paged_kv_cache_176_amd", "csrc", "lds_layout.hpp")
LIB = os.path.join(HERE, "native", "libldslayouthost.so")


def _lib():
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(SRC), os.path.getmtime(HDR)):
        cmd = ["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-x", "hip",
               SRC, "-o", LIB + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"building {LIB} failed:\n{r.stderr}")
        os.replace(LIB + ".tmp", LIB)
    lib = ctypes.CDLL(LIB)
    for n in ("host_row_chunk_swz", "host_fp8_chunk_swz", "host_prefill_k_swz", "host_prefill_v_swz"):
        getattr(lib, n).argtypes = [ctypes.c_int]
    return lib


def ways_64bit(addrs):
    """Largest number of distinct dwords that share a bank within one 32-lane half (1 = no conflict)."""
    worst = 1
    for half in (addrs[:32], addrs[32:]):
        banks = {}
        for a in half:
            for dw in (a // 4, a // 4 + 1):
                banks.setdefault(dw % 64, set()).add(dw)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


def vt_row_pattern(swz, pitch, v_chunk0, d4, key0):
    """The bf16 decode / MLA / MLA-verify V^T read: lane (n, g) = (lane & 15, lane >> 4) reads 8 bytes of
    key key0 + 4g + n/4, dims 16 d4 + 4 (n & 3) of V (V starts at chunk v_chunk0 of the row)."""
    out = []
    for lane in range(64):
        n, g = lane & 15, lane >> 4
        key = key0 + 4 * g + (n >> 2)
        ch = v_chunk0 + 2 * d4 + ((n & 3) >> 1)
        out.append(key * pitch + ((ch & ~7) | ((ch & 7) ^ swz(key))) * 16 + (n & 1) * 8)
    return out


def vt_prefill_pattern(swz, db, key0):
    """Prefill's V^T read over its 256-byte V rows: lane (s16, half, g) = (lane & 15, lane >> 4 & 1,
    lane >> 5) reads 8 bytes of key key0 + 4g + s16/4, dims 32 db + 16 half + 4 (s16 & 3)."""
    out = []
    for lane in range(64):
        s16, half, g = lane & 15, (lane >> 4) & 1, lane >> 5
        key = key0 + 4 * g + (s16 >> 2)
        dim = 32 * db + 16 * half + 4 * (s16 & 3)
        out.append((key * 16 + ((dim >> 3) ^ swz(key))) * 16 + (dim & 7) * 2)
    return out


def old_row(key):  # the row swizzle the kernels used before
    return ((key >> 1) ^ (key << 2)) & 7


def old_prefill_v(key):
    return (key & 7) << 1


@pytest.mark.parametrize("pitch,v_chunk0,n_d4", [(640, 24, 8), (1152, 0, 32)])
def test_bf16_row_vt_reads_conflict_free(pitch, v_chunk0, n_d4):
    """DiffKV rows (640 B, V = chunks 24..39) and MLA rows (1152 B, V = chunks 0..63): every 16-dim block of
    V, both 16-key halves of a 32-key tile (the MLA verify kernel reads both)."""
    swz = _lib().host_row_chunk_swz
    for d4 in range(n_d4):
        for key0 in (0, 16):
            assert ways_64bit(vt_row_pattern(swz, pitch, v_chunk0, d4, key0)) == 1, (pitch, d4, key0)


@pytest.mark.parametrize("db", range(4))
def test_prefill_vt_reads_conflict_free(db):
    swz = _lib().host_prefill_v_swz
    for key0 in (0, 8, 16, 24, 32, 40, 48, 56):          # 16-key groups of a 64-key stage, and the +8 row
        assert ways_64bit(vt_prefill_pattern(swz, db, key0)) == 1, (db, key0)


def test_rule_flags_the_previous_layouts():
    """The rule is not vacuous: the layouts the kernels used before break it, as the counter measured."""
    assert ways_64bit(vt_row_pattern(old_row, 1152, 0, 0, 0)) == 2
    assert ways_64bit(vt_row_pattern(old_row, 640, 24, 0, 0)) == 2
    assert ways_64bit(vt_prefill_pattern(old_prefill_v, 0, 0)) == 2
    assert ways_64bit([lane * 8 for lane in range(64)]) == 1      # a linear 512-byte read


def test_swizzles_stay_in_their_chunk_groups():
    """A swizzle must map a chunk group onto itself (8 chunks; 4 for the fp8 rows) for every key, and the
    bf16 row swizzle must depend on the key mod 16 only (the 16-key halves of a tile share it)."""
    lib = _lib()
    for key in range(64):
        assert 0 <= lib.host_row_chunk_swz(key) < 8 and 0 <= lib.host_prefill_k_swz(key) < 8
        assert 0 <= lib.host_fp8_chunk_swz(key) < 4 and 0 <= lib.host_prefill_v_swz(key) < 16
        assert lib.host_row_chunk_swz(key) == lib.host_row_chunk_swz(key % 16)
