"""E4M3FN codec of the oracle (test infrastructure; see ``oracle/__init__``).

The pages ask for an fp8 "E4M3" KV cache with per-tensor and per-head scales
(vLLM PR #64064, section "Tests"; diffbot MiMo-V2.6-Flash model card, intro and
"What the kernels do") but do not spell out the format or the rounding.  The
reading taken here: the OCP FP8 E4M3FN format (the gfx950 native fp8 flavour)
  * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  * exponent field 0 holds subnormals  m * 2**-9;
  * no infinities; S.1111.111 (0x7F / 0xFF) is NaN; the largest finite value is
    S.1111.110 = 448;
and the quantiser  code = encode(fp32(x) / fp32(scale))  with
  * round to nearest, ties to the even code;
  * saturation: every |q| >= 448 (and +-inf) becomes +-448;
  * underflow to zero keeps the sign (0x80 for negative values);
  * NaN becomes 0x7F whatever its sign bit.

``decode`` is the closed form of the format; ``encode`` is a nearest-neighbour
search over the 127 non-negative finite codes, written from that definition.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F
SAT_CODE = 0x7E


def decode(codes) -> np.ndarray:
    """Value of each E4M3FN byte as float64 (NaN for 0x7F / 0xFF)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & ((b & 0x7) == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite codes 0x00..0x7E, whose values increase with the code
_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)
_POS_VALUES = decode(_POS_CODES.astype(np.uint8))
assert np.all(np.diff(_POS_VALUES) > 0)


def encode(q32) -> np.ndarray:
    """Round fp32 values to E4M3FN bytes: nearest, ties to even, saturating."""
    q = np.asarray(q32, dtype=np.float32)
    a = np.abs(q.astype(np.float64))
    neg = np.signbit(q)
    # nearest representable magnitude by search over the sorted value table
    hi = np.searchsorted(_POS_VALUES, np.minimum(a, MAX_FINITE), side="left")
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_lo = np.abs(a - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a >= MAX_FINITE, SAT_CODE, code)         # saturate (also +-inf)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(np.isnan(q), NAN_CODE, code)
    return code.astype(np.uint8)


def quantize(x_bf16_bits, scale) -> np.ndarray:
    """Cache-write quantiser: encode(fp32(x) / fp32(scale)), the division in binary32.

    ``x_bf16_bits`` are bf16 bit patterns (uint16); ``scale`` broadcasts against them.
    numpy's float32 division is IEEE binary32, correctly rounded.
    """
    x32 = bf16_bits_to_f32(x_bf16_bits)
    q = np.asarray(x32, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return encode(q.astype(np.float32))


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 is the top half of a binary32: widen by a 16-bit shift."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
