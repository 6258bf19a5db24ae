"""Pins of the oracle's E4M3FN codec (OCP FP8 E4M3FN; saturating RNE quantiser).

The pages name an fp8 E4M3 KV cache with per-tensor and per-head scales (vLLM PR
#64064, section "Tests"; diffbot model card, intro).  The codec is pinned to the
format's defining values and to torch's independent float8_e4m3fn cast.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3fn


def torch_cast(q32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(q32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_defining_values():
    d = e4m3fn.decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0         # largest finite
    assert d(0x38) == 1.0                                  # exponent field 7 = bias
    assert d(0x08) == 2.0 ** -6                            # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))         # the only NaNs, no infinities
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert d(0x77) == 240.0                                # 2**7 * 1.875


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = e4m3fn.encode(e4m3fn.decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    vals = e4m3fn.decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        assert float(mid) == (vals[c] + vals[c + 1]) / 2  # exact in binary32
        even = c if c % 2 == 0 else c + 1
        assert e4m3fn.encode(mid) == even, hex(c)
        assert e4m3fn.encode(np.nextafter(mid, np.float32(0))) == c
        assert e4m3fn.encode(np.nextafter(mid, np.float32(np.inf))) == c + 1
        assert e4m3fn.encode(-mid) == (even | 0x80)


def test_saturation_nan_and_signed_zero():
    enc = e4m3fn.encode
    f = np.float32
    assert enc(f(448)) == 0x7E and enc(f(449)) == 0x7E and enc(f(1e30)) == 0x7E
    assert enc(f(np.inf)) == 0x7E and enc(f(-np.inf)) == 0xFE and enc(f(-500)) == 0xFE
    assert enc(f(np.nan)) == 0x7F and enc(-f(np.nan)) == 0x7F
    assert enc(f(-1e-10)) == 0x80 and enc(f(-0.0)) == 0x80 and enc(f(0.0)) == 0x00
    assert enc(f(2.0 ** -10)) == 0x00          # exactly half the smallest subnormal: tie to even (0)
    assert enc(f(3 * 2.0 ** -10)) == 0x02      # 1.5 subnormal steps: tie to even (2)
    assert enc(f(3 * 2.0 ** -11)) == 0x01      # 0.75 subnormal steps: nearest is 1


def test_exhaustive_bf16_times_scales_vs_torch_cast():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x32 = e4m3fn.bf16_bits_to_f32(bits)
    for s in (1.0, 0.0123, 0.05, 0.0678, 0.1, 0.37, 3.0):
        codes = e4m3fn.quantize(bits, np.float32(s))
        q = x32 / np.float32(s)
        ours_range = ~np.isnan(q) & (np.abs(q) <= 464.0)  # torch rounds to NaN above 464
        ref = torch_cast(q)
        assert np.array_equal(codes[ours_range], ref[ours_range]), s
        big = ~np.isnan(q) & (np.abs(q) >= 448.0)
        assert np.all((codes[big] & 0x7F) == 0x7E)
        assert np.all(codes[np.isnan(q)] == 0x7F)


def test_random_fp32_patterns_vs_torch_cast():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    q = u.view(np.float32)
    # bias half the sample into the interesting range
    q[: len(q) // 2] = (rng.standard_normal(len(q) // 2) * 100).astype(np.float32)
    ok = ~np.isnan(q) & (np.abs(q) <= 464.0)
    assert np.array_equal(e4m3fn.encode(q)[ok], torch_cast(q)[ok])


@pytest.mark.parametrize("planted", ["truncate", "ties_away"])
def test_planted_rounding_mistakes_are_caught(planted):
    """A mis-rounding encoder (a plausible mistake) must fail the torch-cast pin."""
    vals = e4m3fn.decode(np.arange(0x7F, dtype=np.uint8))

    def bad_encode(q):
        a = np.abs(np.asarray(q, dtype=np.float64))
        idx = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
        if planted == "ties_away":
            nxt = np.clip(idx + 1, 0, 0x7E)
            idx = np.where(np.abs(vals[nxt] - a) <= np.abs(a - vals[idx]), nxt, idx)
        return (idx | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)

    mids = np.array([(vals[c] + vals[c + 1]) / 2 for c in range(0x7E)], dtype=np.float32)
    q = np.concatenate([mids, mids * np.float32(1.0001)])
    assert not np.array_equal(bad_encode(q), torch_cast(q))
