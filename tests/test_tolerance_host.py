"""CPU pin of the edge-case tolerance helper: bf16_half_ulp is half of torch's own bf16 spacing
(the gap from a bf16 value's magnitude to the next larger bf16), on random values over many
binades and at the binade edges; this is the allowance the small edge-case parity tests add for
the bf16 output's own rounding."""
import numpy as np
import torch

from _gpu_util import bf16_half_ulp


def _torch_half_spacing(b: torch.Tensor) -> np.ndarray:
    mag = b.abs()
    up = (mag.view(torch.int16).int() + 1).short().view(torch.bfloat16)   # next bf16 above |b|
    return ((up.double() - mag.double()) / 2).numpy()


def test_half_ulp_matches_torch_spacing():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 6)
    b = x.to(torch.bfloat16)
    b = b[torch.isfinite(b) & (b != 0)]
    assert np.array_equal(bf16_half_ulp(b.float().numpy()), _torch_half_spacing(b))


def test_half_ulp_binade_edges():
    v = np.array([1.0, 1.9921875, 2.0, 3.984375, 4.0, -4.0, 2.0 ** -126, 2.0 ** -130])
    got = bf16_half_ulp(v)
    assert list(got[:6]) == [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6]
    assert got[6] == 2.0 ** -134 and got[7] == 2.0 ** -134
    b = torch.tensor(v[6:], dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(got[6:], _torch_half_spacing(b))
