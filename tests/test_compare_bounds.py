"""The parity comparison's bounds (tests/_gpu_util.compare), checked on the CPU with synthetic
results: max abs 1e-2 and RMSE 1e-3 for bf16 outputs (the pages' tolerance).  Configuration-size
tests take them as stated (strict); the small edge cases take them beyond the bf16 output's own
rounding (half a bf16 ulp of each output), because an exact result of magnitude ~1 rounded to
bf16 already has an RMSE of ~2e-3.  The allowance must not hide a real error: an extra error
on top of the rounding, or an error on small outputs, still fails."""
import numpy as np
import pytest
import torch

from _gpu_util import compare


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def _ref(scale, seed=0):
    rng = np.random.default_rng(seed)
    sign = np.where(rng.random((64, 4, 128)) < 0.5, -1.0, 1.0)
    return sign * scale * (1.0 + rng.random((64, 4, 128)))      # |ref| in [scale, 2 scale)


def test_exact_result_rounded_to_bf16_passes_the_edge_case_bounds():
    ref = _ref(1.0)
    got = _bf16(ref)
    rmse = float(np.sqrt(np.mean((got.double().numpy() - ref) ** 2)))
    assert rmse > 1e-3                       # the rounding alone is over the stated RMSE bound
    compare(got, ref, what="rounded exact result")
    with pytest.raises(AssertionError, match="rmse"):
        compare(got, ref, what="rounded exact result, strict", strict=True)


@pytest.mark.parametrize("scale,extra", [(1.0, 1.2e-2), (0.3, 4e-3)])
def test_an_error_beyond_the_rounding_still_fails(scale, extra):
    ref = _ref(scale, seed=1)
    got = _bf16(ref + extra)
    with pytest.raises(AssertionError):
        compare(got, ref, what=f"extra error {extra} at |ref| ~ {scale}")


def test_small_outputs_get_no_real_allowance():
    ref = _ref(0.01, seed=2)
    rng = np.random.default_rng(3)
    got = _bf16(ref + 1.5e-3 * rng.standard_normal(ref.shape))
    with pytest.raises(AssertionError, match="rmse"):
        compare(got, ref, what="small outputs with a 1.5e-3 error")


def test_max_abs_bound_beyond_rounding():
    ref = _ref(1.0, seed=4)
    err = np.zeros_like(ref)
    err[0, 0, 0] = 2e-2                      # one element off by twice the bound
    with pytest.raises(AssertionError, match="max abs"):
        compare(_bf16(ref + err), ref, what="one element off")
