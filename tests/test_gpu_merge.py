"""GPU parity of attn_merge_lse against the oracle's log-sum-exp merge, including rows
whose partials are all empty (diffbot model card, "Update 2026-10-01": 0, not NaN)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
from _gpu_util import DEV
from oracle import paged_ref as R

pytestmark = pytest.mark.gpu


# P <= 32 runs the one-thread-per-column kernel (instances for up to 8, 16 and 32
# partitions), larger P the LDS-combining one
@pytest.mark.parametrize("P,Dv", [(1, 128), (8, 128), (9, 512), (16, 128), (32, 128), (33, 128), (96, 512),
                                  (300, 128)])
def test_merge_matches_oracle(gpu_lib, P, Dv):
    rng = np.random.default_rng(P)
    rows, Hq = 5, 12
    po = rng.standard_normal((rows, Hq, P, Dv)).astype(np.float32)
    pl = (rng.standard_normal((rows, Hq, P)) * 3).astype(np.float32)
    pl[rng.random((rows, Hq, P)) < 0.3] = -np.inf         # empty partitions
    pl[1] = -np.inf                                        # a row with no visible key at all
    po[1] = 0
    ref, ref_lse = R.merge_lse(po.astype(np.float64), pl.astype(np.float64))
    out, lse = pk.merge_lse(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV))
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    # bf16 output: half an ulp of |ref| plus fp32 accumulation slack
    tol = np.abs(ref) * 2.0 ** -8 + 1e-6
    assert np.all(np.abs(got - ref) <= tol)
    assert np.all(got[1] == 0) and not np.any(np.signbit(got[1]))
    l = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.abs(l[fin] - ref_lse[fin]).max() <= 1e-5 * max(1.0, np.abs(ref_lse[fin]).max())
