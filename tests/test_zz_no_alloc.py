"""The no-allocation quantile mask (plp_entropy_quantile_mask_noalloc, a
static device scratch instead of a workspace) against the workspace entry
point plp_entropy_quantile_mask, through the C ABI: masks and thresholds equal
bit for bit, on consecutive calls whose later inputs are smaller, so the
shared scratch must be reset by every call."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from tests.gpu_helpers import dev_tensor, require_gpu

pytestmark = pytest.mark.gpu


def _call_both(H, active, q):
    import rl_policy_gradient_amd as plp
    from rl_policy_gradient_amd import _abi
    e, a = dev_tensor(H), dev_tensor(active.astype(np.uint8))
    N = H.shape[0]
    mask_ws, thr_ws = plp.entropy_quantile_mask(e, a, q)
    mask = torch.full((max(N, 1),), 7, dtype=torch.uint8, device="cuda")
    thr = torch.full((1,), 12345.0, dtype=torch.float32, device="cuda")
    L = _abi.lib()
    stream = torch.cuda.current_stream().cuda_stream
    _abi.check(L.plp_entropy_quantile_mask_noalloc(e.data_ptr(), a.data_ptr(), N, float(q), mask.data_ptr(),
                                                   thr.data_ptr(), stream))
    torch.cuda.synchronize()
    return mask_ws.cpu().numpy()[:N], thr_ws.cpu().numpy()[0], mask.cpu().numpy()[:N], thr.cpu().numpy()[0]


@pytest.mark.parametrize("sizes", [((300001, 0.2), (5003, 0.37), (64, 0.0), (4099, 1.0), (2000, 0.8))])
def test_noalloc_matches_workspace_entry_point(sizes):
    require_gpu()
    for k, (N, q) in enumerate(sizes):
        print(f"[case] noalloc call {k}: N={N} q={q}", flush=True)
        sys.stdout.flush()
        r = np.random.default_rng(77 + k)
        H = (r.standard_normal(N) * (1.0 if k % 2 else 1e-3) + 8).astype(np.float32)
        active = r.uniform(size=N) < 0.8
        m_ws, t_ws, m_na, t_na = _call_both(H, active, q)
        np.testing.assert_array_equal(m_na, m_ws)
        if np.isnan(t_ws):
            assert np.isnan(t_na)
        else:
            assert np.float32(t_na).view(np.uint32) == np.float32(t_ws).view(np.uint32), (t_na, t_ws)
        if q < 1.0:
            assert 0 < m_na.sum() <= active.sum()


def test_noalloc_no_active_entry():
    """No active entry: empty mask, NaN threshold, after calls that left
    state behind in the scratch."""
    require_gpu()
    N = 1000
    H = np.linspace(1, 2, N).astype(np.float32)
    _call_both(H, np.ones(N, bool), 0.3)
    m_ws, t_ws, m_na, t_na = _call_both(H, np.zeros(N, bool), 0.3)
    assert m_na.sum() == 0 and np.isnan(t_na) and np.isnan(t_ws)


def test_noalloc_python_binding_into_given_outputs():
    """The package's binding of the same name writes into the caller's
    outputs and agrees with the workspace entry point."""
    require_gpu()
    import rl_policy_gradient_amd as plp
    r = np.random.default_rng(5)
    H = (r.standard_normal(7000) + 3).astype(np.float32)
    active = (r.uniform(size=7000) < 0.7).astype(np.uint8)
    e, a = dev_tensor(H), dev_tensor(active)
    out = (torch.empty(7000, dtype=torch.uint8, device="cuda"), torch.empty(1, dtype=torch.float32, device="cuda"))
    m, t = plp.entropy_quantile_mask_noalloc(e, a, 0.25, out=out)
    m_ws, t_ws = plp.entropy_quantile_mask(e, a, 0.25)
    torch.cuda.synchronize()
    assert m is out[0] and t is out[1]
    assert torch.equal(m, m_ws) and torch.equal(t, t_ws)
