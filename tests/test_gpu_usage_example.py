"""The usage example of the README, run as written (device tensors in logical
token order, the chunk-major permutation, forward, backward, and back), with
its results checked against the oracle on a few rows."""
import numpy as np
import pytest
import torch

from oracle import attention as OA

from .parity_utils import TOL, max_abs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_usage_example():
    print("case usage example", flush=True)
    from exact_long_context_amd import api
    torch.manual_seed(0)
    S, N = 8192, 4
    q, k, v = (torch.randn(1, 8, S, 128, device="cuda").to(torch.bfloat16) for _ in range(3))
    qp, kp, vp = (api.to_chunked(t, "zigzag", N) for t in (q, k, v))
    out, lse = api.ring_forward(qp, kp, vp, seq=S, n_chunks=N, layout="zigzag", causal=True)
    dq, dk, dv = api.ring_backward(qp, kp, vp, out, torch.randn_like(out), lse,
                                   seq=S, n_chunks=N, layout="zigzag", causal=True)
    out_logical = api.from_chunked(out, "zigzag", N)
    torch.cuda.synchronize()
    assert out_logical.shape == q.shape and dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    # a few logical rows against the definition (causal over logical positions)
    rows = np.array([0, 1, 4095, 4096, 8191])
    ref, ref_lse = OA.attention_reference(q[:, :, rows].cpu(), k.cpu(), v.cpu(), causal=True, q_pos=rows,
                                          k_pos=np.arange(S))
    assert max_abs(out_logical[:, :, rows], ref) <= TOL["bf16"]
