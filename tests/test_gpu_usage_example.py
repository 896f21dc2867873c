"""The usage example of the README, run as written (device tensors in logical
token order, the chunk-major permutation, forward, backward, and back, a
strided view, and one query chunk step by step as one device of a ring runs
it), with its results checked against the oracle on a few rows."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import layout as OL

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
    # a [B, S, H, d] buffer read in place through a strided view
    x_bshd = torch.randn(1, S, 8, 128, device="cuda").to(torch.bfloat16)
    xp = api.to_chunked(x_bshd.transpose(1, 2), "zigzag", N)
    torch.cuda.synchronize()
    assert torch.equal(xp, api.to_chunked(x_bshd.transpose(1, 2).contiguous(), "zigzag", N))
    # one device of a ring (ra_ring_step): query chunk i stays, KV chunks arrive in ring order
    i, L = 2, S // N
    qi = qp[:, :, i * L:(i + 1) * L]
    st = api.state_init(qi, kp)
    for t in range(N):
        j = (i - t) % N                                   # the KV chunk held at step t
        api.ring_step(st, qi, kp[:, :, j * L:(j + 1) * L], vp[:, :, j * L:(j + 1) * L],
                      step=t, seq=S, n_chunks=N, layout="zigzag", causal=True, q_chunk=i)
    out_i, lse_i = api.finalize(st, qi)                   # chunk i of out and lse
    torch.cuda.synchronize()
    # the same chunk from the fused launch, and a few of its rows against the definition
    assert max_abs(out_i, out[:, :, i * L:(i + 1) * L]) <= TOL["bf16"]
    assert max_abs(lse_i, lse[:, :, i * L:(i + 1) * L]) <= TOL["bf16"]
    pos_i = OL.chunk_positions("zigzag", S, N, i)
    sel = np.array([0, 1, L // 2 - 1, L // 2, L - 1])
    ref_i, ref_lse_i = OA.attention_reference(qi[:, :, sel].cpu(), k.cpu(), v.cpu(), causal=True,
                                              q_pos=pos_i[sel], k_pos=np.arange(S))
    assert max_abs(out_i[:, :, sel], ref_i) <= TOL["bf16"]
    assert max_abs(lse_i[:, :, sel], ref_lse_i) <= TOL["bf16"]
