"""ra_ring_bwd_noalloc (the backward for callers that cannot allocate device
memory) against ra_ring_bwd with a caller-supplied workspace: two calls in a
row on the same GPU, the first at the entry point's largest workspace, the
second with a smaller input, each compared bit for bit with the workspace
entry point on the same inputs (the same kernels run; only the workspace
differs).  Outputs are poisoned with NaN first, so every value is checked
as written by the call."""
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402
from exact_long_context_amd import ringattn as ra  # noqa: E402


def _inputs(w, seed_do):
    q, k, v = synthetic.draw(w, device="cuda")
    qp, kp, vp = (api.to_chunked(t, w.layout, w.n_chunks) for t in (q, k, v))
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal)
    do = synthetic.normal_draw(qp.shape, seed_do, dtype=torch.bfloat16, device="cuda")
    return qp, kp, vp, out, lse, do


def _grads(qp, kp, vp):
    return tuple(torch.full(t.shape, float("nan"), dtype=torch.float32, device="cuda") for t in (qp, kp, vp))


def test_noalloc_backward_matches_workspace_backward():
    cases = [
        # 32 query heads x 65536 query rows: exactly the largest workspace (16 MiB)
        synthetic.Workload("t", 1, 32, 8, 65536, 4, 128, "bf16", True, "zigzag", seed=71),
        # then a smaller call on the same GPU (the array keeps the first call's contents)
        synthetic.Workload("t", 1, 4, 2, 2400, 4, 128, "bf16", True, "striped", seed=73),
    ]
    for n, w in enumerate(cases):
        print(f"case no-alloc backward {n}: {w.layout} S={w.seq} N={w.n_chunks} hq={w.hq} hkv={w.hkv}", flush=True)
        qp, kp, vp, out, lse, do = _inputs(w, seed_do=75 + n)
        desc = ra.ring_desc(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal, out=out,
                            lse=lse)
        need = ra.ra_ring_bwd_workspace_bytes(desc)
        assert need <= ra.RA_BWD_NOALLOC_MAX_BYTES
        if n == 0:
            assert need == ra.RA_BWD_NOALLOC_MAX_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = _grads(qp, kp, vp)
        ra.ra_ring_bwd(desc, qp, kp, vp, out, do, lse, *ref, ws, need)
        got = _grads(qp, kp, vp)
        ra.ra_ring_bwd_noalloc(desc, qp, kp, vp, out, do, lse, *got)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.isfinite(a).all(), name
            assert torch.equal(a, b), name
        del qp, kp, vp, out, lse, do, ws, ref, got
        torch.cuda.empty_cache()
