"""GPU parity of ra_ring_bwd (bf16 inputs, d = 128) against the float64
backward oracle, element by element on seeded inputs: every layout, causal and
not, grouped heads, query-chunk subsets, chunk lengths that leave ragged
tiles (32-row query steps, 32-key dQ tiles, 256-key dK/dV tiles).

The backward kernel consumes a forward output and lse: the oracle's (cast to
bf16 / fp32) in the unit cases, the library's own forward in the end-to-end
case.  The expected gradients always come from the oracle's definition
(P recomputed from the scores).  Tolerance: max-abs 2e-2 (bf16 inputs, fp32
accumulation, P and dS rounded to bf16 as MFMA operands)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as OA
from oracle import backward as OB
from oracle import layout as OL

from .parity_utils import TOL, max_abs, physical_inputs, query_rows_positions

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402
from exact_long_context_amd import ringattn as ra  # noqa: E402

DEV = "cuda"


def _setup(w, seed_do):
    qp, kp, vp, _, k, v = physical_inputs(w, device=DEV)
    do = synthetic.normal_draw(qp.shape, seed_do, dtype=torch.bfloat16, device=DEV)
    return qp, kp, vp, k, v, do


def _oracle(w, qp, k, v, do):
    qpos = query_rows_positions(w)
    kpos = np.arange(w.seq)
    out, lse = OA.attention_reference(qp.cpu(), k.cpu(), v.cpu(), causal=w.causal, q_pos=qpos, k_pos=kpos)
    dq, dk, dv = OB.attention_backward_reference(qp.cpu(), k.cpu(), v.cpu(), do.cpu(), causal=w.causal,
                                                 q_pos=qpos, k_pos=kpos)
    return out, lse, dq, dk, dv


def _physical_kv(w, x_log):
    """Logical-order [B, H, S, d] float64 -> chunk-major order."""
    return x_log[:, :, OL.all_positions(w.layout, w.seq, w.n_chunks)]


def _check(w, got, want):
    dq, dk, dv = got
    rdq, rdk, rdv = want
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    errs = (max_abs(dq, rdq), max_abs(dk, _physical_kv(w, rdk)), max_abs(dv, _physical_kv(w, rdv)))
    print(f"  max-abs error dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e} (magnitudes "
          f"{np.abs(rdq).max():.2e} {np.abs(rdk).max():.2e} {np.abs(rdv).max():.2e})", flush=True)
    assert max(errs) <= TOL["bf16"]


CASES = [
    # layout, S, N, hq, hkv, causal, q_chunks
    ("contiguous", 1024, 4, 4, 4, True, None),
    ("contiguous", 1024, 4, 8, 2, False, None),
    ("zigzag", 1600, 8, 8, 2, True, None),          # s = 100: ragged 32-row steps and tiles
    ("zigzag", 2048, 4, 4, 1, True, (1, 2)),        # s = 256, a query-chunk subset
    ("striped", 1152, 4, 4, 2, True, None),         # L = 288: two 256-key tiles, the second ragged
    ("striped", 576, 8, 2, 2, False, (3,)),
    ("contiguous", 1000, 4, 2, 1, True, (2, 3)),    # L = 250
    ("zigzag", 8192, 4, 8, 2, True, None),          # dQ: 256 workgroups over 2 KV streams, blocks of 32 per XCD
]


@pytest.mark.parametrize("layout,S,N,hq,hkv,causal,qc", CASES)
def test_ring_bwd_every_element(layout, S, N, hq, hkv, causal, qc):
    print(f"case bwd {layout} S={S} N={N} hq={hq} hkv={hkv} causal={causal} q_chunks={qc}", flush=True)
    w = synthetic.Workload("t", 1, hq, hkv, S, N, 128, "bf16", causal, layout, seed=S + hq, q_chunks=qc)
    qp, kp, vp, k, v, do = _setup(w, seed_do=7 + S)
    out, lse, rdq, rdk, rdv = _oracle(w, qp, k, v, do)
    out_d = torch.from_numpy(out).to(torch.bfloat16).to(DEV)
    lse_d = torch.from_numpy(lse).to(torch.float32).to(DEV)
    dq, dk, dv = api.ring_backward(qp, kp, vp, out_d, do, lse_d, seq=S, n_chunks=N, layout=layout, causal=causal,
                                   q_chunk_first=w.query_chunks[0])
    torch.cuda.synchronize()
    _check(w, (dq, dk, dv), (rdq, rdk, rdv))


@pytest.mark.parametrize("layout,causal", [("zigzag", True), ("striped", True), ("contiguous", False)])
def test_forward_then_backward(layout, causal):
    """The library's own forward (bf16 out, lse) feeding its backward."""
    print(f"case fwd+bwd {layout} causal={causal}", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, 2048, 4, 128, "bf16", causal, layout, seed=41)
    qp, kp, vp, k, v, do = _setup(w, seed_do=43)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=layout, causal=causal)
    dq, dk, dv = api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=w.n_chunks, layout=layout,
                                   causal=causal)
    torch.cuda.synchronize()
    _, _, rdq, rdk, rdv = _oracle(w, qp, k, v, do)
    _check(w, (dq, dk, dv), (rdq, rdk, rdv))


@pytest.mark.parametrize("layout,causal", [("zigzag", True), ("contiguous", False)])
def test_forward_fp32_out_then_backward(layout, causal):
    """An fp32 forward output feeding the backward (its D = rowsum(dO * O)
    reads fp32 out; dout stays bf16 with the same element strides)."""
    print(f"case fwd(fp32 out)+bwd {layout} causal={causal}", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, 1600, 4, 128, "bf16", causal, layout, seed=47)
    qp, kp, vp, k, v, do = _setup(w, seed_do=49)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=layout, causal=causal,
                                out_dtype=torch.float32)
    assert out.dtype == torch.float32 and out.stride() == do.stride()
    dq, dk, dv = api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=w.n_chunks, layout=layout,
                                   causal=causal)
    torch.cuda.synchronize()
    _, _, rdq, rdk, rdv = _oracle(w, qp, k, v, do)
    _check(w, (dq, dk, dv), (rdq, rdk, rdv))


def test_backward_invariants_and_rejections():
    """Key gradients of each KV head sum to zero and value gradients to the
    sum of the upstream gradients of the rows that see a key (every row here);
    unsupported inputs are rejected before any launch."""
    w = synthetic.Workload("t", 1, 8, 2, 4096, 8, 128, "bf16", True, "zigzag", seed=5)
    qp, kp, vp, k, v, do = _setup(w, seed_do=9)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=True)
    dq, dk, dv = api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                                   causal=True)
    torch.cuda.synchronize()
    # sum over keys: exactly 0 in exact arithmetic; here a small fraction of the sum of magnitudes
    ksum = dk.double().sum(dim=2).abs()
    assert (ksum <= 0.02 * dk.double().abs().sum(dim=2) + 1e-3).all()
    # each row's bf16-rounded weights sum to 1 within 2^-9: that bounds the value-gradient sums
    G = 4
    for g in range(2):
        rows = do[:, g * G:(g + 1) * G].double()
        want = rows.sum(dim=(1, 2))
        bound = rows.abs().sum(dim=(1, 2)) * 2.0 ** -9 + 1e-3
        assert ((dv[:, g].double().sum(dim=1) - want).abs() <= bound).all()
    f32 = qp.float()
    desc = ra.ring_desc(f32, kp.float(), vp.float(), seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=True,
                        out=out, lse=lse)
    ws = torch.empty(ra.ra_ring_bwd_workspace_bytes(desc) + 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_bwd(desc, f32, kp.float(), vp.float(), out, do, lse, dq, dk, dv, ws, ws.numel())
    desc = ra.ring_desc(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=True, out=out, lse=lse)
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_bwd(desc, qp, kp, vp, out, do, lse, dq, dk, dv, ws, 8)


def test_backward_is_deterministic():
    """No atomics anywhere in the backward: two calls on the same inputs give
    the same bits, also with a query-chunk subset and grouped heads."""
    print("case bwd determinism", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, 2048, 8, 128, "bf16", True, "zigzag", seed=61, q_chunks=(2, 3, 4))
    qp, kp, vp, k, v, do = _setup(w, seed_do=63)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=True,
                                q_chunk_first=2)
    runs = [api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                              causal=True, q_chunk_first=2) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def _bshd(x: torch.Tensor, dtype=None) -> torch.Tensor:
    """A [B, S, H, d] buffer seen as [B, H, S, d] (row stride H d elements),
    holding x's values (or uninitialised, in dtype, when dtype is given)."""
    B, H, S, d = x.shape
    buf = torch.empty(B, S, H, d, dtype=dtype or x.dtype, device=x.device).transpose(1, 2)
    if dtype is None:
        buf.copy_(x)
    return buf


@pytest.mark.parametrize("batch,hq,hkv,S,N,layout,causal", [(1, 8, 2, 1600, 8, "zigzag", True),
                                                            (2, 3, 3, 1152, 4, "striped", True),
                                                            (2, 4, 1, 1000, 4, "contiguous", False)])
def test_backward_strided_views_bitwise(batch, hq, hkv, S, N, layout, causal):
    """ra_ring_bwd reading q, k, v, out and dout in place from [B, S, H, d]
    buffers (every staged row at a row stride of H d elements, not d) and
    writing the gradients with the same strides: bit for bit the gradients of
    the contiguous call, since no arithmetic depends on the strides."""
    print(f"case bwd strided views B={batch} hq={hq} hkv={hkv} S={S} N={N} {layout} causal={causal}", flush=True)
    w = synthetic.Workload("t", batch, hq, hkv, S, N, 128, "bf16", causal, layout, seed=67)
    qp, kp, vp, k, v, do = _setup(w, seed_do=69)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=causal)
    want = api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                             causal=causal)
    qs, ks, vs, outs, dos = (_bshd(t) for t in (qp, kp, vp, out, do))
    assert qs.stride(2) == w.hq * w.d and ks.stride(2) == w.hkv * w.d
    got = tuple(_bshd(t, torch.float32) for t in (qp, kp, vp))
    desc = ra.ring_desc(qs, ks, vs, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=causal, out=outs,
                        lse=lse)
    need = ra.ra_ring_bwd_workspace_bytes(desc)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    ra.ra_ring_bwd(desc, qs, ks, vs, outs, dos, lse, *got, ws, need)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a.contiguous().view(torch.int32), b.view(torch.int32))
