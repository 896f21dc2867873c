"""GPU parity at the full workload shapes, in the launch configuration the
bench times (one fused ra_ring_fwd, bf16 output plus lse).

The non-causal 8K workloads are compared element by element; the larger
ones on a seeded sample of query rows (always including the first and last
row of every query segment), each row against all its visible keys, plus
properties that hold for every row (finite output, lse at least the largest
visible score)."""
import numpy as np
import pytest
import torch

import synthetic

from .parity_utils import TOL, max_abs, oracle_all_rows, oracle_sampled, physical_inputs, sample_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402


def _run(w):
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                q_chunk_first=w.query_chunks[0])
    torch.cuda.synchronize()
    return out, lse, qp, k, v


@pytest.mark.parametrize("name", ["mha_8k", "mha_8k_sharp"])
def test_full_noncausal_8k_every_element(name):
    w = synthetic.WORKLOADS[name]
    print(f"case full {name}", flush=True)
    out, lse, qp, k, v = _run(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal=False)
    assert max_abs(out, ref) <= TOL["bf16"]
    rel = np.max(np.abs(lse.cpu().double().numpy() - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))
    assert rel <= TOL["bf16"]


@pytest.mark.parametrize("name,n", [("causal_contig_32k", 1024), ("causal_striped_128k", 1024),
                                    ("zigzag_1m_gqa", 768), ("usp_1m_share", 512)])
def test_full_causal_sampled_rows(name, n):
    w = synthetic.WORKLOADS[name]
    print(f"case full {name} ({n} sampled rows)", flush=True)
    out, lse, qp, k, v = _run(w)
    assert torch.isfinite(out.float()).all()
    assert torch.isfinite(lse).all()
    samples = sample_rows(w, n, seed=sum(map(ord, name)))
    ref, ref_lse = oracle_sampled(w, samples, qp, k, v, causal=True)
    hs = torch.tensor([h for h, _ in samples], device=out.device)
    rs = torch.tensor([r for _, r in samples], device=out.device)
    got = out[0, hs, rs].float().cpu().double().numpy()
    got_lse = lse[0, hs, rs].cpu().double().numpy()
    assert max_abs(got, ref) <= TOL["bf16"]
    assert max_abs(got_lse, ref_lse) <= TOL["bf16"]
    if name == "zigzag_1m_gqa":
        # the last query chunk against all 32 KV chunks as well
        w2 = w.scaled(q_chunks=(31,))
        print("case full zigzag_1m_gqa chunk 31", flush=True)
        out2, lse2, qp2, k2, v2 = _run(w2)
        s2 = sample_rows(w2, 256, seed=31)
        ref2, ref2_lse = oracle_sampled(w2, s2, qp2, k2, v2, causal=True)
        hs2 = torch.tensor([h for h, _ in s2], device=out2.device)
        rs2 = torch.tensor([r for _, r in s2], device=out2.device)
        assert max_abs(out2[0, hs2, rs2].float().cpu().double().numpy(), ref2) <= TOL["bf16"]
        assert max_abs(lse2[0, hs2, rs2].cpu().double().numpy(), ref2_lse) <= TOL["bf16"]


def test_full_backward_zigzag_1m_sampled():
    """ra_ring_bwd at the 1M-token zig-zag GQA shape, in the configuration the
    bench times (the library's forward output and lse as inputs): dq on a
    seeded sample of query rows against the oracle (each row against all its
    visible keys); dk and dv finite everywhere, with the sums over the keys of
    each KV head that hold at any size (key gradients cancel; value gradients
    add up to the upstream gradients within the bf16 rounding of the
    weights)."""
    from oracle import backward as OB
    from .parity_utils import query_rows_positions
    w = synthetic.WORKLOADS["zigzag_1m_gqa"]
    print("case full backward zigzag_1m_gqa", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=True)
    do = synthetic.normal_draw(qp.shape, 77, dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                                   causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    G = w.hq // w.hkv
    for g in range(w.hkv):
        ksum = dk[0, g].double().sum(dim=0).abs()
        assert (ksum <= 0.02 * dk[0, g].double().abs().sum(dim=0) + 1e-3).all()
        rows = do[0, g * G:(g + 1) * G].double()
        bound = rows.abs().sum(dim=(0, 1)) * 2.0 ** -9 + 1e-2
        assert ((dv[0, g].double().sum(dim=0) - rows.sum(dim=(0, 1))).abs() <= bound).all()
    del kp, vp
    samples = sample_rows(w, 48, seed=1234)
    qpos = query_rows_positions(w)
    qc, doc = qp.cpu(), do.cpu()
    by_kv = {}
    for i, (h, r) in enumerate(samples):
        by_kv.setdefault(h // G, []).append(i)
    want = np.zeros((len(samples), w.d))
    for g, idx in by_kv.items():
        # the sampled rows of the group's heads as one block of rows against KV head g
        kg, vg = k[:, g:g + 1].cpu(), v[:, g:g + 1].cpu()
        hs_, rs_ = [samples[i][0] for i in idx], [samples[i][1] for i in idx]
        qsel = torch.stack([qc[0, h, r] for h, r in zip(hs_, rs_)])[None, None]
        dsel = torch.stack([doc[0, h, r] for h, r in zip(hs_, rs_)])[None, None]
        dqr, _, _ = OB.attention_backward_reference(qsel, kg, vg, dsel, causal=True, q_pos=qpos[rs_],
                                                    k_pos=np.arange(w.seq))
        want[idx] = dqr[0, 0]
    hs = torch.tensor([h for h, _ in samples], device=dq.device)
    rs = torch.tensor([r for _, r in samples], device=dq.device)
    err = max_abs(dq[0, hs, rs].cpu().double().numpy(), want)
    print(f"  dq max-abs error on {len(samples)} rows {err:.2e} (magnitude {np.abs(want).max():.2e})", flush=True)
    assert err <= TOL["bf16"]


def _check_sampled(w, out, lse, qp, k, v, n, seed):
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    samples = sample_rows(w, n, seed=seed)
    ref, ref_lse = oracle_sampled(w, samples, qp, k, v, causal=w.causal)
    hs = torch.tensor([h for h, _ in samples], device=out.device)
    rs = torch.tensor([r for _, r in samples], device=out.device)
    e_out = max_abs(out[0, hs, rs].float().cpu().double().numpy(), ref)
    e_lse = max_abs(lse[0, hs, rs].cpu().double().numpy(), ref_lse)
    print(f"  max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]


@pytest.mark.parametrize("name,qc", [("mha_8k", 0), ("causal_striped_128k", 15)])
def test_full_split_kv_one_chunk_sampled(name, qc):
    """Split-KV in the configuration the bench times: one query chunk of the
    workload with the library's suggested number of KV ranges."""
    from exact_long_context_amd import ringattn as ra
    w = synthetic.WORKLOADS[name].scaled(q_chunks=(qc,))
    q = torch.empty(w.batch, w.hq, w.chunk, w.d, dtype=torch.bfloat16)
    kk = torch.empty(w.batch, w.hkv, w.seq, w.d, dtype=torch.bfloat16)
    splits = ra.ra_ring_kv_splits_hint(ra.ring_desc(q, kk, kk, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                                                    causal=w.causal, q_chunk_first=qc))
    assert splits > 1
    print(f"case full split-KV {name} chunk {qc}, {splits} ranges", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                q_chunk_first=qc, kv_splits=splits)
    torch.cuda.synchronize()
    _check_sampled(w, out, lse, qp, k, v, 512, seed=qc + 7)


def test_full_ring_step_zigzag_1m_sampled():
    """The 1M-token zig-zag share run step by step as the bench times it: state
    init, 32 ra_ring_step calls each given only its KV chunk, finalize."""
    w = synthetic.WORKLOADS["zigzag_1m_gqa"]
    print("case full ring step zigzag_1m_gqa", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = api.ring_forward_stepwise(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                                         causal=True, q_chunk=w.query_chunks[0])
    torch.cuda.synchronize()
    _check_sampled(w, out, lse, qp, k, v, 512, seed=1234)
