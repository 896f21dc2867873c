"""GPU parity at the full workload shapes, in the launch configuration the
bench times (one fused ra_ring_fwd, bf16 output plus lse; the 8K workloads
also with fp32 output, which isolates the accumulation error from the output
rounding).

* 8K MHA and its sharp-score variant: every element.
* Causal contiguous 32K: every element of all 32 heads (the oracle runs one
  head per thread).
* Causal striped 128K: 4096 sampled query rows.
* The 1M-token zig-zag GQA share: 4096 sampled rows of query chunk 0, spread
  evenly over its two segments and all 32 heads, with the first and last row
  of each segment for every head; 1024 rows of query chunk 31.
* The Ulysses-hybrid share: 1024 sampled rows.
Each sampled row is checked against all its visible keys; every row is also
checked for finite values.  Tolerances: max-abs 2e-2 on out and on lse
(absolute), the bf16 budget."""
import numpy as np
import pytest
import torch

import synthetic

from .parity_utils import (TOL, max_abs, oracle_all_rows, oracle_heads, oracle_sampled, physical_inputs,
                           sample_rows)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402


def _run(w, out_dtype=None):
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                q_chunk_first=w.query_chunks[0], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse, qp, k, v


@pytest.mark.parametrize("name", ["mha_8k", "mha_8k_sharp"])
def test_full_noncausal_8k_every_element(name):
    w = synthetic.WORKLOADS[name]
    print(f"case full {name}", flush=True)
    out, lse, qp, k, v = _run(w)
    out32, lse32, *_ = _run(w, out_dtype=torch.float32)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal=False)
    e16, e32, el = max_abs(out, ref), max_abs(out32, ref), max_abs(lse, ref_lse)
    print(f"  max-abs out bf16 {e16:.3e} fp32 {e32:.3e} lse {el:.3e}", flush=True)
    assert e16 <= TOL["bf16"] and e32 <= TOL["bf16"] and el <= TOL["bf16"]
    assert torch.equal(lse, lse32)


_CONTIG = {}


def _contig_32k():
    if not _CONTIG:
        w = synthetic.WORKLOADS["causal_contig_32k"]
        out, lse, qp, k, v = _run(w)
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
        _CONTIG.update(w=w, out=out.cpu(), lse=lse.cpu(), qp=qp.cpu(), k=k.cpu(), v=v.cpu())
        del out, lse, qp, k, v
        torch.cuda.empty_cache()
    return _CONTIG


@pytest.mark.parametrize("h0", [0, 8, 16, 24])
def test_full_causal_contig_32k_every_element(h0):
    """All 32768 rows of heads h0 .. h0 + 7 (the four cases cover all 32)."""
    print(f"case full causal_contig_32k every element, heads {h0}..{h0 + 7}", flush=True)
    c = _contig_32k()
    refs = oracle_heads(c["w"], range(h0, h0 + 8), c["qp"], c["k"], c["v"], causal=True)
    worst_o = worst_l = 0.0
    for h, (ro, rl) in refs.items():
        worst_o = max(worst_o, max_abs(c["out"][0, h], ro))
        worst_l = max(worst_l, max_abs(c["lse"][0, h], rl))
    print(f"  max-abs out {worst_o:.3e} lse {worst_l:.3e}", flush=True)
    assert worst_o <= TOL["bf16"] and worst_l <= TOL["bf16"]


def _check_sampled(w, out, lse, qp, k, v, samples):
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ref, ref_lse = oracle_sampled(w, samples, qp, k, v, causal=w.causal)
    hs = torch.tensor([h for h, _ in samples], device=out.device)
    rs = torch.tensor([r for _, r in samples], device=out.device)
    e_out = max_abs(out[0, hs, rs].float().cpu().double().numpy(), ref)
    e_lse = max_abs(lse[0, hs, rs].cpu().double().numpy(), ref_lse)
    print(f"  {len(samples)} rows: max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]


@pytest.mark.parametrize("name,qc,n,ends", [("causal_striped_128k", None, 4096, False),
                                            ("zigzag_1m_gqa", 0, 4096, True),
                                            ("zigzag_1m_gqa", 31, 1024, False),
                                            ("usp_1m_share", 0, 1024, True)])
def test_full_causal_sampled_rows(name, qc, n, ends):
    w = synthetic.WORKLOADS[name]
    if qc is not None:
        w = w.scaled(q_chunks=(qc,))
    print(f"case full {name} query chunks {w.query_chunks[0]}.. ({n} sampled rows)", flush=True)
    out, lse, qp, k, v = _run(w)
    samples = sample_rows(w, n, seed=sum(map(ord, name)) + (qc or 0), every_head_ends=ends)
    assert len(samples) >= n
    _check_sampled(w, out, lse, qp, k, v, samples)


def test_full_backward_zigzag_1m_sampled():
    """ra_ring_bwd at the 1M-token zig-zag GQA shape, in the configuration the
    bench times (the library's forward output and lse as inputs): dq on 512
    seeded query rows against the oracle (each row against all its visible
    keys; a dq row needs only its own row's scores); dk and dv, whose rows
    depend on up to every query row of the chunk, element by element on the
    last 32 keys of every KV head (seen by only the chunk's last 32 rows) and,
    for all keys, through the sums over the keys of each KV head that hold at
    any size (key gradients cancel; value gradients add up to the upstream
    gradients within the bf16 rounding of the weights), and finite
    everywhere."""
    from oracle import backward as OB
    from .parity_utils import query_rows_positions, run_threaded
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
    samples = sample_rows(w, 512, seed=1234)
    qpos = query_rows_positions(w)
    qc, doc, kc, vc = qp.cpu(), do.cpu(), k.cpu(), v.cpu()
    groups = {}
    for i, (h, r) in enumerate(samples):
        groups.setdefault((h // G, int(qpos[r]) * 8 // w.seq), []).append(i)

    def one(item):
        (g, _), idx = item
        hs_, rs_ = [samples[i][0] for i in idx], [samples[i][1] for i in idx]
        kmax = int(qpos[rs_].max()) + 1
        qsel = torch.stack([qc[0, h, r] for h, r in zip(hs_, rs_)])[None, None]
        dsel = torch.stack([doc[0, h, r] for h, r in zip(hs_, rs_)])[None, None]
        dqr, _, _ = OB.attention_backward_reference(qsel, kc[:, g:g + 1, :kmax], vc[:, g:g + 1, :kmax], dsel,
                                                    causal=True, q_pos=qpos[rs_], k_pos=np.arange(kmax))
        return idx, dqr[0, 0]

    want = np.zeros((len(samples), w.d))
    for idx, dqr in run_threaded(one, sorted(groups.items())):
        want[idx] = dqr
    hs = torch.tensor([h for h, _ in samples], device=dq.device)
    rs = torch.tensor([r for _, r in samples], device=dq.device)
    err = max_abs(dq[0, hs, rs].cpu().double().numpy(), want)
    print(f"  dq max-abs error on {len(samples)} rows {err:.2e} (magnitude {np.abs(want).max():.2e})", flush=True)
    assert err <= TOL["bf16"]

    # dk and dv of the last M keys of the sequence, the end of the query chunk's
    # own late segment: of all query rows of the chunk only its last M rows see
    # them, so the oracle's ring-order backward over those rows (given their
    # out and lse over all their visible keys) yields these key rows exactly
    from oracle import attention as OA
    from oracle import layout as OL
    M = 32
    tail = np.arange(w.chunk - M, w.chunk)                # buffer rows of query chunk 0 and KV chunk 0
    tpos = OL.chunk_positions(w.layout, w.seq, w.n_chunks, 0)[tail]
    assert (tpos == np.arange(w.seq - M, w.seq)).all()

    def tail_grads(g):
        hs_ = list(range(g * G, (g + 1) * G))
        qs, dos = qc[:, hs_][:, :, tail], doc[:, hs_][:, :, tail]
        o_ref, lse_ref = OA.attention_reference(qs, kc[:, g:g + 1], vc[:, g:g + 1], causal=True, q_pos=tpos,
                                                k_pos=np.arange(w.seq))
        _, dks, dvs = OB.ring_attention_backward([qs], [kc[:, g:g + 1, w.seq - M:]], [vc[:, g:g + 1, w.seq - M:]],
                                                 [dos], [o_ref], [lse_ref], {0: tpos}, query_chunks=[0],
                                                 causal=True)
        return g, dks[0][0, 0], dvs[0][0, 0]

    for name, lib, pick in (("dk", dk, 1), ("dv", dv, 2)):
        ref = np.stack([r[pick] for r in sorted(run_threaded(tail_grads, range(w.hkv)))])  # [Hkv, M, d]
        got = lib[0, :, w.chunk - M:w.chunk].cpu().double().numpy()
        err, mag = max_abs(got, ref), float(np.abs(ref).max())
        print(f"  {name} on the last {M} keys of every KV head: max-abs error {err:.2e} (magnitude {mag:.2e})",
              flush=True)
        # every row that sees these keys spreads its weight over 1M keys, so their gradients are far
        # below the absolute budget; P and dS are rounded to bf16 (relative 2^-9 per term), which
        # bounds the error relative to the largest entry well under 2^-6
        assert err <= 2.0 ** -6 * mag


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
    _check_sampled(w, out, lse, qp, k, v, sample_rows(w, 1024, seed=qc + 7))


def test_full_ring_step_zigzag_1m_sampled():
    """The 1M-token zig-zag share run step by step as the bench times it: state
    init, 32 ra_ring_step calls each given only its KV chunk, finalize."""
    w = synthetic.WORKLOADS["zigzag_1m_gqa"]
    print("case full ring step zigzag_1m_gqa", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = api.ring_forward_stepwise(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                                         causal=True, q_chunk=w.query_chunks[0])
    torch.cuda.synchronize()
    _check_sampled(w, out, lse, qp, k, v, sample_rows(w, 1024, seed=1234))
