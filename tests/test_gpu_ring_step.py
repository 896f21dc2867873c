"""GPU parity of ``ra_ring_step``: the ring of one query chunk run step by step,
each step given only its KV chunk (as a device of the ring receives it), the
running state in device memory between steps.  Compared element by element
with the float64 oracle (the plain definition) on every layout, causal and
not, grouped heads and ragged tiles, in bf16 and fp32; steps in another order
give the same result up to rounding; a step with nothing visible leaves the
state untouched."""
import numpy as np
import pytest
import torch

import synthetic

from .parity_utils import TOL, max_abs, oracle_all_rows, physical_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402


def _chunk_rows(w, x, i):
    L = w.chunk
    return x[:, :, i * L:(i + 1) * L].contiguous()


def _stepwise(w, qp, kp, vp, i, order=None, out_dtype=None):
    L = w.chunk
    qi = _chunk_rows(w, qp, i)
    st = api.state_init(qi, kp)
    for t in (range(w.n_chunks) if order is None else order):
        j = (i - t) % w.n_chunks
        api.ring_step(st, qi, kp[:, :, j * L:(j + 1) * L], vp[:, :, j * L:(j + 1) * L], step=t, seq=w.seq,
                      n_chunks=w.n_chunks, layout=w.layout, causal=w.causal, q_chunk=i)
    out, lse = api.finalize(st, qi, out_dtype)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # layout, S, N, hq, hkv, batch, causal
    ("contiguous", 800, 4, 8, 2, 1, True),     # L = 200: ragged row and key tiles, GQA 4
    ("contiguous", 800, 4, 4, 4, 2, False),
    ("striped", 1536, 16, 4, 4, 1, True),      # L = 96
    ("zigzag", 1600, 8, 6, 3, 1, True),        # L = 200, s = 100, GQA 2
    ("zigzag", 64, 32, 2, 2, 1, True),         # L = 2, s = 1
]


@pytest.mark.parametrize("layout,S,N,hq,hkv,B,causal", CASES)
def test_ring_step_bf16_every_row(layout, S, N, hq, hkv, B, causal):
    print(f"case ring step bf16 {layout} S={S} N={N} hq={hq} hkv={hkv} B={B} causal={causal}", flush=True)
    w = synthetic.Workload("t", B, hq, hkv, S, N, 128, "bf16", causal, layout, seed=S + N + hq + 2)
    qp, kp, vp, q, k, v = physical_inputs(w)
    for i in sorted({0, N // 2, N - 1}):
        out, lse = _stepwise(w, qp, kp, vp, i, out_dtype=torch.float32)
        ref, ref_lse = oracle_all_rows(w.scaled(q_chunks=(i,)), _chunk_rows(w, qp, i), k, v, causal)
        e_out, e_lse = max_abs(out, ref), max_abs(lse, ref_lse)
        print(f"  chunk {i}: max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
        assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]


@pytest.mark.parametrize("d", [16, 128])
@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("zigzag", True), ("striped", True)])
def test_ring_step_fp32(d, layout, causal):
    print(f"case ring step fp32 d={d} {layout} {causal}", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, 400, 4, d, "f32", causal, layout, seed=d + 9)
    qp, kp, vp, q, k, v = physical_inputs(w)
    for i in range(w.n_chunks):
        out, lse = _stepwise(w, qp, kp, vp, i)
        ref, ref_lse = oracle_all_rows(w.scaled(q_chunks=(i,)), _chunk_rows(w, qp, i), k, v, causal)
        assert max_abs(out, ref) <= TOL["f32"] and max_abs(lse, ref_lse) <= TOL["f32"]


def test_four_device_simulation_stepwise():
    """The glossary page's experiment as the four devices would run it: each
    device holds one query chunk and folds in one KV chunk per step."""
    w = synthetic.WORKLOADS["tiny_sim"]
    print("case ring step tiny_sim", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal=False)
    L = w.chunk
    for i in range(w.n_chunks):
        out, lse = _stepwise(w, qp, kp, vp, i)
        assert max_abs(out, ref[:, :, i * L:(i + 1) * L]) <= TOL["f32"]
        assert max_abs(lse, ref_lse[:, :, i * L:(i + 1) * L]) <= TOL["f32"]


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_ring_step_order_and_fused(layout):
    """Ring order, reversed and shuffled step orders and the fused ring agree up
    to rounding."""
    print(f"case ring step order {layout}", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, 2048, 8, 128, "bf16", True, layout, seed=31)
    qp, kp, vp, *_ = physical_inputs(w)
    i = 5
    base, base_lse = _stepwise(w, qp, kp, vp, i, out_dtype=torch.float32)
    fused, fused_lse = api.ring_forward(_chunk_rows(w, qp, i), kp, vp, seq=w.seq, n_chunks=w.n_chunks,
                                        layout=layout, causal=True, q_chunk_first=i, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert max_abs(base, fused) <= 1e-2 and max_abs(base_lse, fused_lse) <= 1e-3
    rng = np.random.default_rng(4)
    for order in (list(range(w.n_chunks))[::-1], rng.permutation(w.n_chunks).tolist()):
        out, lse = _stepwise(w, qp, kp, vp, i, order=order, out_dtype=torch.float32)
        assert max_abs(out, base) <= 1e-2 and max_abs(lse, base_lse) <= 1e-3


def test_skipped_step_leaves_state():
    """Contiguous causal: KV chunks after the query chunk are wholly in the
    future, so their steps return without touching the state."""
    print("case ring step skip", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, 1024, 4, 128, "bf16", True, "contiguous", seed=8)
    qp, kp, vp, *_ = physical_inputs(w)
    L, i = w.chunk, 1
    qi = _chunk_rows(w, qp, i)
    st = api.state_init(qi, kp)
    api.ring_step(st, qi, kp[:, :, i * L:(i + 1) * L], vp[:, :, i * L:(i + 1) * L], step=0, seq=w.seq,
                  n_chunks=w.n_chunks, layout="contiguous", causal=True, q_chunk=i)
    torch.cuda.synchronize()
    m0, l0, o0 = st.m.clone(), st.l.clone(), st.o.clone()
    for t in (2, 3):  # KV chunks 3 and 2: after the query chunk
        j = (i - t) % w.n_chunks
        assert j > i
        api.ring_step(st, qi, kp[:, :, j * L:(j + 1) * L], vp[:, :, j * L:(j + 1) * L], step=t, seq=w.seq,
                      n_chunks=w.n_chunks, layout="contiguous", causal=True, q_chunk=i)
    torch.cuda.synchronize()
    assert torch.equal(st.m, m0) and torch.equal(st.l, l0) and torch.equal(st.o, o0)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_rows_that_see_no_key_keep_their_state(dtype, d):
    """Striped causal, query chunk i: the step that brings KV chunk j > i is a
    masked pair in which query row 0 sees no key (key row k is visible from
    row p only when k <= p - 1).  That step must leave row 0's m, l and o
    exactly as they were, and m of every row whose maximum does not grow."""
    print(f"case ring step rows without keys {dtype} d={d}", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, 1024, 8, d, dtype, True, "striped", seed=21)
    qp, kp, vp, *_ = physical_inputs(w)
    L, i = w.chunk, 2
    qi = _chunk_rows(w, qp, i)
    st = api.state_init(qi, kp)
    # steps 0 .. i bring KV chunks i .. 0 (none after the query chunk)
    for t in range(i + 1):
        j = (i - t) % w.n_chunks
        api.ring_step(st, qi, kp[:, :, j * L:(j + 1) * L], vp[:, :, j * L:(j + 1) * L], step=t, seq=w.seq,
                      n_chunks=w.n_chunks, layout=w.layout, causal=True, q_chunk=i)
    torch.cuda.synchronize()
    m0, l0, o0 = st.m.clone(), st.l.clone(), st.o.clone()
    t = i + 1
    j = (i - t) % w.n_chunks
    assert j > i
    api.ring_step(st, qi, kp[:, :, j * L:(j + 1) * L], vp[:, :, j * L:(j + 1) * L], step=t, seq=w.seq,
                  n_chunks=w.n_chunks, layout=w.layout, causal=True, q_chunk=i)
    torch.cuda.synchronize()
    assert torch.equal(st.m[:, :, 0], m0[:, :, 0])
    assert torch.equal(st.l[:, :, 0], l0[:, :, 0])
    assert torch.equal(st.o[:, :, 0], o0[:, :, 0])
    # rows whose running maximum did not move hand m back bit for bit
    same = st.m == m0
    assert same[:, :, 0].all()
    assert (st.m >= m0).all()
