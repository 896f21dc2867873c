"""Pins for the backward oracle (CPU only): central finite differences of the
forward definition, invariants of the attention gradient, special cases with
closed forms, and agreement of the two routes (definition and ring order)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as BW
from oracle import layout as LY


def _inputs(seed, B, hq, hkv, Lq, Lk, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, hq, Lq, d))
    k = rng.standard_normal((B, hkv, Lk, d))
    v = rng.standard_normal((B, hkv, Lk, d))
    do = rng.standard_normal((B, hq, Lq, d))
    return q, k, v, do


def _numeric_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2)])
def test_gradient_matches_finite_differences(causal, hq, hkv):
    """Every entry of dq, dk, dv against central differences of
    sum(dout * attention(q, k, v)); positions make some rows see few keys."""
    q, k, v, do = _inputs(3, 1, hq, hkv, 5, 7, 4)
    q_pos = np.array([2, 4, 6, 1, 5])
    k_pos = np.arange(7)
    kw = dict(causal=causal, q_pos=q_pos, k_pos=k_pos)
    dq, dk, dv = BW.attention_backward_reference(q, k, v, do, **kw)
    f = lambda: BW.loss_and_forward(q, k, v, do, **kw)  # noqa: E731
    for x, g in ((q, dq), (k, dk), (v, dv)):
        assert np.max(np.abs(_numeric_grad(f, x) - g)) <= 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance_and_value_sum(causal):
    """Adding one vector to every key shifts each row's scores by a constant,
    which softmax ignores: the key gradients of a head sum to zero.  Each
    row's weights sum to one: the value gradients sum to the upstream
    gradients of the rows that see a key."""
    q, k, v, do = _inputs(5, 2, 4, 2, 9, 9, 8)
    dq, dk, dv = BW.attention_backward_reference(q, k, v, do, causal=causal)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    G = 2
    for g in range(2):
        want = do[:, g * G:(g + 1) * G].sum(axis=(1, 2))
        assert np.max(np.abs(dv[:, g].sum(axis=1) - want)) <= 1e-12


def test_single_key_and_uniform_rows():
    """Row 0 of a causal block sees key 0 only: P = 1, so dS = 0 there (dq row
    0 is zero) and dv of key 0 receives that row's dout in full.  With q = 0
    every visible weight is 1/n and dv of key j is the sum over visible rows
    of dout / n_row (closed form)."""
    q, k, v, do = _inputs(7, 1, 1, 1, 6, 6, 4)
    dq, dk, dv = BW.attention_backward_reference(q, k, v, do, causal=True)
    assert np.max(np.abs(dq[0, 0, 0])) <= 1e-15
    q0 = np.zeros_like(q)
    dq, dk, dv = BW.attention_backward_reference(q0, k, v, do, causal=True)
    want = np.zeros((6, 4))
    for r in range(6):
        want[: r + 1] += do[0, 0, r] / (r + 1)
    assert np.max(np.abs(dv[0, 0] - want)) <= 1e-14
    # and dk = 0 because dS multiplies q = 0
    assert np.max(np.abs(dk)) == 0.0


def _chunks(x, layout, S, N):
    return [x[:, :, LY.chunk_positions(layout, S, N, c)] for c in range(N)]


@pytest.mark.parametrize("layout", LY.LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("query_chunks", [[0, 1, 2, 3], [2]])
def test_ring_order_equals_definition(layout, causal, query_chunks):
    """The ring route (P from the forward's lse, blocks visited in ring order,
    KV gradients accumulated per chunk) equals the definition; with a subset
    of query chunks the KV gradients are those rows' share."""
    S, N, d = 32, 4, 8
    q, k, v, do = _inputs(13, 1, 4, 2, S, S, d)
    pos = [LY.chunk_positions(layout, S, N, c) for c in range(N)]
    qc, kc, vc, doc = (_chunks(x, layout, S, N) for x in (q, k, v, do))
    outs, lses = [], []
    for i in query_chunks:
        o, l = A.attention_reference(qc[i], k, v, causal=causal, q_pos=pos[i], k_pos=np.arange(S))
        outs.append(o)
        lses.append(l)
    dqs, dks, dvs = BW.ring_attention_backward([qc[i] for i in query_chunks], kc, vc,
                                               [doc[i] for i in query_chunks], outs, lses, pos,
                                               query_chunks=query_chunks, causal=causal)
    rows = np.concatenate([pos[i] for i in query_chunks])
    dq_ref, dk_ref, dv_ref = BW.attention_backward_reference(q[:, :, rows], k, v, do[:, :, rows], causal=causal,
                                                             q_pos=rows)
    got_dq = np.concatenate(dqs, axis=2)
    assert np.max(np.abs(got_dq - dq_ref)) <= 1e-12
    for j in range(N):
        assert np.max(np.abs(dks[j] - dk_ref[:, :, pos[j]])) <= 1e-12
        assert np.max(np.abs(dvs[j] - dv_ref[:, :, pos[j]])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_matches_torch_autograd(causal):
    """A library routine: torch's float64 scaled_dot_product_attention on the
    CPU, differentiated by autograd, with grouped heads and the causal rule
    written as a mask over arbitrary positions; every entry of dq, dk, dv."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, hq, hkv, Lq, Lk, d = 2, 4, 2, 33, 47, 16
    q, k, v, do = _inputs(11, B, hq, hkv, Lq, Lk, d)
    rng = np.random.default_rng(12)
    q_pos = np.sort(rng.choice(np.arange(Lk), size=Lq, replace=False))
    k_pos = np.arange(Lk)  # key 0 is visible to every query
    kw = dict(causal=causal, q_pos=q_pos, k_pos=k_pos)
    dq, dk, dv = BW.attention_backward_reference(q, k, v, do, **kw)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = None
    if causal:
        mask = torch.tensor(k_pos[None, :] <= q_pos[:, None])
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True)
    out.backward(torch.tensor(do, dtype=torch.float64))
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(got - want.numpy())) <= 1e-11
