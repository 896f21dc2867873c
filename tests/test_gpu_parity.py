"""GPU parity: every entry point of libringattn against the float64 oracle on
the same seeded inputs (small and ragged shapes; the full workload shapes are
in test_gpu_full.py).  Tolerances: max-abs 1e-4 for fp32 inputs, 2e-2 for bf16
inputs with fp32 accumulation; index work (permutations) bit-exact."""
import math

import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as OA
from oracle import layout as OL

from .parity_utils import TOL, gather_chunked, max_abs, oracle_all_rows, physical_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402
from exact_long_context_amd import ringattn as ra  # noqa: E402

DEV = "cuda"


def _ring(w, qp, kp, vp, out_dtype=None, q_first=0):
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                q_chunk_first=q_first, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


# ---------------------------------------------------------------------------
# the pages' own experiment
# ---------------------------------------------------------------------------

def test_tiny_simulation_fp32():
    w = synthetic.WORKLOADS["tiny_sim"]
    print("case tiny_sim", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = _ring(w, qp, kp, vp)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal=False)
    assert max_abs(out, ref) <= TOL["f32"]
    assert max_abs(lse, ref_lse) <= TOL["f32"]
    # the glossary page's verdict: allclose to full softmax attention at atol 1e-5
    full = torch.softmax(q[0, 0].cpu() @ k[0, 0].cpu().T / math.sqrt(16), dim=-1) @ v[0, 0].cpu()
    assert torch.allclose(out[0, 0].cpu(), full, atol=1e-5)


# ---------------------------------------------------------------------------
# permutation: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,S,N", [("contiguous", 96, 8), ("striped", 96, 8), ("zigzag", 96, 8),
                                        ("striped", 16, 16), ("zigzag", 64, 32)])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 16), (torch.bfloat16, 3),
                                     (torch.float32, 5)])
def test_permute_round_trip_bit_exact(layout, S, N, dtype, d):
    print(f"case permute {layout} {S} {N} {dtype} {d}", flush=True)
    x = synthetic.normal_draw((2, 3, S, d), seed=S + d, dtype=dtype, device=DEV)
    y = torch.empty_like(x)
    ra.ra_permute(layout, True, x, y, N)
    phys = torch.from_numpy(OL.all_positions(layout, S, N)).to(DEV)
    expect = x[:, :, phys]
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       expect.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    z = torch.empty_like(x)
    ra.ra_permute(layout, False, y, z, N)
    torch.cuda.synchronize()
    assert torch.equal(z, x)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("layout,S,N", [("contiguous", 96, 8), ("striped", 96, 8), ("zigzag", 96, 8),
                                        ("zigzag", 64, 32)])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 16), (torch.bfloat16, 3),
                                     (torch.float32, 5)])
def test_permute_strided_bshd_bit_exact(layout, S, N, dtype, d):
    """[B, S, H, d] buffers read and written in place through strided views,
    against the oracle's positions; a destination with padded rows keeps its
    padding."""
    print(f"case permute strided {layout} {S} {N} {dtype} {d}", flush=True)
    B, H = 2, 3
    x_bshd = synthetic.normal_draw((B, S, H, d), seed=7 * S + d, dtype=dtype, device=DEV)
    x = x_bshd.transpose(1, 2)                       # [B, H, S, d] view, row stride H d
    phys = torch.from_numpy(OL.all_positions(layout, S, N)).to(DEV)
    expect = x[:, :, phys].contiguous()
    y = api.to_chunked(x, layout, N)                 # strided source, contiguous result
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(expect))
    # padded destination rows: [B, H, S, d + 5] buffer, the first d columns written
    pad = torch.full((B, H, S, d + 5), -7.0, dtype=dtype, device=DEV)
    ra.ra_permute_strided(layout, True, x, pad[..., :d], N)
    torch.cuda.synchronize()
    assert torch.equal(_bits(pad[..., :d].contiguous()), _bits(expect))
    assert bool((pad[..., d:] == -7.0).all())
    # back to logical order straight into a [B, S, H, d] buffer
    z_bshd = torch.empty_like(x_bshd)
    ra.ra_permute_strided(layout, False, y, z_bshd.transpose(1, 2), N)
    back = api.from_chunked(pad[..., :d], layout, N)
    torch.cuda.synchronize()
    assert torch.equal(_bits(z_bshd), _bits(x_bshd))
    assert torch.equal(_bits(back), _bits(x.contiguous()))


def test_permute_many_heads_bit_exact():
    """More (batch, head) pairs than one grid dimension holds (65535)."""
    print("case permute 70000 heads", flush=True)
    x = synthetic.normal_draw((1, 70000, 4, 2), seed=3, dtype=torch.bfloat16, device=DEV)
    phys = torch.from_numpy(OL.all_positions("striped", 4, 2)).to(DEV)
    y = api.to_chunked(x, "striped", 2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(x[:, :, phys].contiguous()))


# ---------------------------------------------------------------------------
# the fused ring on small and ragged shapes, every row compared
# ---------------------------------------------------------------------------

SMALL = [
    # layout, S, N, hq, hkv, batch, causal
    ("contiguous", 800, 4, 8, 2, 1, True),     # L = 200: ragged row tiles and key tiles, GQA 4
    ("contiguous", 800, 4, 4, 4, 2, False),
    ("striped", 1536, 16, 4, 4, 1, True),      # L = 96
    ("striped", 1536, 16, 6, 3, 1, False),
    ("zigzag", 1600, 8, 6, 3, 1, True),        # L = 200, s = 100, GQA 2
    ("zigzag", 1024, 4, 8, 1, 2, True),        # GQA 8
    ("contiguous", 256, 1, 2, 2, 1, True),     # one chunk
    ("zigzag", 64, 32, 2, 2, 1, True),         # L = 2, s = 1
    ("striped", 64, 64, 2, 1, 1, True),        # L = 1
    ("zigzag", 1024, 512, 2, 1, 1, True),      # 1024 KV segments: the largest run table
    ("contiguous", 1024, 1024, 2, 2, 1, True),  # 1024 chunks of one token
    ("zigzag", 8192, 4, 8, 2, 1, True),        # 256 workgroups over 2 KV streams: blocks of 32 per XCD
]


@pytest.mark.parametrize("layout,S,N,hq,hkv,B,causal", SMALL)
def test_ring_bf16_small_every_row(layout, S, N, hq, hkv, B, causal):
    print(f"case ring bf16 {layout} S={S} N={N} hq={hq} hkv={hkv} B={B} causal={causal}", flush=True)
    w = synthetic.Workload("t", B, hq, hkv, S, N, 128, "bf16", causal, layout, seed=S + N + hq)
    qp, kp, vp, q, k, v = physical_inputs(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    out32, lse = _ring(w, qp, kp, vp, out_dtype=torch.float32)
    assert max_abs(out32, ref) <= TOL["bf16"]
    assert max_abs(lse, ref_lse) <= TOL["bf16"]
    out16, lse16 = _ring(w, qp, kp, vp)
    assert out16.dtype == torch.bfloat16
    assert max_abs(out16, ref) <= TOL["bf16"]
    assert torch.equal(lse16, lse)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True), ("striped", True),
                                           ("zigzag", True)])
def test_ring_bf16_query_chunk_subset(layout, causal):
    """Only some query chunks computed (one GPU's share)."""
    S, N = 1024, 8
    print(f"case ring subset {layout} {causal}", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, S, N, 128, "bf16", causal, layout, seed=77)
    qp, kp, vp, q, k, v = physical_inputs(w)
    L = S // N
    for first, count in ((0, 1), (N - 1, 1), (2, 3)):
        out, lse = _ring(w, qp[:, :, first * L:(first + count) * L].contiguous(), kp, vp, out_dtype=torch.float32,
                         q_first=first)
        ws = w.scaled(q_chunks=tuple(range(first, first + count)))
        ref, ref_lse = oracle_all_rows(ws, qp[:, :, first * L:(first + count) * L], k, v, causal)
        assert max_abs(out, ref) <= TOL["bf16"]
        assert max_abs(lse, ref_lse) <= TOL["bf16"]


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("zigzag", True), ("striped", True)])
def test_ring_fp32_small(d, layout, causal):
    print(f"case ring fp32 d={d} {layout} {causal}", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, 400, 4, d, "f32", causal, layout, seed=d)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = _ring(w, qp, kp, vp)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    assert max_abs(out, ref) <= TOL["f32"]
    assert max_abs(lse, ref_lse) <= TOL["f32"]


def test_sharp_scores_running_max():
    """Scaled queries (scores of tens to hundreds) exercise the running-max rescale."""
    print("case sharp", flush=True)
    w = synthetic.Workload("t", 1, 4, 4, 2048, 4, 128, "bf16", False, "contiguous", seed=5, q_scale=8.0)
    qp, kp, vp, q, k, v = physical_inputs(w)
    out, lse = _ring(w, qp, kp, vp, out_dtype=torch.float32)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, False)
    e_out, e_lse = max_abs(out, ref), max_abs(lse, ref_lse)
    print(f"  max-abs out {e_out:.3e} lse {e_lse:.3e} (largest lse {np.abs(ref_lse).max():.1f})", flush=True)
    assert e_out <= TOL["bf16"]
    assert e_lse <= TOL["bf16"]


@pytest.mark.parametrize("profile", ["ramp_fast", "ramp_slow", "falling", "jumps"])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_reference_updates(profile, causal):
    """Scores whose maximum keeps growing along the keys (in log2 units per key:
    0.1, 0.02, falling, and jumps of 12 every third tile of 64 keys) drive every
    reference update of the online softmax: exponentials above 1 kept while
    their sums stay small, a moved reference when they do not, and the exact
    maximum taken when the growth is abrupt."""
    print(f"case growing {profile} causal={causal}", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, 2048, 4, 128, "bf16", causal, "contiguous", seed=17)
    q, k, v = synthetic.draw(w, device=DEV)
    S, d = w.seq, w.d
    pos = torch.arange(S, device=DEV, dtype=torch.float32)
    if profile == "ramp_fast":
        t = 0.1 * pos
    elif profile == "ramp_slow":
        t = 0.02 * pos
    elif profile == "falling":
        t = 60.0 - 0.05 * pos
    else:
        t = 12.0 * torch.div(pos, 192, rounding_mode="floor") + 0.5 * torch.sin(pos)
    # q = 0.5 + noise, k = (t / (0.5 c d)) + noise: c q.k is about t (log2 units)
    c = (1.0 / math.sqrt(d)) / math.log(2.0)
    q = (0.5 + 0.05 * q.float()).to(torch.bfloat16)
    k = ((t / (0.5 * c * d))[None, None, :, None] + 0.05 * k.float()).to(torch.bfloat16)
    kp = api.to_chunked(k, w.layout, w.n_chunks)
    vp = api.to_chunked(v, w.layout, w.n_chunks)
    qp = gather_chunked(w, q)
    out, lse = _ring(w, qp, kp, vp, out_dtype=torch.float32)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    assert max_abs(out, ref) <= TOL["bf16"]
    e_lse = max_abs(lse, ref_lse)
    print(f"  max-abs lse {e_lse:.3e} (largest lse {np.abs(np.asarray(ref_lse)).max():.1f})", flush=True)
    assert e_lse <= TOL["bf16"]


# ---------------------------------------------------------------------------
# chunk update, finalize, merge
# ---------------------------------------------------------------------------

def _rand_state(B, H, L, d, seed, empty_rows=True):
    m = synthetic.normal_draw((B, H, L), seed, device=DEV, std=2.0)
    l = synthetic.uniform_draw((B, H, L), seed + 1, device=DEV, lo=0.5, hi=4.0)
    o = synthetic.normal_draw((B, H, L, d), seed + 2, device=DEV)
    if empty_rows:
        m[:, :, ::7] = -math.inf
        l[:, :, ::7] = 0
        o[:, :, ::7] = 0
    return m, l, o


CHUNK_CASES = [
    # dtype, d, B, hq, hkv, lq, lk, causal, delta
    ("bf16", 128, 1, 4, 4, 200, 136, False, 0),
    ("bf16", 128, 2, 8, 2, 130, 130, True, 0),
    ("bf16", 128, 1, 4, 1, 64, 300, True, 170),
    ("bf16", 128, 1, 2, 2, 100, 100, True, -30),
    ("bf16", 128, 1, 2, 2, 70, 40, True, 1000),
    ("bf16", 128, 1, 6, 3, 1, 1, False, 0),
    ("f32", 16, 1, 2, 1, 37, 53, True, 5),
    ("f32", 64, 2, 2, 2, 65, 64, False, 0),
    ("f32", 128, 1, 2, 2, 33, 33, True, -3),
]


@pytest.mark.parametrize("dt,d,B,hq,hkv,lq,lk,causal,delta", CHUNK_CASES)
def test_chunk_fwd_updates_state_like_oracle(dt, d, B, hq, hkv, lq, lk, causal, delta):
    print(f"case chunk {dt} d={d} B={B} hq={hq} hkv={hkv} lq={lq} lk={lk} causal={causal} delta={delta}",
          flush=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q = synthetic.normal_draw((B, hq, lq, d), 1, dtype=tdt, device=DEV)
    k = synthetic.normal_draw((B, hkv, lk, d), 2, dtype=tdt, device=DEV)
    v = synthetic.normal_draw((B, hkv, lk, d), 3, dtype=tdt, device=DEV)
    m0, l0, o0 = _rand_state(B, hq, lq, d, seed=lq + lk)
    st = api.ChunkState(q)
    st.m.copy_(m0), st.l.copy_(l0), st.o.copy_(o0)
    api.chunk_forward(st, q, k, v, causal=causal, delta=delta)
    out, lse = api.finalize(st, q, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rm, rl, ro = OA.chunk_update(m0.cpu(), l0.cpu(), o0.cpu(), q.cpu(), k.cpu(), v.cpu(), causal=causal, delta=delta)
    rout, rlse = OA.finalize(rm, rl, ro)
    tol = TOL[dt]
    assert max_abs(st.m, rm) <= tol
    assert max_abs(out, rout) <= tol
    assert max_abs(lse, rlse) <= tol
    # the state itself: l and o relative to the common max
    assert max_abs(st.l, rl) <= tol * max(1.0, float(np.max(rl)))


def test_chunk_steps_then_finalize_equals_ring():
    """The per-step path (state init, one ra_chunk_fwd per schedule pair,
    finalize) equals the fused ring."""
    S, N, layout = 1600, 8, "zigzag"
    print("case stepwise", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, S, N, 128, "bf16", True, layout, seed=9)
    qp, kp, vp, q, k, v = physical_inputs(w)
    fused, fused_lse = _ring(w, qp, kp, vp, out_dtype=torch.float32)
    L = S // N
    desc = ra.ring_desc(qp, kp, vp, seq=S, n_chunks=N, layout=layout, causal=True)
    outs, lses = [], []
    for i in range(N):
        qi = qp[:, :, i * L:(i + 1) * L]
        st = api.state_init(qi, kp)
        for t in ra.ra_ring_schedule(desc, i):
            if t["kind"] == ra.RA_SKIP:
                continue
            sub = st.__class__.__new__(st.__class__)
            qs = slice(t["q_row0"], t["q_row0"] + t["q_len"])
            sub.m, sub.l, sub.o = st.m[:, :, qs], st.l[:, :, qs], st.o[:, :, qs]
            r0 = t["kv_chunk"] * L + t["kv_row0"]
            api.chunk_forward(sub, qi[:, :, qs], kp[:, :, r0:r0 + t["kv_len"]], vp[:, :, r0:r0 + t["kv_len"]],
                              causal=True, delta=t["delta"])
        o, l = api.finalize(st, qi, out_dtype=torch.float32)
        outs.append(o)
        lses.append(l)
    step = torch.cat(outs, dim=2)
    step_lse = torch.cat(lses, dim=2)
    torch.cuda.synchronize()
    # both paths round P to bf16, but relative to different reference maxima
    # (the stepwise state is renormalised to the exact maximum after every
    # step), so they agree to about the bf16 rounding of P, 2^-9 relative
    assert max_abs(step, fused) <= 1e-2
    assert max_abs(step_lse, fused_lse) <= 1e-2
    ref, ref_lse = oracle_all_rows(w, qp, k, v, True)
    assert max_abs(step, ref) <= TOL["bf16"]


def test_finalize_like_oracle():
    print("case finalize", flush=True)
    B, H, L, d = 2, 3, 77, 128
    m, l, o = _rand_state(B, H, L, d, seed=4)
    q = torch.empty(B, H, L, d, dtype=torch.bfloat16, device=DEV)
    st = api.ChunkState(q)
    st.m.copy_(m), st.l.copy_(l), st.o.copy_(o)
    for odt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        out, lse = api.finalize(st, q, out_dtype=odt)
        torch.cuda.synchronize()
        rout, rlse = OA.finalize(m.cpu(), l.cpu(), o.cpu())
        assert max_abs(out, rout) <= tol
        assert max_abs(lse, rlse) <= 1e-5
        assert torch.isinf(lse[:, :, ::7]).all() and (out[:, :, ::7] == 0).all()


@pytest.mark.parametrize("inplace", [None, "a", "b"])
def test_merge_like_oracle(inplace):
    print(f"case merge {inplace}", flush=True)
    B, H, L, d = 2, 4, 93, 64
    la = synthetic.normal_draw((B, H, L), 1, device=DEV, std=30.0)
    lb = synthetic.normal_draw((B, H, L), 2, device=DEV, std=30.0)
    la[:, :, ::5] = -math.inf
    lb[:, :, ::3] = -math.inf
    oa = synthetic.normal_draw((B, H, L, d), 3, device=DEV)
    ob = synthetic.normal_draw((B, H, L, d), 4, device=DEV)
    rl, ro = OA.lse_merge(la.cpu(), oa.cpu(), lb.cpu(), ob.cpu())
    if inplace == "a":
        lo, oo = api.merge(la, oa, lb, ob, lse_out=la, o_out=oa)
    elif inplace == "b":
        lo, oo = api.merge(la, oa, lb, ob, lse_out=lb, o_out=ob)
    else:
        lo, oo = api.merge(la, oa, lb, ob)
    torch.cuda.synchronize()
    assert max_abs(lo, rl) <= 1e-4 and max_abs(oo, ro) <= 1e-5


def test_merge_of_split_kv_equals_full():
    """Two halves of the keys, each finalized, merged by lse: equals the whole."""
    print("case split-kv merge", flush=True)
    q = synthetic.normal_draw((1, 4, 96, 128), 1, dtype=torch.bfloat16, device=DEV)
    k = synthetic.normal_draw((1, 4, 300, 128), 2, dtype=torch.bfloat16, device=DEV)
    v = synthetic.normal_draw((1, 4, 300, 128), 3, dtype=torch.bfloat16, device=DEV)
    parts = []
    for sl in (slice(0, 137), slice(137, 300)):
        st = api.state_init(q, k)
        api.chunk_forward(st, q, k[:, :, sl].contiguous(), v[:, :, sl].contiguous())
        parts.append(api.finalize(st, q, out_dtype=torch.float32))
    (oa, la), (ob, lb) = parts
    lse, o = api.merge(la, oa, lb, ob)
    torch.cuda.synchronize()
    ref, ref_lse = OA.attention_reference(q.cpu(), k.cpu(), v.cpu())
    assert max_abs(o, ref) <= TOL["bf16"] and max_abs(lse, ref_lse) <= TOL["bf16"]


def test_ring_is_deterministic():
    print("case determinism", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, 2048, 4, 128, "bf16", True, "zigzag", seed=3)
    qp, kp, vp, *_ = physical_inputs(w)
    a, la = _ring(w, qp, kp, vp)
    b, lb = _ring(w, qp, kp, vp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_strided_inputs():
    """Non-contiguous head / row strides (a [B, S, H, d] buffer viewed as [B, H, S, d])."""
    print("case strided", flush=True)
    B, S, H, d, N = 1, 512, 4, 128, 4
    base_q = synthetic.normal_draw((B, S, H, d), 1, dtype=torch.bfloat16, device=DEV)
    base_k = synthetic.normal_draw((B, S, H, d), 2, dtype=torch.bfloat16, device=DEV)
    base_v = synthetic.normal_draw((B, S, H, d), 3, dtype=torch.bfloat16, device=DEV)
    q, k, v = (t.transpose(1, 2) for t in (base_q, base_k, base_v))
    out, lse = api.ring_forward(q, k, v, seq=S, n_chunks=N, layout="contiguous", causal=True,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ref_lse = OA.attention_reference(q.cpu(), k.cpu(), v.cpu(), causal=True)
    assert max_abs(out, ref) <= TOL["bf16"] and max_abs(lse, ref_lse) <= TOL["bf16"]


@pytest.mark.parametrize("splits", [0, 3])
def test_strided_inputs_and_outputs(splits):
    """Strided q / k / v / out views and a padded lse, single-pass and split-KV
    (the split merge writes through the same out / lse strides)."""
    print(f"case strided out splits={splits}", flush=True)
    B, S, H, d, N = 2, 768, 4, 128, 4
    base = [synthetic.normal_draw((B, S, H, d), 11 + i, dtype=torch.bfloat16, device=DEV) for i in range(3)]
    q, k, v = (t.transpose(1, 2) for t in base)
    out_base = torch.full((B, S, H, d), 7.0, dtype=torch.float32, device=DEV)
    out = out_base.transpose(1, 2)
    lse_base = torch.full((B, H, S + 40), 7.0, dtype=torch.float32, device=DEV)
    lse = lse_base[:, :, :S]
    desc = ra.ring_desc(q, k, v, seq=S, n_chunks=N, layout="striped", causal=True, out=out, lse=lse,
                        kv_splits=splits)
    nws = ra.ra_ring_workspace_bytes(desc)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    pos = torch.from_numpy(OL.all_positions("striped", S, N))
    qp = q.index_select(2, pos.to(DEV)).contiguous()
    kp = api.to_chunked(k.contiguous(), "striped", N)
    vp = api.to_chunked(v.contiguous(), "striped", N)
    # physical inputs copied back into strided views of the same shape
    qs, ks, vs = (torch.empty_like(b).transpose(1, 2) for b in base)
    qs.copy_(qp), ks.copy_(kp), vs.copy_(vp)
    ra.ra_ring_fwd(desc, qs, ks, vs, out, lse, ws, nws)
    torch.cuda.synchronize()
    ref, ref_lse = OA.attention_reference(qp.cpu(), k.cpu(), v.cpu(), causal=True, q_pos=pos.numpy(),
                                          k_pos=np.arange(S))
    assert max_abs(out, ref) <= TOL["bf16"] and max_abs(lse, ref_lse) <= TOL["bf16"]
    assert torch.all(lse_base[:, :, S:] == 7.0)  # padding untouched
