"""GPU parity of the split-KV ring forward (``ra_ring_desc.kv_splits`` > 1):
every query tile's KV tiles, in ring order, cut into ranges walked by separate
workgroups and merged by log-sum-exp.  Compared element by element with the
float64 oracle (the plain definition) on small and ragged shapes, with more
ranges than some query tiles have tiles (empty ranges), on query-chunk subsets
(one GPU's share), in fp32 and bf16; and against the unsplit path."""
import pytest
import torch

import synthetic

from .parity_utils import TOL, max_abs, oracle_all_rows, physical_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402
from exact_long_context_amd import ringattn as ra  # noqa: E402


def _ring(w, qp, kp, vp, splits, out_dtype=None, q_first=0):
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                q_chunk_first=q_first, out_dtype=out_dtype, kv_splits=splits)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # layout, S, N, hq, hkv, batch, causal
    ("contiguous", 800, 4, 8, 2, 1, True),     # L = 200: ragged row and key tiles, GQA 4
    ("contiguous", 800, 4, 4, 4, 2, False),
    ("striped", 1536, 16, 4, 4, 1, True),      # L = 96
    ("zigzag", 1600, 8, 6, 3, 1, True),        # L = 200, s = 100, GQA 2
    ("zigzag", 64, 32, 2, 2, 1, True),         # L = 2: most ranges empty
    ("zigzag", 1024, 512, 2, 1, 1, True),      # 1024 KV segments
]


@pytest.mark.parametrize("splits", [2, 3, 7, ra.RA_MAX_KV_SPLITS])
@pytest.mark.parametrize("layout,S,N,hq,hkv,B,causal", CASES)
def test_split_bf16_every_row(layout, S, N, hq, hkv, B, causal, splits):
    print(f"case split bf16 {layout} S={S} N={N} hq={hq} hkv={hkv} B={B} causal={causal} splits={splits}",
          flush=True)
    w = synthetic.Workload("t", B, hq, hkv, S, N, 128, "bf16", causal, layout, seed=S + N + hq + 1)
    qp, kp, vp, q, k, v = physical_inputs(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    out32, lse = _ring(w, qp, kp, vp, splits, out_dtype=torch.float32)
    e_out, e_lse = max_abs(out32, ref), max_abs(lse, ref_lse)
    print(f"  max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]
    out16, lse16 = _ring(w, qp, kp, vp, splits)
    assert out16.dtype == torch.bfloat16
    assert max_abs(out16, ref) <= TOL["bf16"]
    assert torch.equal(lse16, lse)


@pytest.mark.parametrize("d", [16, 128])
@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("zigzag", True), ("striped", True)])
def test_split_fp32(d, layout, causal):
    print(f"case split fp32 d={d} {layout} {causal}", flush=True)
    w = synthetic.Workload("t", 1, 4, 2, 400, 4, d, "f32", causal, layout, seed=d + 5)
    qp, kp, vp, q, k, v = physical_inputs(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    for splits in (2, 5, 33):
        out, lse = _ring(w, qp, kp, vp, splits)
        assert max_abs(out, ref) <= TOL["f32"]
        assert max_abs(lse, ref_lse) <= TOL["f32"]


def test_tiny_simulation_split_fp32():
    """The pages' four-device fp32 experiment with split-KV."""
    w = synthetic.WORKLOADS["tiny_sim"]
    print("case split tiny_sim", flush=True)
    qp, kp, vp, q, k, v = physical_inputs(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal=False)
    for splits in (2, 4, 64):
        out, lse = _ring(w, qp, kp, vp, splits)
        assert max_abs(out, ref) <= TOL["f32"] and max_abs(lse, ref_lse) <= TOL["f32"]


@pytest.mark.parametrize("layout,causal", [("contiguous", True), ("striped", True), ("zigzag", True),
                                           ("contiguous", False)])
def test_split_query_chunk_subset(layout, causal):
    """One query chunk (one GPU's share): the case split-KV is for."""
    S, N = 2048, 8
    print(f"case split subset {layout} {causal}", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, S, N, 128, "bf16", causal, layout, seed=91)
    qp, kp, vp, q, k, v = physical_inputs(w)
    L = S // N
    for first, count, splits in ((0, 1, 4), (N - 1, 1, 16), (3, 2, 5)):
        qs = qp[:, :, first * L:(first + count) * L].contiguous()
        out, lse = _ring(w, qs, kp, vp, splits, out_dtype=torch.float32, q_first=first)
        ws = w.scaled(q_chunks=tuple(range(first, first + count)))
        ref, ref_lse = oracle_all_rows(ws, qs, k, v, causal)
        assert max_abs(out, ref) <= TOL["bf16"]
        assert max_abs(lse, ref_lse) <= TOL["bf16"]


def test_split_close_to_unsplit_and_deterministic():
    """Same result as the single-pass kernel up to rounding; a given split count
    gives bitwise-identical results on every call; 0 and 1 mean no split."""
    print("case split vs unsplit", flush=True)
    w = synthetic.Workload("t", 1, 8, 2, 4096, 4, 128, "bf16", True, "zigzag", seed=12)
    qp, kp, vp, *_ = physical_inputs(w)
    base, base_lse = _ring(w, qp, kp, vp, 0, out_dtype=torch.float32)
    one, one_lse = _ring(w, qp, kp, vp, 1, out_dtype=torch.float32)
    assert torch.equal(base, one) and torch.equal(base_lse, one_lse)
    for splits in (2, 8):
        a, la = _ring(w, qp, kp, vp, splits, out_dtype=torch.float32)
        b, lb = _ring(w, qp, kp, vp, splits, out_dtype=torch.float32)
        assert torch.equal(a, b) and torch.equal(la, lb)
        assert max_abs(a, base) <= 1e-2 and max_abs(la, base_lse) <= 1e-3
