"""Seeded random configurations through every forward entry point, each
compared element by element with the float64 oracle: layout, chunk count and
length (odd ones too, where the layout allows), heads and grouping, batch,
causal or not, input dtype, and the split-KV range count; the step-by-step
path runs on one query chunk of each."""
import numpy as np
import pytest
import torch

import synthetic

from .parity_utils import TOL, max_abs, oracle_all_rows, physical_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    layout = ["contiguous", "striped", "zigzag"][int(rng.integers(3))]
    N = int(rng.choice([1, 2, 3, 5, 8]))
    L = int(rng.integers(1, 90)) * (2 if layout == "zigzag" else 1)
    hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([1, 2]))
    causal = bool(rng.integers(2))
    f32 = bool(rng.integers(4) == 0)
    d = int(rng.choice([16, 64])) if f32 else 128
    splits = int(rng.choice([0, 2, 5]))
    return layout, N, L, hkv * G, hkv, B, causal, f32, d, splits


@pytest.mark.parametrize("seed", range(24))
def test_random_config(seed):
    layout, N, L, hq, hkv, B, causal, f32, d, splits = _config(seed)
    print(f"case random {seed}: {layout} N={N} L={L} hq={hq} hkv={hkv} B={B} causal={causal} "
          f"{'f32' if f32 else 'bf16'} d={d} splits={splits}", flush=True)
    w = synthetic.Workload("t", B, hq, hkv, N * L, N, d, "f32" if f32 else "bf16", causal, layout, seed=seed + 40)
    qp, kp, vp, q, k, v = physical_inputs(w)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    tol = TOL["f32" if f32 else "bf16"]
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=N, layout=layout, causal=causal,
                                out_dtype=torch.float32, kv_splits=splits)
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= tol and max_abs(lse, ref_lse) <= tol
    i = seed % N
    qi = qp[:, :, i * L:(i + 1) * L].contiguous()
    out_s, lse_s = api.ring_forward_stepwise(qi, kp, vp, seq=w.seq, n_chunks=N, layout=layout, causal=causal,
                                             q_chunk=i, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert max_abs(out_s, ref[:, :, i * L:(i + 1) * L]) <= tol
    assert max_abs(lse_s, ref_lse[:, :, i * L:(i + 1) * L]) <= tol
