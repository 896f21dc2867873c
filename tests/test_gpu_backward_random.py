"""Seeded random configurations through ra_ring_bwd, element by element
against the float64 backward oracle: layout, chunk count and length (ragged
32-row steps, 32-key and 256-key tiles), heads and grouping, batch, causal or
not, and a random range of query chunks; the library's own forward output and
lse feed the backward."""
import numpy as np
import pytest
import torch

import synthetic

from .test_gpu_backward import _check, _oracle, _setup

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_long_context_amd import api  # noqa: E402


def _config(seed):
    rng = np.random.default_rng(2000 + seed)
    layout = ["contiguous", "striped", "zigzag"][int(rng.integers(3))]
    N = int(rng.choice([1, 2, 3, 4, 6]))
    L = int(rng.integers(1, 160)) * (2 if layout == "zigzag" else 1)
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([1, 2]))
    causal = bool(rng.integers(2))
    first = int(rng.integers(N))
    count = int(rng.integers(1, N - first + 1))
    return layout, N, L, hkv * G, hkv, B, causal, first, count


@pytest.mark.parametrize("seed", range(12))
def test_backward_random_config(seed):
    layout, N, L, hq, hkv, B, causal, first, count = _config(seed)
    qc = tuple(range(first, first + count))
    print(f"case bwd random {seed}: {layout} N={N} L={L} hq={hq} hkv={hkv} B={B} causal={causal} q_chunks={qc}",
          flush=True)
    w = synthetic.Workload("t", B, hq, hkv, N * L, N, 128, "bf16", causal, layout, seed=seed + 70,
                           q_chunks=None if count == N else qc)
    qp, kp, vp, k, v, do = _setup(w, seed_do=seed + 90)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=N, layout=layout, causal=causal,
                                q_chunk_first=w.query_chunks[0])
    dq, dk, dv = api.ring_backward(qp, kp, vp, out, do, lse, seq=w.seq, n_chunks=N, layout=layout, causal=causal,
                                   q_chunk_first=w.query_chunks[0])
    torch.cuda.synchronize()
    _, _, rdq, rdk, rdv = _oracle(w, qp, k, v, do)
    _check(w, (dq, dk, dv), (rdq, rdk, rdv))
