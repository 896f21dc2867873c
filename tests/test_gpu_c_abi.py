"""The C ABI as a C program uses it: tests/c_abi/ring_fwd_example.c (C99,
hipMalloc / hipMemcpy and the ra_* calls of include/ringattn.h, no Python in
the process) runs the fused ring forward on seeded bf16 inputs that this test
writes in chunk-major order (a plain index gather over the oracle's position
maps); its out and lse are compared with the float64 oracle on every row.
The program also checks that a NULL input is rejected with a message and
that no workspace is asked for without split-KV."""
import os
import subprocess

import numpy as np
import pytest
import torch

import synthetic

from .parity_utils import TOL, gather_chunked, max_abs, oracle_all_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "ring_fwd_example")
LAYOUT_CODE = {"contiguous": 0, "striped": 1, "zigzag": 2}


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("layout,S,N,hq,hkv,causal", [("zigzag", 1024, 4, 4, 2, True),
                                                      ("striped", 768, 4, 2, 2, True),
                                                      ("contiguous", 640, 2, 2, 1, False)])
def test_c_program_ring_forward(tmp_path, layout, S, N, hq, hkv, causal):
    print(f"case C ABI program {layout} {S} {N} {hq}/{hkv} causal={causal}", flush=True)
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} not built: run __graft_entry__.build()")
    w = synthetic.Workload("t", 1, hq, hkv, S, N, 128, "bf16", causal, layout, seed=S + hq)
    q, k, v = synthetic.draw(w, device="cuda")
    qp, kp, vp = (gather_chunked(w, t) for t in (q, k, v))
    for name, t in (("q", qp), ("k", kp), ("v", vp)):
        _bits(t).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "meta.txt").write_text(f"1 {hq} {hkv} {S} {N} {LAYOUT_CODE[layout]} {int(causal)}\n")
    run = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    out = torch.from_numpy(np.fromfile(tmp_path / "out.bin", dtype=np.int16)).view(torch.bfloat16)
    out = out.reshape(1, hq, S, 128)
    lse = torch.from_numpy(np.fromfile(tmp_path / "lse.bin", dtype=np.float32)).reshape(1, hq, S)
    ref, ref_lse = oracle_all_rows(w, qp, k, v, causal)
    e_out, e_lse = max_abs(out, ref), max_abs(lse, ref_lse)
    print(f"  max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]
