"""Helpers shared by the GPU parity tests: inputs from ``synthetic``, the
oracle on all rows or on sampled rows, and error measures."""
from __future__ import annotations

import numpy as np
import torch

import synthetic
from oracle import attention as OA
from oracle import layout as OL

TOL = {"f32": 1e-4, "bf16": 2e-2}


def query_rows_positions(w: synthetic.Workload) -> np.ndarray:
    """Global position of every row of the (chunk-major) query buffer."""
    return np.concatenate([OL.chunk_positions(w.layout, w.seq, w.n_chunks, c) for c in w.query_chunks])


def gather_chunked(w: synthetic.Workload, x: torch.Tensor) -> torch.Tensor:
    """Logical [B, H, S, d] -> chunk-major order by a plain index gather over
    the oracle's own position maps (no library code involved)."""
    pos = torch.from_numpy(OL.all_positions(w.layout, w.seq, w.n_chunks)).to(x.device)
    return x.index_select(2, pos).contiguous()


def physical_inputs(w: synthetic.Workload, device="cuda"):
    """(q_phys, k_phys, v_phys, q_logical_or_rows, k_log, v_log) on the device.

    K and V are reordered to chunk-major order by the library's permutation
    kernel (they feed only the GPU path; the oracle reads the logical k, v).
    The query rows, which both sides read, come from a plain index gather over
    the oracle's position maps; the library's permutation of q is checked
    against that gather bit for bit here."""
    from exact_long_context_amd import api
    q, k, v = synthetic.draw(w, device=device)
    kp = api.to_chunked(k, w.layout, w.n_chunks)
    vp = api.to_chunked(v, w.layout, w.n_chunks)
    if w.q_chunks is None:
        qp = gather_chunked(w, q)
        assert torch.equal(api.to_chunked(q, w.layout, w.n_chunks), qp)
    else:
        qp = q
    return qp, kp, vp, q, k, v


def oracle_all_rows(w, q_rows_phys, k_log, v_log, causal):
    """Oracle out / lse for every row of the physical query buffer."""
    qpos = query_rows_positions(w)
    out, lse = OA.attention_reference(q_rows_phys.cpu(), k_log.cpu(), v_log.cpu(), causal=causal, q_pos=qpos,
                                      k_pos=np.arange(w.seq))
    return out, lse


def sample_rows(w: synthetic.Workload, n: int, seed: int):
    """Seeded (head, buffer row) sample; always includes the first and last row of
    every query segment of every query chunk."""
    L = w.chunk
    rng = np.random.default_rng(seed)
    rows = set()
    nq = len(w.query_chunks)
    seg = L // 2 if w.layout == "zigzag" else L
    for ci in range(nq):
        for s0 in range(0, L, seg):
            for r in (s0, s0 + seg - 1):
                rows.add(ci * L + r)
    rows = sorted(rows)
    out = []
    for r in rows:
        out.append((int(rng.integers(w.hq)), r))
    extra = n - len(out)
    if extra > 0:
        hs = rng.integers(w.hq, size=extra)
        rs = rng.integers(nq * L, size=extra)
        out += list(zip(hs.tolist(), rs.tolist()))
    return out


def oracle_sampled(w, samples, q_rows_phys, k_log, v_log, causal):
    """Oracle out / lse for the sampled (head, buffer row) pairs; each row sees
    all its visible keys.  K / V are converted to float64 one KV head at a time."""
    qpos = query_rows_positions(w)
    G = w.hq // w.hkv
    by_kv = {}
    for i, (h, r) in enumerate(samples):
        by_kv.setdefault(h // G, []).append(i)
    out = np.zeros((len(samples), w.d))
    lse = np.zeros(len(samples))
    qc = q_rows_phys.cpu()
    for g, idx in by_kv.items():
        kg = k_log[:, g:g + 1].cpu()
        vg = v_log[:, g:g + 1].cpu()
        hs = [samples[i][0] for i in idx]
        rs = [samples[i][1] for i in idx]
        qsel = torch.stack([qc[0, h, r] for h, r in zip(hs, rs)])[None, None]   # [1, 1, n, d]
        o, l = OA.attention_reference(qsel, kg, vg, causal=causal, q_pos=qpos[rs], k_pos=np.arange(w.seq))
        out[idx] = o[0, 0]
        lse[idx] = l[0, 0]
    return out, lse


def max_abs(a, b) -> float:
    a = a.detach().float().cpu().double().numpy() if hasattr(a, "detach") else np.asarray(a, dtype=np.float64)
    b = b.detach().float().cpu().double().numpy() if hasattr(b, "detach") else np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, a - b))
    return float(np.nanmax(d, initial=0.0)) if not np.isnan(d).any() else float("nan")
