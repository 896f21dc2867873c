"""Helpers shared by the GPU parity tests: inputs from ``synthetic``, the
oracle on all rows or on sampled rows, and error measures."""
from __future__ import annotations

import concurrent.futures
import os

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


def sample_rows(w: synthetic.Workload, n: int, seed: int, every_head_ends: bool = False):
    """Seeded (head, buffer row) sample of about n pairs; always includes the
    first and last row of every query segment of every query chunk (for one
    random head, or for every head with every_head_ends), the rest drawn
    evenly over the query segments, heads uniform."""
    L = w.chunk
    rng = np.random.default_rng(seed)
    nq = len(w.query_chunks)
    seg = L // 2 if w.layout == "zigzag" else L
    segs = [(ci * L + s0, seg) for ci in range(nq) for s0 in range(0, L, seg)]
    out = []
    for r0, ln in segs:
        for r in (r0, r0 + ln - 1):
            if every_head_ends:
                out += [(h, r) for h in range(w.hq)]
            else:
                out.append((int(rng.integers(w.hq)), r))
    extra = n - len(out)
    if extra > 0:
        per = -(-extra // len(segs))
        for r0, ln in segs:
            hs = rng.integers(w.hq, size=per)
            rs = r0 + rng.integers(ln, size=per)
            out += list(zip(hs.tolist(), rs.tolist()))
    return out


def oracle_threads() -> int:
    """Worker threads for the oracle: the host's cores, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_threaded(fn, items):
    """fn over items in a pool of oracle_threads() threads, each numpy call
    single-threaded (numpy releases the GIL in its loops and in BLAS)."""
    import threadpoolctl
    with threadpoolctl.threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(oracle_threads()) as ex:
            return list(ex.map(fn, items))


def oracle_sampled(w, samples, q_rows_phys, k_log, v_log, causal):
    """Oracle out / lse for the sampled (head, buffer row) pairs; each row sees
    all its visible keys.  Rows are grouped by KV head and, for causal
    workloads, by how far their visible keys reach (keys are in logical order,
    so the keys past the group's last query position, which none of its rows
    sees, are left out); the groups run in parallel threads."""
    qpos = query_rows_positions(w)
    G = w.hq // w.hkv
    qc = q_rows_phys.cpu()
    kc, vc = k_log.cpu(), v_log.cpu()
    groups = {}
    for i, (h, r) in enumerate(samples):
        reach = (int(qpos[r]) * 8 // w.seq) if causal else 0   # eighths of the sequence
        groups.setdefault((h // G, reach), []).append(i)

    def one(item):
        (g, _), idx = item
        hs = [samples[i][0] for i in idx]
        rs = [samples[i][1] for i in idx]
        kmax = int(qpos[rs].max()) + 1 if causal else w.seq
        qsel = torch.stack([qc[0, h, r] for h, r in zip(hs, rs)])[None, None]   # [1, 1, n, d]
        o, l = OA.attention_reference(qsel, kc[:, g:g + 1, :kmax], vc[:, g:g + 1, :kmax], causal=causal,
                                      q_pos=qpos[rs], k_pos=np.arange(kmax))
        return idx, o[0, 0], l[0, 0]

    out = np.zeros((len(samples), w.d))
    lse = np.zeros(len(samples))
    for idx, o, l in run_threaded(one, sorted(groups.items())):
        out[idx] = o
        lse[idx] = l
    return out, lse


def oracle_heads(w, heads, q_rows_phys, k_log, v_log, causal):
    """Oracle out / lse of every query row of the given query heads, one head
    per thread: {head: (out [rows, d], lse [rows])}."""
    qpos = query_rows_positions(w)
    G = w.hq // w.hkv
    qc, kc, vc = q_rows_phys.cpu(), k_log.cpu(), v_log.cpu()

    def one(h):
        g = h // G
        o, l = OA.attention_reference(qc[:, h:h + 1], kc[:, g:g + 1], vc[:, g:g + 1], causal=causal, q_pos=qpos,
                                      k_pos=np.arange(w.seq))
        return h, o[0, 0], l[0, 0]

    return {h: (o, l) for h, o, l in run_threaded(one, list(heads))}


def max_abs(a, b) -> float:
    a = a.detach().float().cpu().double().numpy() if hasattr(a, "detach") else np.asarray(a, dtype=np.float64)
    b = b.detach().float().cpu().double().numpy() if hasattr(b, "detach") else np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, a - b))
    return float(np.nanmax(d, initial=0.0)) if not np.isnan(d).any() else float("nan")
