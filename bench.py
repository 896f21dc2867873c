"""Throughput of the ring-ordered exact attention forward on one MI355X.

A step is one fused ``ra_ring_fwd`` over the whole workload: every ring step
of the query chunk(s), causal classification and skipping, the online-softmax
chunk updates, and the final normalization with lse.  Inputs are resident in
HBM in chunk-major order before timing starts (the layout permutation is the
data pipeline's job and is not timed).

Default workload: one GPU's share of a 1M-token causal layer, zig-zag layout
(32 chunks of 32768 tokens; one query chunk of 32 query heads against all 32
KV chunks of 8 KV heads, d = 128, bf16).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 (matrix and packed vector)
# the sources the forward kernel is compiled from (the traffic record is keyed by their hash)
# the forward kernel's sources and the build script that holds its compiler flags
KERNEL_SOURCES = [os.path.join(ROOT, "exact_long_context_amd", "csrc", f)
                  for f in ("attn_fwd_bf16.hip", "fwd_common.h", "kernels.h", "schedule.h")] + \
                 [os.path.join(ROOT, "exact_long_context_amd", "build.py")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_fwd_bf16_zigzag_1m_gqa.json")
TRAFFIC_WORKLOAD = "zigzag_1m_gqa"   # the workload the counter runs were taken on


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(tasks) -> int:
    """Visible (query, key) pairs of a schedule, from each task's kind and offset."""
    tot = 0
    for t in tasks:
        if t["kind"] == 0:
            tot += t["q_len"] * t["kv_len"]
        elif t["kind"] == 1:
            p = np.arange(t["q_len"], dtype=np.int64)
            tot += int(np.clip(p + t["delta"] + 1, 0, t["kv_len"]).sum())
    return tot


def workload_flop(w, ra) -> float:
    import torch
    q = torch.empty(1, w.hq, len(w.query_chunks) * w.chunk, w.d, dtype=torch.bfloat16)
    k = torch.empty(1, w.hkv, w.seq, w.d, dtype=torch.bfloat16)
    desc = ra.ring_desc(q, k, k, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                        q_chunk_first=w.query_chunks[0], q_chunk_count=len(w.query_chunks))
    pairs = sum(visible_pairs(ra.ra_ring_schedule(desc, i)) for i in w.query_chunks)
    return 4.0 * w.d * w.hq * w.batch * pairs


def launch_stats(ms):
    """Mean, median, min and max of per-launch times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"n": int(a.size), "mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "min": round(float(a.min()), 5), "max": round(float(a.max()), 5)}


def time_launches(fn, stream, n, warmup, torch):
    """Per-launch times of n back-to-back calls of fn (after `warmup` untimed
    ones): HIP events recorded on the launch stream between the calls, with a
    device synchronization on both sides of the timed run."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def workload_inputs(w, api, torch):
    """Device inputs in chunk-major order (the permutation is the library's)."""
    import synthetic
    q, k, v = synthetic.draw(w, device="cuda")
    kp = api.to_chunked(k, w.layout, w.n_chunks)
    vp = api.to_chunked(v, w.layout, w.n_chunks)
    qp = api.to_chunked(q, w.layout, w.n_chunks) if w.q_chunks is None else q
    return qp, kp, vp


def time_workload(w, steps, warmup, api, torch, kv_splits=0):
    """Per-launch times (ms) of ra_ring_fwd on the workload, bf16 (or fp32) out plus lse."""
    qp, kp, vp = workload_inputs(w, api, torch)
    out = torch.empty(qp.shape, dtype=qp.dtype, device="cuda")
    lse = torch.empty(qp.shape[:3], dtype=torch.float32, device="cuda")
    from exact_long_context_amd import ringattn as ra
    desc = ra.ring_desc(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                        q_chunk_first=w.query_chunks[0], out=out, lse=lse, kv_splits=kv_splits)
    nws = ra.ra_ring_workspace_bytes(desc)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    return time_launches(lambda: ra.ra_ring_fwd(desc, qp, kp, vp, out, lse, ws, nws, stream=stream), stream, steps,
                         warmup, torch)


def computed_tile_flop(w, ra):
    """FLOP the forward kernel executes, masked parts of its tiles included:
    every workgroup computes tiles of 64 keys for all its query rows (64 rows
    of 4 heads with 4 or more query heads per KV head, 128 rows of 2 heads
    with 2, else 256 rows of one head), over the keys up to the last one its
    last row sees."""
    import torch
    G = w.hq // w.hkv
    hpw = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    R = 256 // hpw
    q = torch.empty(1, w.hq, len(w.query_chunks) * w.chunk, w.d, dtype=torch.bfloat16)
    k = torch.empty(1, w.hkv, w.seq, w.d, dtype=torch.bfloat16)
    desc = ra.ring_desc(q, k, k, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                        q_chunk_first=w.query_chunks[0], q_chunk_count=len(w.query_chunks))
    pairs = 0
    for i in w.query_chunks:
        for t in ra.ra_ring_schedule(desc, i):
            p_hi = np.minimum(np.arange(0, t["q_len"], R, dtype=np.int64) + R, t["q_len"]) - 1
            k_end = np.clip(p_hi + t["delta"] + 1, 0, t["kv_len"]) if w.causal else np.full(p_hi.shape, t["kv_len"])
            pairs += int(((k_end + 63) // 64).sum()) * 64 * R
    return 4.0 * w.d * w.hq * w.batch * pairs


def time_backward(w, steps, warmup, api, torch):
    """Per-launch times (ms) of ra_ring_bwd on the workload: the library's
    forward output and lse (not timed) and a seeded upstream gradient as
    inputs, inputs and outputs resident in HBM."""
    import synthetic
    from exact_long_context_amd import ringattn as ra
    qp, kp, vp = workload_inputs(w, api, torch)
    out, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                q_chunk_first=w.query_chunks[0])
    dout = synthetic.normal_draw(qp.shape, w.seed + 101, dtype=torch.bfloat16, device="cuda")
    dq = torch.empty(qp.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(kp.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(vp.shape, dtype=torch.float32, device="cuda")
    desc = ra.ring_desc(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                        q_chunk_first=w.query_chunks[0], out=out, lse=lse)
    nws = ra.ra_ring_bwd_workspace_bytes(desc)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    return time_launches(lambda: ra.ra_ring_bwd(desc, qp, kp, vp, out, dout, lse, dq, dk, dv, ws, nws,
                                                stream=stream), stream, steps, warmup, torch)


def time_memory_kernels(w, torch, reps=10):
    """The memory-bound entry points at the workload's shapes: the layout
    permutation of one K tensor (logical -> chunk-major and back), and state
    initialization, finalize and the lse merge on the query chunk(s)' state.
    Algorithmic bytes are what each call must read and write once; HIP events
    on the launch stream around `reps` calls."""
    from exact_long_context_amd import ringattn as ra
    B, Hq, Hkv, d = w.batch, w.hq, w.hkv, w.d
    rows = len(w.query_chunks) * w.chunk
    stream = torch.cuda.current_stream()
    res = {}

    def timed(name, fn, nbytes):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bytes": int(nbytes), "gb_per_s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"  {name}: {ms:.3f} ms  {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS * 100:.1f}% of HBM peak)")

    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    timed("torch device copy, 1 GiB (practical ceiling)", lambda: b.copy_(a), 2 * a.numel() * 4)
    del a, b
    k = torch.empty(B, Hkv, w.seq, d, dtype=torch.bfloat16, device="cuda").normal_()
    kc = torch.empty_like(k)
    nb = 2 * k.numel() * k.element_size()
    timed("ra_permute to chunk-major (K)", lambda: ra.ra_permute(w.layout, True, k, kc, w.n_chunks, stream), nb)
    timed("ra_permute to logical (K)", lambda: ra.ra_permute(w.layout, False, kc, k, w.n_chunks, stream), nb)
    kv = k.view(B, w.seq, Hkv, d).transpose(1, 2)   # the same bytes read as a [B, S, H, d] buffer
    timed("ra_permute_strided [B, S, H, d] to chunk-major (K)",
          lambda: ra.ra_permute_strided(w.layout, True, kv, kc, w.n_chunks, stream), nb)
    del k, kc, kv
    torch.cuda.empty_cache()

    q = torch.empty(B, Hq, rows, d, dtype=torch.bfloat16, device="cuda")
    m = torch.empty(B, Hq, rows, dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    o = torch.empty(B, Hq, rows, d, dtype=torch.float32, device="cuda")
    desc = ra.attn_desc(q, q, q, ml=m, o=o)
    n_o, n_r = o.numel() * 4, m.numel() * 4
    timed("ra_state_init", lambda: ra.ra_state_init(desc, m, l, o, stream), n_o + 2 * n_r)
    o.normal_()
    l.uniform_(1.0, 2.0)
    m.normal_()
    out = torch.empty_like(q)
    lse = torch.empty_like(m)
    fdesc = ra.attn_desc(q, q, q, out=out, ml=m, o=o)
    timed("ra_finalize", lambda: ra.ra_finalize(fdesc, m, l, o, out, lse, stream),
          n_o + 2 * n_r + out.numel() * 2 + n_r)
    o2 = torch.randn_like(o)
    lse2 = torch.randn_like(m)
    o3 = torch.empty_like(o)
    lse3 = torch.empty_like(m)
    mdesc = ra.ra_attn_desc()
    mdesc.batch, mdesc.hq, mdesc.hkv, mdesc.lq, mdesc.lk, mdesc.d = B, Hq, Hq, rows, rows, d
    mdesc.in_dtype = mdesc.out_dtype = ra.RA_F32
    mdesc.q = mdesc.k = mdesc.v = mdesc.out = ra.strides_of(o)
    mdesc.ml = ra.ra_strides(m.stride(0), m.stride(1), 1)
    mdesc.o = ra.strides_of(o)
    timed("ra_merge", lambda: ra.ra_merge(mdesc, lse, o, lse2, o2, lse3, o3, stream), 3 * (n_o + n_r))
    del q, m, l, o, out, lse, o2, lse2, o3, lse3
    torch.cuda.empty_cache()
    return res


def time_stepwise(w, steps, warmup, api, torch):
    """The workload's query chunk as one device of the ring runs it: state
    init, one ra_ring_step per ring step (each given only its KV chunk, a view
    of the resident chunk-major K / V standing for the received buffer, the
    running state in HBM between steps), finalize.  Per-pass times (ms)."""
    import synthetic
    from exact_long_context_amd import ringattn as ra
    assert len(w.query_chunks) == 1
    i = w.query_chunks[0]
    q, k, v = synthetic.draw(w, device="cuda")
    kp = api.to_chunked(k, w.layout, w.n_chunks)
    vp = api.to_chunked(v, w.layout, w.n_chunks)
    del k, v
    L = w.chunk
    st = api.ChunkState(q)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    adesc = ra.attn_desc(q, kp, vp, ml=st.m, o=st.o)
    fdesc = ra.attn_desc(q, q, q, out=out, ml=st.m, o=st.o)
    views = []
    for t in range(w.n_chunks):
        j = (i - t) % w.n_chunks
        kj, vj = kp[:, :, j * L:(j + 1) * L], vp[:, :, j * L:(j + 1) * L]
        d = ra.ring_desc(q, kj, vj, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                         q_chunk_first=i, q_chunk_count=1, lse=st.m)
        d.attn.o = ra.strides_of(st.o)
        views.append((t, d, kj, vj))
    stream = torch.cuda.current_stream()

    def one_pass():
        ra.ra_state_init(adesc, st.m, st.l, st.o, stream)
        for t, d, kj, vj in views:
            ra.ra_ring_step(d, t, q, kj, vj, st.m, st.l, st.o, stream)
        ra.ra_finalize(fdesc, st.m, st.l, st.o, out, lse, stream)

    return time_launches(one_pass, stream, steps, warmup, torch)


def split_kv_report(api, torch, steps=10):
    """One GPU's share of three workloads whose query tiles alone do not keep
    the chip busy (few query rows, or causal work that differs between query
    tiles): the single-pass ring forward against split-KV with the library's
    suggested number of KV ranges (partials merged by log-sum-exp)."""
    import synthetic
    from exact_long_context_amd import ringattn as ra
    res = {}
    for name, qc in (("mha_8k", 0), ("causal_striped_128k", 15), ("causal_contig_32k", 7)):
        w = synthetic.WORKLOADS[name].scaled(q_chunks=(qc,))
        fl = workload_flop(w, ra)
        q = torch.empty(w.batch, w.hq, w.chunk, w.d, dtype=torch.bfloat16)
        k = torch.empty(w.batch, w.hkv, w.seq, w.d, dtype=torch.bfloat16)
        hint = ra.ra_ring_kv_splits_hint(ra.ring_desc(q, k, k, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout,
                                                      causal=w.causal, q_chunk_first=qc))
        t1 = launch_stats(time_workload(w, steps, 2, api, torch, kv_splits=0))
        t2 = launch_stats(time_workload(w, steps, 2, api, torch, kv_splits=hint))
        m1, ms = t1["mean"], t2["mean"]
        res[f"{name} query chunk {qc}"] = {
            "kv_splits": hint, "ms_single_pass": t1, "ms_split": t2,
            "tflops_single_pass": round(fl / (m1 * 1e-3) / 1e12, 2), "tflops_split": round(fl / (ms * 1e-3) / 1e12, 2),
            "speedup": round(m1 / ms, 3)}
        log(f"  split-KV {name} chunk {qc}: {m1:.3f} ms -> {ms:.3f} ms with {hint} ranges ({m1 / ms:.2f}x)")
        torch.cuda.empty_cache()
    return res


def balance_report(w, api, torch, reps=10):
    """Per-query-chunk work of a causal workload in its own layout and in the
    contiguous layout at the same shape: visible pairs from the schedule and the
    measured time (median of `reps` launches) of each query chunk computed alone
    (one device's share)."""
    import synthetic
    from exact_long_context_amd import ringattn as ra
    q, k, v = synthetic.draw(w, device="cuda")
    rep = {}
    for layout in (w.layout, "contiguous"):
        qp = api.to_chunked(q, layout, w.n_chunks)
        kp = api.to_chunked(k, layout, w.n_chunks)
        vp = api.to_chunked(v, layout, w.n_chunks)
        L = w.chunk
        pairs, ms = [], []
        for i in range(w.n_chunks):
            qi = qp[:, :, i * L:(i + 1) * L].contiguous()
            out = torch.empty(qi.shape, dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(qi.shape[:3], dtype=torch.float32, device="cuda")
            desc = ra.ring_desc(qi, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=layout, causal=w.causal,
                                q_chunk_first=i, out=out, lse=lse)
            pairs.append(visible_pairs(ra.ra_ring_schedule(desc, i)))
            stream = torch.cuda.current_stream()
            t = time_launches(lambda: ra.ra_ring_fwd(desc, qi, kp, vp, out, lse, stream=stream), stream, reps, 1,
                              torch)
            ms.append(float(np.median(t)))
        rep[layout] = {"visible_pairs_max_over_min": round(max(pairs) / min(pairs), 6),
                       "visible_pairs_max_over_mean": round(max(pairs) / (sum(pairs) / len(pairs)), 6),
                       "ms_max_over_min": round(max(ms) / min(ms), 3),
                       "ms_per_query_chunk": [round(x, 3) for x in ms]}
        del qp, kp, vp
        torch.cuda.empty_cache()
    return rep


# Workloads the oracle leg checks: every element where the oracle finishes in
# seconds to a minute, else sampled query rows (each against all its visible keys).
ORACLE_FULL = ("tiny_sim", "mha_8k", "mha_8k_sharp", "causal_contig_32k", "f32_causal_8k")
ORACLE_SAMPLED = (("causal_striped_128k", 1024), ("zigzag_1m_gqa", 1024))


def _sample(w, n, seed):
    """Seeded (head, buffer row) pairs spread evenly over the query segments,
    with the first and last row of every segment."""
    L = w.chunk
    seg = L // 2 if w.layout == "zigzag" else L
    rng = np.random.default_rng(seed)
    out = []
    starts = [ci * L + s0 for ci in range(len(w.query_chunks)) for s0 in range(0, L, seg)]
    per = max(1, n // len(starts) - 2)
    for r0 in starts:
        rows = [r0, r0 + seg - 1] + (r0 + rng.integers(seg, size=per)).tolist()
        out += [(int(rng.integers(w.hq)), int(r)) for r in rows]
    return out


def gpu_outputs(api, torch):
    """The library's outputs for the oracle leg, computed outside every timed
    region: per workload, out in the input dtype and in fp32 and lse (all rows,
    or the sampled rows), with the inputs the oracle reads (logical k, v; query
    rows in chunk-major order), all on the host."""
    import synthetic
    res = {}
    for name, n in [(x, None) for x in ORACLE_FULL] + list(ORACLE_SAMPLED):
        w = synthetic.WORKLOADS[name]
        q, k, v = synthetic.draw(w, device="cuda")
        kp = api.to_chunked(k, w.layout, w.n_chunks)
        vp = api.to_chunked(v, w.layout, w.n_chunks)
        qp = api.to_chunked(q, w.layout, w.n_chunks) if w.q_chunks is None else q
        o_in, lse = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                     q_chunk_first=w.query_chunks[0])
        o32, _ = api.ring_forward(qp, kp, vp, seq=w.seq, n_chunks=w.n_chunks, layout=w.layout, causal=w.causal,
                                  q_chunk_first=w.query_chunks[0], out_dtype=torch.float32, return_lse=False)
        torch.cuda.synchronize()
        rec = {"w": w, "q": q.cpu(), "k": k.cpu(), "v": v.cpu(), "finite": bool(torch.isfinite(o_in.float()).all())}
        if n is None:
            rec.update(out_in=o_in.cpu(), out_f32=o32.cpu(), lse=lse.cpu(), samples=None)
        else:
            smp = _sample(w, n, seed=sum(map(ord, name)))
            hs = torch.tensor([h for h, _ in smp], device="cuda")
            rs = torch.tensor([r for _, r in smp], device="cuda")
            rec.update(out_in=o_in[0, hs, rs].cpu(), out_f32=o32[0, hs, rs].cpu(), lse=lse[0, hs, rs].cpu(),
                       samples=smp)
        res[name] = rec
        del q, k, v, kp, vp, qp, o_in, o32, lse
        torch.cuda.empty_cache()
    return res


def cpu_oracle_leg(w, flop_total, gpu, ra):
    """Everything that runs the float64 oracle (as it stands), on the host:

    * cpu_baseline: the headline workload on a bounded sample (2048 query rows
      of KV head 0, both zig-zag segments, against all their visible keys; one
      oracle call, numpy's BLAS threads), scaled to the metric's unit by the
      sample's own FLOP count;
    * the oracle timed in full on the small workloads (one query head per
      thread), and its max-abs differences from the library's outputs of
      gpu_outputs(): every element there, sampled rows on the large ones."""
    import concurrent.futures

    import threadpoolctl
    import torch

    import synthetic
    from oracle import attention as OA
    from oracle import layout as OL

    info = threadpoolctl.threadpool_info()
    blas_threads = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"), default=1)
    n_threads = max(1, min(16, len(os.sched_getaffinity(0))))

    def positions(wk):
        return np.concatenate([OL.chunk_positions(wk.layout, wk.seq, wk.n_chunks, c) for c in wk.query_chunks])

    def query_rows(wk, q):
        # chunk-major query rows by a plain gather over the oracle's own map
        if wk.q_chunks is not None:
            return q
        return q.index_select(2, torch.from_numpy(OL.all_positions(wk.layout, wk.seq, wk.n_chunks)))

    # -- headline sample
    q, k, v = synthetic.draw(w, device="cuda")
    G = w.hq // w.hkv
    rng = np.random.default_rng(2024)
    L = w.chunk
    qpos_all = positions(w)
    n_rows = 2048
    rows = np.sort(rng.choice(len(w.query_chunks) * L, size=n_rows, replace=False))
    heads = rng.integers(0, G, size=n_rows)          # query heads of KV head 0
    qsel = torch.stack([q[0, int(h), int(r)] for h, r in zip(heads, rows)]).cpu()[None, None]
    kg, vg = k[:, 0:1].cpu(), v[:, 0:1].cpu()
    del q, k, v
    torch.cuda.empty_cache()
    qpos = qpos_all[rows]
    pairs = int(np.minimum(qpos + 1, w.seq).sum()) if w.causal else n_rows * w.seq
    flop = 4.0 * w.d * pairs
    t0 = time.perf_counter()
    OA.attention_reference(qsel, kg, vg, causal=w.causal, q_pos=qpos, k_pos=np.arange(w.seq))
    dt = time.perf_counter() - t0
    baseline = {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
                "kind": "oracle",
                "sample": f"{n_rows} query rows of KV head 0 (seeded, both zig-zag segments) against all their "
                          f"visible keys: {flop:.3e} FLOP in {dt:.2f} s, float64 numpy; the full step would take "
                          f"{flop_total / (flop / dt) / 3600:.1f} h at this rate"}
    del qsel, kg, vg

    # -- the other workloads: full (timed) or sampled, and the differences from the library
    full, parity = {}, {}
    for name, rec in gpu.items():
        wk = rec["w"]
        qr = query_rows(wk, rec["q"])
        qpos = positions(wk)
        Gk = wk.hq // wk.hkv
        if rec["samples"] is None:
            def one(h, qr=qr, rec=rec, qpos=qpos, Gk=Gk, wk=wk):
                g = h // Gk
                o, l = OA.attention_reference(qr[:, h:h + 1], rec["k"][:, g:g + 1], rec["v"][:, g:g + 1],
                                              causal=wk.causal, q_pos=qpos, k_pos=np.arange(wk.seq))
                return o[0, 0], l[0, 0]
            items = list(range(wk.hq))
        else:
            groups = {}
            for i, (h, r) in enumerate(rec["samples"]):
                reach = int(qpos[r]) * 8 // wk.seq if wk.causal else 0
                groups.setdefault((h // Gk, reach), []).append(i)
            items = sorted(groups.items())

            def one(item, qr=qr, rec=rec, qpos=qpos, wk=wk):
                (g, _), idx = item
                hs = [rec["samples"][i][0] for i in idx]
                rs = [rec["samples"][i][1] for i in idx]
                kmax = int(qpos[rs].max()) + 1 if wk.causal else wk.seq
                qs = torch.stack([qr[0, h, r] for h, r in zip(hs, rs)])[None, None]
                o, l = OA.attention_reference(qs, rec["k"][:, g:g + 1, :kmax], rec["v"][:, g:g + 1, :kmax],
                                              causal=wk.causal, q_pos=qpos[rs], k_pos=np.arange(kmax))
                return o[0, 0], l[0, 0]
        t0 = time.perf_counter()
        with threadpoolctl.threadpool_limits(1):
            with concurrent.futures.ThreadPoolExecutor(n_threads) as ex:
                res = list(ex.map(one, items))
        dt = time.perf_counter() - t0
        if rec["samples"] is None:
            ref = np.stack([o for o, _ in res])[None]
            ref_lse = np.stack([l for _, l in res])[None]
        else:
            ref = np.zeros((len(rec["samples"]), wk.d))
            ref_lse = np.zeros(len(rec["samples"]))
            for (_, idx), (o, l) in zip(items, res):
                ref[idx], ref_lse[idx] = o, l

        def err(a, b):
            return float(np.max(np.abs(a.float().double().numpy() - b)))
        tol = 1e-4 if wk.dtype == "f32" else 2e-2
        e = {"rows": "all" if rec["samples"] is None else f"{len(rec['samples'])} sampled",
             "max_abs_out": err(rec["out_in"], ref), "max_abs_out_fp32_output": err(rec["out_f32"], ref),
             "max_abs_lse": err(rec["lse"], ref_lse), "tolerance": tol, "out_finite": rec["finite"]}
        e["within_tolerance"] = bool(max(e["max_abs_out"], e["max_abs_out_fp32_output"], e["max_abs_lse"]) <= tol
                                     and rec["finite"])
        parity[name] = e
        log(f"  oracle vs library, {name} ({e['rows']} rows): out {e['max_abs_out']:.3e} "
            f"(fp32 out {e['max_abs_out_fp32_output']:.3e}), lse {e['max_abs_lse']:.3e}, oracle {dt:.1f} s")
        if rec["samples"] is None:
            fl = workload_flop(wk, ra)
            full[name] = {"seconds": round(dt, 3), "gflops": round(fl / dt / 1e9, 3), "threads": n_threads,
                          "flop": fl}
    return baseline, full, parity


def mfma_ceiling(random_operands, iters=160000):
    """Sustained v_mfma_f32_32x32x16_bf16 rate of this GPU with operands in
    registers (libramfmaprobe.so, a measurement helper beside the library):
    2048 workgroups of 8 waves, each wave 4 x iters MFMA, about as long as one
    headline launch, so that the chip settles at the clock it holds under
    matrix-core load."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_long_context_amd", "libramfmaprobe.so"))
    lib.ra_probe_mfma_bf16.restype = ctypes.c_int
    ms, tf, ghz = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = lib.ra_probe_mfma_bf16(2048, iters, random_operands, ctypes.byref(ms), ctypes.byref(tf), ctypes.byref(ghz))
    if rc != 0:
        raise SystemExit(f"MFMA probe failed with HIP error {rc}")
    return {"operands": "N(0,1)-like bf16" if random_operands else "zero", "ms": round(ms.value, 3),
            "tflops": round(tf.value, 1), "clock_ghz": round(ghz.value, 3),
            "frac_of_peak": round(tf.value / PEAK_BF16_TFLOPS, 4)}


def kernel_sources_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_record(workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on this workload and on the kernel source as it is now."""
    if workload != TRAFFIC_WORKLOAD or not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_per_dispatch(csv_path, counter, name_part):
    """Mean per-dispatch value of one rocprofv3 counter over the dispatches whose
    kernel name contains name_part (values of one dispatch summed)."""
    import collections
    import csv
    per = collections.defaultdict(float)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{csv_path}: no {counter} rows for kernels matching '{name_part}'")
    return sum(per.values()) / len(per), len(per)


def write_traffic(fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes=1 << 30):
    """HBM bytes per launch of the attention kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes, each scaled by what the same counter reads for a plain
    device copy of copy_bytes (bench.py --copy-calib)."""
    kib = 1024.0
    f_attn, n1 = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "attn_fwd_bf16")
    w_attn, n2 = _counter_per_dispatch(write_csv, "WRITE_SIZE", "attn_fwd_bf16")
    f_copy, _ = _counter_per_dispatch(cfetch_csv, "FETCH_SIZE", "copyBuffer")
    w_copy, _ = _counter_per_dispatch(cwrite_csv, "WRITE_SIZE", "copyBuffer")
    rf = f_copy * kib / copy_bytes   # counter bytes per byte actually read
    wf = w_copy * kib / copy_bytes
    read_b = f_attn * kib / rf
    write_b = w_attn * kib / wf
    rec = {"kernel_sources_sha256": kernel_sources_sha256(),
           "hbm_bytes_per_launch": read_b + write_b,
           "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
           "fetch_size_kib_per_launch": f_attn, "write_size_kib_per_launch": w_attn,
           "copy_calibration": {"bytes": copy_bytes, "fetch_size_kib": f_copy, "write_size_kib": w_copy,
                                "read_factor": rf, "write_factor": wf},
           "dispatches": [n1, n2]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="zigzag_1m_gqa")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads, the split-KV report and the step-by-step timing")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-memory", action="store_true", help="skip the memory-bound entry points")
    ap.add_argument("--memory-only", action="store_true",
                    help="only time the memory-bound entry points (for profiling) and exit")
    ap.add_argument("--split-only", action="store_true",
                    help="only run the split-KV report on the one-chunk shares (for profiling) and exit")
    ap.add_argument("--stepwise-only", action="store_true",
                    help="only time the workload step by step through ra_ring_step (for profiling) and exit")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time ra_ring_bwd on the workload (for profiling) and exit")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run N plain 1 GiB device copies (counter calibration) and exit")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the sustained bf16 MFMA rate (zero and random operands) and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 counter CSVs into the traffic record under profiles/ and exit")
    args = ap.parse_args()

    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic), indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the ring runs over KV chunks resident in this GPU's HBM, "
              f"so --gpus {args.gpus} is not supported (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic
    from exact_long_context_amd import api
    from exact_long_context_amd import ringattn as ra

    if args.mfma_ceiling:
        print(json.dumps({"v_mfma_f32_32x32x16_bf16_sustained": {
            name: mfma_ceiling(rnd) for name, rnd in (("zero_operands", 0), ("random_operands", 1))}}))
        return

    if args.copy_calib:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(args.copy_calib):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 2, "copy_bytes_written": b.numel() * 2,
                          "copies": args.copy_calib}))
        return

    w = synthetic.WORKLOADS[args.workload]
    flop = workload_flop(w, ra)
    if args.backward_only:
        t = launch_stats(time_backward(w, args.steps, args.warmup, api, torch))
        print(json.dumps({"backward_ms": t, "tflops": round(2.5 * flop / (t["mean"] * 1e-3) / 1e12, 2)}))
        return
    if args.memory_only:
        print(json.dumps(time_memory_kernels(w, torch, max(1, args.steps))))
        return
    if args.split_only:
        print(json.dumps(split_kv_report(api, torch, max(1, args.steps))))
        return
    if args.stepwise_only:
        t = launch_stats(time_stepwise(w, max(1, args.steps), args.warmup, api, torch))
        print(json.dumps({"stepwise_ms": t, "tflops": round(flop / (t["mean"] * 1e-3) / 1e12, 2)}))
        return
    log(f"workload {w.name}: {flop:.4e} FLOP per step (causal-adjusted)")
    head = launch_stats(time_workload(w, args.steps, args.warmup, api, torch))
    ms = head["mean"]
    tflops = flop / (ms * 1e-3) / 1e12
    log(f"  {ms:.3f} ms/step (median {head['median']:.3f}, min {head['min']:.3f})  {tflops:.1f} TFLOP/s  "
        f"({tflops / PEAK_BF16_TFLOPS * 100:.1f}% of bf16 peak)")
    torch.cuda.empty_cache()
    ceiling = mfma_ceiling(1)
    log(f"  measured bf16 MFMA ceiling (random operands): {ceiling['tflops']} TFLOP/s at {ceiling['clock_ghz']} GHz")
    ctile = computed_tile_flop(w, ra)

    others = {}
    if not args.no_others:
        # launches per workload: at least 50 for the small ones, 10 for the large ones
        for name, n in (("tiny_sim", 200), ("mha_8k", 50), ("mha_8k_sharp", 50), ("causal_contig_32k", 50),
                        ("causal_striped_128k", 10), ("usp_1m_share", 10), ("f32_causal_8k", 20)):
            wo = synthetic.WORKLOADS[name]
            fo = workload_flop(wo, ra)
            t = launch_stats(time_workload(wo, max(n, args.steps), 3, api, torch))
            others[name] = {"ms": t, "tflops": round(fo / (t["mean"] * 1e-3) / 1e12, 4),
                            "tflops_at_median": round(fo / (t["median"] * 1e-3) / 1e12, 4), "flop": fo}
            if wo.dtype == "bf16":
                others[name]["computed_tile_flop"] = computed_tile_flop(wo, ra)
            else:
                # fp32 inputs run on the fp32 matrix cores (v_mfma_f32_32x32x2_f32)
                others[name]["frac_of_fp32_mfma_peak"] = round(others[name]["tflops"] / PEAK_FP32_TFLOPS, 4)
            log(f"  {name}: {t['mean']:.4f} ms (median {t['median']:.4f}, min {t['min']:.4f})  "
                f"{others[name]['tflops']} TFLOP/s")
            torch.cuda.empty_cache()
            if name == "causal_striped_128k":
                others[name]["per_query_chunk_balance"] = balance_report(wo, api, torch)
                for lay, r in others[name]["per_query_chunk_balance"].items():
                    log(f"    {lay}: visible pairs max/min {r['visible_pairs_max_over_min']}, "
                        f"time max/min {r['ms_max_over_min']}")
                torch.cuda.empty_cache()

    split = None
    stepwise = None
    if not args.no_others:
        split = split_kv_report(api, torch, max(10, args.steps))
        t = launch_stats(time_stepwise(w, max(3, args.steps // 3), 1, api, torch))
        stepwise = {"entry_point": "ra_ring_step", "steps_per_pass": w.n_chunks, "ms": t,
                    "tflops": round(flop / (t["mean"] * 1e-3) / 1e12, 2), "ms_fused": round(ms, 3),
                    "stepwise_over_fused": round(t["mean"] / ms, 4)}
        log(f"  step by step (ra_ring_step x {w.n_chunks}): {t['mean']:.3f} ms  {stepwise['tflops']} TFLOP/s "
            f"({t['mean'] / ms:.3f} x the fused launch)")
        torch.cuda.empty_cache()

    backward = None
    if not args.no_backward:
        torch.cuda.empty_cache()
        t = launch_stats(time_backward(w, max(3, args.steps // 3), 1, api, torch))
        bflop = 2.5 * flop  # five products of 2 d per visible pair (S recomputed, dP, dV, dQ, dK)
        btf = bflop / (t["mean"] * 1e-3) / 1e12
        backward = {"entry_point": "ra_ring_bwd", "ms": t, "tflops": round(btf, 2),
                    "flop_per_step": bflop, "frac_of_bf16_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                    "flop_rule": "10 d per visible (query, key) pair and query head (2.5 x the forward)"}
        log(f"  backward: {t['mean']:.3f} ms  {btf:.1f} TFLOP/s ({btf / PEAK_BF16_TFLOPS * 100:.1f}% of bf16 peak)")
        torch.cuda.empty_cache()

    memory = None
    if not args.no_memory:
        memory = time_memory_kernels(w, torch)

    cpu = cpu_full = parity = None
    if not args.no_cpu:
        log("library outputs for the oracle comparison (not timed) ...")
        gpu = gpu_outputs(api, torch)
        log("the float64 oracle: a bounded sample of the headline workload, the small workloads in full ...")
        cpu, cpu_full, parity = cpu_oracle_leg(w, flop, gpu, ra)
        del gpu
        log(f"  cpu oracle {cpu['value']} TFLOP/s on {cpu['cores']} threads")

    achieved = tflops  # one launch per step: algorithmic FLOP per launch / mean launch time
    res = {
        "metric": "ring-chunked attention fwd TFLOP/s (causal-adjusted), % of bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: one query chunk of a {w.seq}-token causal layer, {w.layout} layout, "
                               f"{w.n_chunks} chunks of {w.chunk}, {w.hq} query / {w.hkv} KV heads, d={w.d}, "
                               f"all KV chunks resident in HBM",
                   "global_batch": w.batch, "seq_len": w.seq, "parallelism": "none (one GPU's share)",
                   "flop_per_step": flop, "pct_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS * 100, 2)},
        "launch_ms": head,
        "tflops_at_median": round(flop / (head["median"] * 1e-3) / 1e12, 3),
        "computed_tile_flop_per_step": ctile,
        "computed_tile_tflops": round(ctile / (ms * 1e-3) / 1e12, 3),
        "mfma_ceiling_measured": ceiling,
        "pct_of_measured_mfma_ceiling": round(tflops / ceiling["tflops"] * 100, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_record(w.name)},
        "cpu_baseline": cpu,
        "cpu_oracle_full": cpu_full,
        "parity_vs_oracle": parity,
        "other_workloads": others,
        "backward": backward,
        "split_kv_one_gpu_share": split,
        "ring_step_one_gpu_share": stepwise,
        "memory_bound_entry_points": memory,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
