"""Gradients of exact softmax attention in float64 (oracle side).

Test infrastructure only; see the package docstring.

For one query head with scores s = scale * q k^T (masked entries -inf),
P = softmax(s) per row and out = P v, an upstream gradient dout gives
(``ring_attention_backward`` on the youngju.dev page, "Ring Attention 논문
분석", the backward listing):

* D = rowsum(dout * out), one value per query row;
* dv = P^T dout;
* dP = dout v^T;
* dS = P * (dP - D) * scale;
* dq = dS k and dk = dS^T q.

P is recomputed from the forward's log-sum-exp, P = exp(s - lse), instead of
being stored (the same listing; lecture 013 notes, section 03 for lse).
With grouped heads the gradients of a key/value head are the sums over the
query heads that read it (query head h reads KV head h // (Hq // Hkv)), the
reading taken for the grouped-query workload as in the forward.

Readings (also in the design notes): masked pairs have P = 0 and so receive
no gradient; a query row that sees no key has out = 0 and contributes
nothing; scale is 1/sqrt(d) unless given.
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, _f64, _kv_head, attention_reference, default_scale


def attention_backward_reference(q, k, v, dout, *, scale=None, causal=False, q_pos=None, k_pos=None):
    """dq, dk, dv of sum(dout * attention(q, k, v)) by the steps listed in the
    module docstring, with P taken from the plain definition (no lse input).

    q, dout ``[B, Hq, Lq, d]``; k, v ``[B, Hkv, Lk, d]``; positions as in
    :func:`oracle.attention.attention_reference`.  Returns float64 arrays of
    the shapes of q, k, v."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Lq, d = q.shape
    _, Hkv, Lk, dv = v.shape
    scale = default_scale(d) if scale is None else float(scale)
    qp = np.arange(Lq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    kp = np.arange(Lk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    vis = (kp[None, :] <= qp[:, None]) if causal else np.ones((Lq, Lk), dtype=bool)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            K, V = k[b, g], v[b, g]
            s = np.where(vis, (q[b, h] @ K.T) * scale, NEG_INF)
            m = s.max(axis=1, initial=NEG_INF)
            seen = m > NEG_INF
            p = np.exp(s - np.where(seen, m, 0.0)[:, None])
            den = p.sum(axis=1)
            P = np.where(seen[:, None], p / np.where(seen, den, 1.0)[:, None], 0.0)
            out = P @ V
            D = (dout[b, h] * out).sum(axis=1)
            dvv[b, g] += P.T @ dout[b, h]
            dP = dout[b, h] @ V.T
            dS = P * (dP - D[:, None]) * scale
            dq[b, h] = dS @ K
            dk[b, g] += dS.T @ q[b, h]
    return dq, dk, dvv


def ring_attention_backward(q_chunks, k_chunks, v_chunks, dout_chunks, out_chunks, lse_chunks, chunk_pos, *,
                            query_chunks, causal, scale=None):
    """The ring way, following the backward listing step by step.

    For every query chunk i (``q_chunks[n]`` holds chunk ``query_chunks[n]``,
    with its forward output ``out_chunks[n]``, log-sum-exp ``lse_chunks[n]``
    and upstream gradient ``dout_chunks[n]``): D = rowsum(dout * out); at
    step t the KV chunk is j = (i - t) mod N; P = exp(scale q k_j^T - lse)
    with the causal mask of the chunk pair (masked P = 0); dv_j and dk_j
    receive this step's block gradients (on several devices they are reduced
    to the owner of chunk j) and dq accumulates dS k_j.

    Returns (dq per query chunk, dk per KV chunk, dv per KV chunk); the KV
    gradients are summed over the given query chunks only."""
    N = len(k_chunks)
    kc = [_f64(x) for x in k_chunks]
    vc = [_f64(x) for x in v_chunks]
    dk = [np.zeros_like(x) for x in kc]
    dvs = [np.zeros_like(x) for x in vc]
    dqs = []
    for n, i in enumerate(query_chunks):
        qi, oi, doi, li = _f64(q_chunks[n]), _f64(out_chunks[n]), _f64(dout_chunks[n]), _f64(lse_chunks[n])
        B, Hq, L, d = qi.shape
        sc = default_scale(d) if scale is None else float(scale)
        D = (doi * oi).sum(axis=-1)                       # [B, Hq, L]
        dq = np.zeros_like(qi)
        qpos = np.asarray(chunk_pos[i])
        for t in range(N):
            j = (i - t) % N
            kpos = np.asarray(chunk_pos[j])
            Hkv = kc[j].shape[1]
            vis = (kpos[None, :] <= qpos[:, None]) if causal else np.ones((L, len(kpos)), dtype=bool)
            for b in range(B):
                for h in range(Hq):
                    g = _kv_head(h, Hq, Hkv)
                    K, V = kc[j][b, g], vc[j][b, g]
                    lse = li[b, h]
                    fin = lse > NEG_INF
                    s = (qi[b, h] @ K.T) * sc
                    P = np.where(vis & fin[:, None], np.exp(s - np.where(fin, lse, 0.0)[:, None]), 0.0)
                    dvs[j][b, g] += P.T @ doi[b, h]
                    dP = doi[b, h] @ V.T
                    dS = P * (dP - D[b, h][:, None]) * sc
                    dq[b, h] += dS @ K
                    dk[j][b, g] += dS.T @ qi[b, h]
        dqs.append(dq)
    return dqs, dk, dvs


def loss_and_forward(q, k, v, dout, **kw):
    """sum(dout * attention(q, k, v)): the scalar whose gradient the two
    functions above return (used by the finite-difference pins)."""
    out, _ = attention_reference(q, k, v, **kw)
    return float((out * _f64(dout)).sum())
