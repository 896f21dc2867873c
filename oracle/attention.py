"""Exact softmax attention in float64 (oracle side).

Test infrastructure only; see the package docstring.

Notation follows the pages: for one query row the scores are
s_u = scale * <q, k_u> with scale = 1/sqrt(d); m is the largest score seen so
far, l the sum of exp(s - m) over the keys seen so far and o the sum of
exp(s - m) * v over those keys (the "Context Parallelism" page of
llm-engineer.pages.dev, section "Method 2: Ring Attention").  The final output
is o / l and the log-sum-exp is lse = m + ln l (GPU MODE lecture 013 notes,
section 03, stable softmax and log-sum-exp).

Tensor shapes: q ``[B, Hq, Lq, d]``, k and v ``[B, Hkv, Lk, d]``; query head h
reads KV head ``h // (Hq // Hkv)``.  The pages show only Hq == Hkv; the grouped
mapping is the reading taken for the grouped-query workload and equals
``repeat_interleave`` of the KV heads.

Readings of silent or inconsistent passages (each also listed in the design
notes of the repository):

* Masked scores are -inf, as in ``ring_attention_forward`` and
  ``ring_attention_causal_step`` of the youngju.dev page; the -1e9 sentinel of
  the ``ring_attention_jax`` listing would give a fully masked row weight 1
  per key, which is wrong.  A row that sees no key in a step is left
  unchanged by that step; a row that sees no key at all returns o = 0 and
  lse = -inf.
* The logarithm is natural.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(d: int) -> float:
    """1/sqrt(d_k): the scale of every listing on the youngju.dev page and of
    the glossary simulation."""
    return 1.0 / math.sqrt(d)


def _kv_head(h: int, hq: int, hkv: int) -> int:
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


# ---------------------------------------------------------------------------
# 1. The plain definition
# ---------------------------------------------------------------------------

def attention_reference(q, k, v, *, scale=None, causal=False, q_pos=None, k_pos=None,
                        max_block_elems=1 << 24):
    """Exact attention by its definition: softmax(scale * q k^T) v per row.

    With ``causal`` a key is seen only when its global position is at most the
    query's (lecture 013 notes: query token i sees key tokens j <= i).
    ``q_pos`` / ``k_pos`` are the global positions of the rows (default
    0..Lq-1 and 0..Lk-1).  The rows are processed in blocks to bound memory;
    each block is still the full softmax over every key of its rows.

    Returns (out ``[B, Hq, Lq, dv]``, lse ``[B, Hq, Lq]``), both float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, d = q.shape
    _, Hkv, Lk, dv = v.shape
    scale = default_scale(d) if scale is None else float(scale)
    qp = np.arange(Lq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    kp = np.arange(Lk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    out = np.zeros((B, Hq, Lq, dv))
    lse = np.full((B, Hq, Lq), NEG_INF)
    rb = max(1, max_block_elems // max(Lk, 1))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            K, V = k[b, g], v[b, g]
            for r0 in range(0, Lq, rb):
                r1 = min(Lq, r0 + rb)
                s = (q[b, h, r0:r1] @ K.T) * scale
                if causal:
                    s = np.where(kp[None, :] <= qp[r0:r1, None], s, NEG_INF)
                m = s.max(axis=1, initial=NEG_INF)
                seen = m > NEG_INF
                msafe = np.where(seen, m, 0.0)
                p = np.exp(s - msafe[:, None])          # exp(-inf) = 0 for masked keys
                den = p.sum(axis=1)
                num = p @ V
                out[b, h, r0:r1] = np.where(seen[:, None], num / np.where(seen, den, 1.0)[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(seen, msafe + np.log(np.where(seen, den, 1.0)), NEG_INF)
    return out, lse


# ---------------------------------------------------------------------------
# 2. The chunked (m, l, o) loop in ring order
# ---------------------------------------------------------------------------

def init_state(B, Hq, L, dv):
    """m = -inf, l = 0, o = 0 (the accumulators of ``ring_attention_forward``)."""
    return (np.full((B, Hq, L), NEG_INF), np.zeros((B, Hq, L)), np.zeros((B, Hq, L, dv)))


def chunk_update(m, l, o, q, k, v, *, scale=None, causal=False, delta=0):
    """Fold one KV chunk into the running state (m, l, o), returning new arrays.

    The update of ``blockwise_attention`` / ``ring_attention_forward`` on the
    youngju.dev page: the new maximum is the larger of the old one and the
    block's row maximum, the old sums are multiplied by exp(old - new), and the
    block adds exp(s - new) to l and exp(s - new) v to o.

    Causal masking uses row indices local to the chunk pair: key row kk is
    hidden from query row p when kk - p > delta.  delta = 0 is the
    ``triu(diagonal=1)`` mask of ``ring_attention_causal_step``; other values
    express any pair of position progressions with a common step.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    m, l, o = _f64(m).copy(), _f64(l).copy(), _f64(o).copy()
    B, Hq, Lq, d = q.shape
    _, Hkv, Lk, _ = k.shape
    scale = default_scale(d) if scale is None else float(scale)
    prow = np.arange(Lq)[:, None]
    kcol = np.arange(Lk)[None, :]
    hide = (kcol - prow > delta) if causal else np.zeros((Lq, Lk), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = (q[b, h] @ k[b, g].T) * scale
            s = np.where(hide, NEG_INF, s)
            m_new = np.maximum(m[b, h], s.max(axis=1, initial=NEG_INF))
            live = m_new > NEG_INF                        # rows that have seen a key
            mn = np.where(live, m_new, 0.0)
            alpha = np.where(live, np.exp(np.where(live, m[b, h], 0.0) - mn), 1.0)
            alpha = np.where(m[b, h] == NEG_INF, 0.0, alpha)   # exp(-inf - m') = 0
            p = np.exp(s - mn[:, None])
            p = np.where(live[:, None], p, 0.0)
            l[b, h] = np.where(live, alpha * l[b, h] + p.sum(axis=1), l[b, h])
            o[b, h] = np.where(live[:, None], alpha[:, None] * o[b, h] + p @ v[b, g], o[b, h])
            m[b, h] = m_new
    return m, l, o


def finalize(m, l, o):
    """out = o / l and lse = m + ln l; rows with l = 0 give out = 0, lse = -inf."""
    m, l, o = _f64(m), _f64(l), _f64(o)
    seen = l > 0
    ls = np.where(seen, l, 1.0)
    out = np.where(seen[..., None], o / ls[..., None], 0.0)
    lse = np.where(seen, m + np.log(ls), NEG_INF)
    return out, lse


def ring_attention(q_chunks, k_chunks, v_chunks, chunk_pos, *, query_chunks, causal, scale=None):
    """Exact attention computed the ring way, one query chunk at a time.

    ``k_chunks[j]`` / ``v_chunks[j]`` hold the rows of KV chunk j, ``chunk_pos[j]``
    their global positions; ``q_chunks[n]`` holds the rows of query chunk
    ``query_chunks[n]`` (same positions as that chunk).  For query chunk i the
    state starts empty and step t folds in KV chunk (i - t) mod N, masking by
    global position, as in the four-device simulation of the glossary page and
    ``ring_attention_forward`` of the youngju.dev page.  The mask of each step
    is built from the position arrays directly (not from a delta).

    Returns a list of (out, lse) per query chunk.
    """
    N = len(k_chunks)
    results = []
    for n, i in enumerate(query_chunks):
        qi = _f64(q_chunks[n])
        B, Hq, L, d = qi.shape
        dv = _f64(v_chunks[0]).shape[-1]
        sc = default_scale(d) if scale is None else float(scale)
        m, l, o = init_state(B, Hq, L, dv)
        qpos = np.asarray(chunk_pos[i])
        for t in range(N):
            j = (i - t) % N
            kj, vj = _f64(k_chunks[j]), _f64(v_chunks[j])
            kpos = np.asarray(chunk_pos[j])
            Hkv = kj.shape[1]
            vis = (kpos[None, :] <= qpos[:, None]) if causal else np.ones((L, len(kpos)), dtype=bool)
            for b in range(B):
                for h in range(Hq):
                    g = _kv_head(h, Hq, Hkv)
                    s = np.where(vis, (qi[b, h] @ kj[b, g].T) * sc, NEG_INF)
                    rowmax = s.max(axis=1, initial=NEG_INF)
                    m_new = np.maximum(m[b, h], rowmax)
                    seen = m_new > NEG_INF              # rows with no key so far are skipped
                    mn = np.where(seen, m_new, 0.0)
                    old = m[b, h]
                    a = np.where(old > NEG_INF, np.exp(np.where(old > NEG_INF, old, 0.0) - mn), 0.0)
                    p = np.exp(s - mn[:, None])
                    l[b, h] = np.where(seen, a * l[b, h] + p.sum(axis=1), l[b, h])
                    o[b, h] = np.where(seen[:, None], a[:, None] * o[b, h] + p @ vj[b, g], o[b, h])
                    m[b, h] = m_new
        results.append(finalize(m, l, o))
    return results


# ---------------------------------------------------------------------------
# 3. Log-sum-exp merge of two partials
# ---------------------------------------------------------------------------

def lse_merge(lse_a, o_a, lse_b, o_b):
    """Combine two normalized partials over disjoint key sets.

    GPU MODE lecture 013 notes, section 03: the log-sum-exp of the union is the
    log-sum-exp of the two partial log-sum-exps, and each partial softmax is
    reweighted by its own normalizer over the joint one.  With M = max(lse_a,
    lse_b): lse = M + ln(exp(lse_a - M) + exp(lse_b - M)) and
    o = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b.  A partial with
    lse = -inf (no key) is the identity.
    """
    la, lb = _f64(lse_a), _f64(lse_b)
    oa, ob = _f64(o_a), _f64(o_b)
    M = np.maximum(la, lb)
    fin = M > NEG_INF
    Ms = np.where(fin, M, 0.0)
    ea = np.where(la > NEG_INF, np.exp(np.where(fin, la, 0.0) - Ms), 0.0)
    eb = np.where(lb > NEG_INF, np.exp(np.where(fin, lb, 0.0) - Ms), 0.0)
    tot = ea + eb
    lse = np.where(fin, Ms + np.log(np.where(fin, tot, 1.0)), NEG_INF)
    wa = np.where(fin, ea / np.where(fin, tot, 1.0), 0.0)
    wb = np.where(fin, eb / np.where(fin, tot, 1.0), 0.0)
    o = wa[..., None] * oa + wb[..., None] * ob
    return lse, o


def ring_attention_by_merge(q_chunks, k_chunks, v_chunks, chunk_pos, *, query_chunks, causal, scale=None):
    """A third route: every ring step becomes a normalized partial (lse_t, o_t)
    from the plain definition restricted to that KV chunk, and the partials are
    folded with :func:`lse_merge` in ring order.  This is the bottom-up use of
    log-sum-exp associativity in the lecture 013 notes (section 03)."""
    N = len(k_chunks)
    results = []
    for n, i in enumerate(query_chunks):
        qi = _f64(q_chunks[n])
        B, Hq, L, _ = qi.shape
        dv = _f64(v_chunks[0]).shape[-1]
        lse = np.full((B, Hq, L), NEG_INF)
        o = np.zeros((B, Hq, L, dv))
        for t in range(N):
            j = (i - t) % N
            o_t, lse_t = attention_reference(qi, k_chunks[j], v_chunks[j], scale=scale, causal=causal,
                                             q_pos=chunk_pos[i], k_pos=chunk_pos[j])
            lse, o = lse_merge(lse, o, lse_t, o_t)
        results.append((o, lse))
    return results
