"""Token layouts, ring order and causal classification (oracle side).

Test infrastructure only; see the package docstring.

Everything here is derived from explicit integer position arrays, so that the
host scheduler of the library (which works from closed-form offsets) can be
checked against a derivation that shares nothing with it.

Sources:

* Contiguous chunks: the collator listing ``LongContextDataCollator`` on the
  youngju.dev page "Ring Attention 논문 분석" cuts the token sequence into
  ``world_size`` equal consecutive chunks; the "Context Parallelism" page of
  llm-engineer.pages.dev shows GPU g owning tokens g*s/4 .. (g+1)*s/4.
* Striped: the Ultralytics glossary page "Ring Attention" (how it works) and
  the GPU MODE lecture 013 notes (causal imbalance, first remedy) spread the
  tokens of every device evenly over the whole sequence.  Reading taken:
  token t goes to chunk t mod N at row t div N.
* Zig-zag: the "Context Parallelism" page (causal imbalance section) gives
  each GPU early and late tokens without a formula.  Reading taken: split the
  sequence into 2N segments of s = L/2 tokens; chunk c holds segment c then
  segment 2N-1-c.
* Ring order: the four-device simulation of the glossary page and the
  ``ring_attention_jax`` listing visit KV chunk (i - step) mod N at step
  ``step`` for query chunk i.
* Causality: the lecture notes state that query token i attends to key
  tokens j <= i; the ``ring_attention_causal_step`` listing masks with
  ``triu(diagonal=1)``, which keeps the diagonal.
"""
from __future__ import annotations

import numpy as np

LAYOUTS = ("contiguous", "striped", "zigzag")

FULL, MASKED, SKIP = 0, 1, 2


def _check(layout: str, S: int, N: int):
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    if N <= 0 or S <= 0 or S % N:
        raise ValueError("S must be a positive multiple of N")
    if layout == "zigzag" and (S // N) % 2:
        raise ValueError("zig-zag needs an even chunk length")


def chunk_positions(layout: str, S: int, N: int, c: int) -> np.ndarray:
    """Global token position of every row of chunk ``c`` (int64, length L)."""
    _check(layout, S, N)
    L = S // N
    rows = np.arange(L, dtype=np.int64)
    if layout == "contiguous":
        return c * L + rows
    if layout == "striped":
        return rows * N + c
    s = L // 2
    early = c * s + np.arange(s, dtype=np.int64)
    late = (2 * N - 1 - c) * s + np.arange(s, dtype=np.int64)
    return np.concatenate([early, late])


def all_positions(layout: str, S: int, N: int) -> np.ndarray:
    """Chunk-major concatenation of every chunk's positions: physical row -> position."""
    return np.concatenate([chunk_positions(layout, S, N, c) for c in range(N)])


def owner_of(layout: str, S: int, N: int) -> tuple[np.ndarray, np.ndarray]:
    """Inverse map by brute force: for every position t, (chunk, row)."""
    phys = all_positions(layout, S, N)
    L = S // N
    chunk = np.empty(S, dtype=np.int64)
    row = np.empty(S, dtype=np.int64)
    chunk[phys] = np.repeat(np.arange(N, dtype=np.int64), L)
    row[phys] = np.tile(np.arange(L, dtype=np.int64), N)
    return chunk, row


def segments(layout: str, S: int, N: int, c: int) -> list[tuple[int, int]]:
    """Row ranges (row0, length) of chunk ``c``: the whole chunk, or for zig-zag
    its early and late halves.  On each range the positions form an arithmetic
    progression, which :func:`delta_of` checks from the position array."""
    _check(layout, S, N)
    L = S // N
    if layout == "zigzag":
        return [(0, L // 2), (L // 2, L // 2)]
    return [(0, L)]


def ring_order(N: int, i: int) -> list[int]:
    """KV chunk visited at each step by query chunk i."""
    return [(i - t) % N for t in range(N)]


def visible_count(qpos: np.ndarray, kpos: np.ndarray, causal: bool) -> int:
    """Number of (query, key) pairs that attend, by brute force."""
    if not causal:
        return int(len(qpos) * len(kpos))
    ks = np.sort(kpos)
    return int(np.searchsorted(ks, qpos, side="right").sum())


def classify(qpos: np.ndarray, kpos: np.ndarray, causal: bool) -> int:
    """FULL when every key is visible to every query, SKIP when none is."""
    if not causal:
        return FULL
    if kpos.max() <= qpos.min():
        return FULL
    if kpos.min() > qpos.max():
        return SKIP
    return MASKED


def delta_of(qpos: np.ndarray, kpos: np.ndarray) -> int:
    """The integer delta with: key row k visible to query row p  <=>  k - p <= delta.

    Exists when both position arrays are progressions with one common step
    g > 0: pos_k <= pos_q  <=>  kb + g k <= qb + g p  <=>  k - p <= (qb - kb) / g,
    and since k - p is an integer the bound is floor((qb - kb) / g)."""
    g = int(qpos[1] - qpos[0]) if len(qpos) > 1 else int(kpos[1] - kpos[0]) if len(kpos) > 1 else 1
    if len(qpos) > 1:
        assert np.all(np.diff(qpos) == g)
    if len(kpos) > 1:
        assert np.all(np.diff(kpos) == g)
    return int((int(qpos[0]) - int(kpos[0])) // g)


def ring_schedule(layout: str, S: int, N: int, i: int, causal: bool) -> list[dict]:
    """Every (query segment, KV segment) pair that query chunk i meets, in ring order.

    Within a step the pairs are listed query segment by query segment, KV
    segments in ascending row order.  Each entry has the step, the KV chunk,
    the two row ranges, the kind (FULL / MASKED / SKIP) and delta (0 when the
    attention is not causal)."""
    qsegs = segments(layout, S, N, i)
    qpos_all = chunk_positions(layout, S, N, i)
    out = []
    for t, j in enumerate(ring_order(N, i)):
        kpos_all = chunk_positions(layout, S, N, j)
        for (q0, ql) in qsegs:
            for (k0, kl) in segments(layout, S, N, j):
                qp = qpos_all[q0:q0 + ql]
                kp = kpos_all[k0:k0 + kl]
                kind = classify(qp, kp, causal)
                out.append(dict(step=t, kv_chunk=j, q_row0=q0, q_len=ql, kv_row0=k0, kv_len=kl,
                                kind=kind, delta=delta_of(qp, kp) if causal else 0,
                                visible=visible_count(qp, kp, causal)))
    return out


def chunk_visible_pairs(layout: str, S: int, N: int, i: int, causal: bool) -> int:
    """Visible pairs of query chunk i against the whole sequence (per head)."""
    qp = chunk_positions(layout, S, N, i)
    return sum(visible_count(qp, chunk_positions(layout, S, N, j), causal) for j in range(N))
