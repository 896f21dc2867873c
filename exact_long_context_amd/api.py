"""Tensor-level helpers over the C ABI: allocate outputs with torch, build the
descriptors, call the library.  No arithmetic happens here."""
from __future__ import annotations

from typing import Optional

import torch

from . import ringattn as ra


def to_chunked(x: torch.Tensor, layout: str, n_chunks: int, stream=None) -> torch.Tensor:
    """Logical token order [B, H, S, d] -> chunk-major physical order (a new
    contiguous tensor).  x may be a strided view, e.g. a [B, S, H, d] buffer
    transposed to [B, H, S, d]; its last dimension must be contiguous."""
    if x.stride(-1) != 1:
        x = x.contiguous()
    out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    ra.ra_permute_strided(layout, True, x, out, n_chunks, stream)
    return out


def from_chunked(x: torch.Tensor, layout: str, n_chunks: int, stream=None) -> torch.Tensor:
    """Chunk-major physical order -> logical token order (a new contiguous
    tensor); x may be a strided view with a contiguous last dimension."""
    if x.stride(-1) != 1:
        x = x.contiguous()
    out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    ra.ra_permute_strided(layout, False, x, out, n_chunks, stream)
    return out


def ring_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, seq: int, n_chunks: int, layout: str,
                 causal: bool, q_chunk_first: int = 0, out_dtype: Optional[torch.dtype] = None,
                 return_lse: bool = True, scale: float = 0.0, kv_splits: int = 0, stream=None):
    """All ring steps for the query chunks held in ``q`` (physical order).

    q: [B, Hq, n_q * L, d]; k, v: [B, Hkv, seq, d] in chunk-major order.
    ``kv_splits`` > 1 runs the split-KV forward (workspace allocated here).
    Returns (out [B, Hq, n_q * L, d], lse [B, Hq, n_q * L] fp32 or None)."""
    B, Hq, rows, d = q.shape
    out = torch.empty(B, Hq, rows, d, dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty(B, Hq, rows, dtype=torch.float32, device=q.device) if return_lse else None
    desc = ra.ring_desc(q, k, v, seq=seq, n_chunks=n_chunks, layout=layout, causal=causal,
                        q_chunk_first=q_chunk_first, out=out, lse=lse, scale=scale, kv_splits=kv_splits)
    nws = ra.ra_ring_workspace_bytes(desc)
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    ra.ra_ring_fwd(desc, q, k, v, out, lse, ws, nws, stream=stream)
    return out, lse


def ring_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                  lse: torch.Tensor, *, seq: int, n_chunks: int, layout: str, causal: bool, q_chunk_first: int = 0,
                  scale: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients of ``ring_forward`` for the query chunks held in ``q``.

    q, out, dout: [B, Hq, n_q * L, d] (physical order; dout bf16); k, v:
    [B, Hkv, seq, d] chunk-major; lse: [B, Hq, n_q * L] fp32 as ring_forward
    returns it.  Returns fp32 (dq like q, dk and dv like k and v); dk and dv
    hold the share of the given query rows."""
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.stride() != ref.stride():
            raise ValueError("gradients take the strides of their inputs: pass contiguous q, k, v")
    if dout.stride() != out.stride() or dout.dtype != q.dtype:
        raise ValueError("dout must have the strides of out and the dtype of q")
    desc = ra.ring_desc(q, k, v, seq=seq, n_chunks=n_chunks, layout=layout, causal=causal,
                        q_chunk_first=q_chunk_first, out=out, lse=lse, scale=scale)
    need = ra.ra_ring_bwd_workspace_bytes(desc)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ra.ra_ring_bwd(desc, q, k, v, out, dout, lse, dq, dk, dv, workspace, need, stream)
    return dq, dk, dv


class ChunkState:
    """Running (m, l, o) of a query block, fp32, contiguous."""

    def __init__(self, q: torch.Tensor):
        B, Hq, Lq, d = q.shape
        self.m = torch.empty(B, Hq, Lq, dtype=torch.float32, device=q.device)
        self.l = torch.empty_like(self.m)
        self.o = torch.empty(B, Hq, Lq, d, dtype=torch.float32, device=q.device)


def state_init(q: torch.Tensor, k: torch.Tensor, stream=None) -> ChunkState:
    st = ChunkState(q)
    desc = ra.attn_desc(q, k, k, ml=st.m, o=st.o)
    ra.ra_state_init(desc, st.m, st.l, st.o, stream)
    return st


def chunk_forward(st: ChunkState, q, k, v, *, causal: bool = False, delta: int = 0, scale: float = 0.0,
                  stream=None) -> ChunkState:
    desc = ra.attn_desc(q, k, v, ml=st.m, o=st.o, scale=scale)
    ra.ra_chunk_fwd(desc, q, k, v, st.m, st.l, st.o, delta, causal, stream)
    return st


def finalize(st: ChunkState, q, out_dtype: Optional[torch.dtype] = None, stream=None):
    B, Hq, Lq, d = q.shape
    out = torch.empty(B, Hq, Lq, d, dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=q.device)
    desc = ra.attn_desc(q, q, q, out=out, ml=st.m, o=st.o)
    ra.ra_finalize(desc, st.m, st.l, st.o, out, lse, stream)
    return out, lse


def ring_step(st: ChunkState, q, k_chunk, v_chunk, *, step: int, seq: int, n_chunks: int, layout: str,
              causal: bool, q_chunk: int, scale: float = 0.0, stream=None) -> ChunkState:
    """Ring step ``step`` of query chunk ``q_chunk``: ``k_chunk`` / ``v_chunk``
    hold KV chunk (q_chunk - step) mod N only, [B, Hkv, L, d]."""
    desc = ra.ring_desc(q, k_chunk, v_chunk, seq=seq, n_chunks=n_chunks, layout=layout, causal=causal,
                        q_chunk_first=q_chunk, q_chunk_count=1, lse=st.m, scale=scale)
    desc.attn.o = ra.strides_of(st.o)
    ra.ra_ring_step(desc, step, q, k_chunk, v_chunk, st.m, st.l, st.o, stream)
    return st


def ring_forward_stepwise(q, k, v, *, seq: int, n_chunks: int, layout: str, causal: bool, q_chunk: int,
                          out_dtype: Optional[torch.dtype] = None, scale: float = 0.0, stream=None):
    """The ring of one query chunk as a device runs it: state init, the N steps
    in ring order, each given only its KV chunk (a view of the chunk-major k, v
    here, standing for the received buffer), then finalize."""
    L = seq // n_chunks
    st = state_init(q, k, stream)
    for t in range(n_chunks):
        j = (q_chunk - t) % n_chunks
        ring_step(st, q, k[:, :, j * L:(j + 1) * L], v[:, :, j * L:(j + 1) * L], step=t, seq=seq,
                  n_chunks=n_chunks, layout=layout, causal=causal, q_chunk=q_chunk, scale=scale, stream=stream)
    return finalize(st, q, out_dtype, stream)


def merge(lse_a, o_a, lse_b, o_b, lse_out=None, o_out=None, stream=None):
    """Log-sum-exp merge of two normalized fp32 partials [B, H, L] / [B, H, L, d]."""
    lse_out = torch.empty_like(lse_a) if lse_out is None else lse_out
    o_out = torch.empty_like(o_a) if o_out is None else o_out
    B, H, L, d = o_a.shape
    desc = ra.ra_attn_desc()
    desc.batch, desc.hq, desc.hkv, desc.lq, desc.lk, desc.d = B, H, H, L, L, d
    desc.in_dtype = desc.out_dtype = ra.RA_F32
    desc.q = desc.k = desc.v = desc.out = ra.ra_strides(H * L * d, L * d, d)
    desc.ml = ra.ra_strides(lse_a.stride(0), lse_a.stride(1), 1)
    desc.o = ra.strides_of(o_a)
    for t in (lse_b, lse_out):
        if t.stride() != lse_a.stride():
            raise ValueError("lse tensors must share strides")
    for t in (o_b, o_out):
        if t.stride() != o_a.stride():
            raise ValueError("o tensors must share strides")
    ra.ra_merge(desc, lse_a, o_a, lse_b, o_b, lse_out, o_out, stream)
    return lse_out, o_out
