"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds workload shapes and random draws only: no attention
arithmetic, no layout or schedule logic.  Both the float64 oracle and the HIP
path are fed from here so that they see identical bytes.

Workloads (all batch 1, i.i.d. N(0, 1) entries):

* ``tiny_sim``       -- one head, 32 tokens in 4 chunks of 8, d=16, fp32,
  non-causal.  The draw is the four-device simulation of the Ultralytics
  glossary page "Ring Attention" (section "How Ring Attention works"): a
  global seed of 0 and one ``randn(3, 32, 16)`` call split into q, k, v.
* ``mha_8k``         -- 8 heads, 8192 tokens in 4 chunks of 2048, d=128, bf16,
  non-causal; ``mha_8k_sharp`` multiplies q by 8 (exact in bf16).
* ``causal_contig_32k`` -- 32 heads, 32768 tokens in 8 contiguous chunks.
* ``causal_striped_128k`` -- 8 heads, 131072 tokens in 16 striped chunks.
* ``zigzag_1m_gqa``  -- 32 query heads sharing 8 KV heads, 1048576 tokens in
  32 zig-zag chunks of 32768; one query chunk is computed against all 32 KV
  chunks.
* ``f32_causal_8k``  -- fp32 inputs at d = 128: 8 heads, 8192 tokens in 4
  contiguous chunks, causal (the fp32 path at a real head dimension).
* ``usp_1m_share``   -- the same layer as one GPU's share under the hybrid of
  the youngju.dev page (``hybrid_ulysses_ring_attention``) with a head
  all-to-all over 8 GPUs and a ring over 4: 4 query heads sharing 1 KV head,
  1048576 tokens in 4 zig-zag chunks of 262144; one query chunk against all 4.

Draw recipe for the bf16 workloads: a ``torch.Generator`` on the requested
device seeded with the workload's seed; fp32 N(0,1) samples in the order q, k,
v; each tensor drawn in its logical token order ``[B, H, S, d]`` and rounded to
bf16 (round-to-nearest-even).  For ``zigzag_1m_gqa`` and ``usp_1m_share``
only the rows of the computed query chunk are drawn for q, in that chunk's own row order
``[B, Hq, L, d]``; k and v cover all S tokens.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    seq: int
    n_chunks: int
    d: int
    dtype: str          # "f32" | "bf16"
    causal: bool
    layout: str         # "contiguous" | "striped" | "zigzag"
    seed: int
    q_scale: float = 1.0
    q_chunks: Optional[tuple] = None   # None: every chunk is a query chunk

    @property
    def chunk(self) -> int:
        return self.seq // self.n_chunks

    @property
    def query_chunks(self) -> tuple:
        return self.q_chunks if self.q_chunks is not None else tuple(range(self.n_chunks))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_sim": Workload("tiny_sim", 1, 1, 1, 32, 4, 16, "f32", False, "contiguous", 0),
    "mha_8k": Workload("mha_8k", 1, 8, 8, 8192, 4, 128, "bf16", False, "contiguous", 2),
    "mha_8k_sharp": Workload("mha_8k_sharp", 1, 8, 8, 8192, 4, 128, "bf16", False, "contiguous", 2, q_scale=8.0),
    "causal_contig_32k": Workload("causal_contig_32k", 1, 32, 32, 32768, 8, 128, "bf16", True, "contiguous", 3),
    "causal_striped_128k": Workload("causal_striped_128k", 1, 8, 8, 131072, 16, 128, "bf16", True, "striped", 4),
    "zigzag_1m_gqa": Workload("zigzag_1m_gqa", 1, 32, 8, 1048576, 32, 128, "bf16", True, "zigzag", 5, q_chunks=(0,)),
    "usp_1m_share": Workload("usp_1m_share", 1, 4, 1, 1048576, 4, 128, "bf16", True, "zigzag", 6, q_chunks=(0,)),
    "f32_causal_8k": Workload("f32_causal_8k", 1, 8, 8, 8192, 4, 128, "f32", True, "contiguous", 7),
}


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def tiny_sim_draw():
    """The glossary page's draw: global seed 0, one randn(3, 32, 16) split into q, k, v."""
    torch.manual_seed(0)
    q, k, v = torch.randn(3, 32, 16)
    return q, k, v


def draw(w: Workload, device="cpu"):
    """Return (q, k, v).

    q is ``[B, Hq, S, d]`` in logical order when every chunk is a query chunk,
    else ``[B, Hq, len(q_chunks) * L, d]`` holding the rows of the query chunks
    in their chunk-local order (the caller maps rows to positions).
    k and v are ``[B, Hkv, S, d]`` in logical token order.
    """
    if w.name == "tiny_sim":
        q, k, v = tiny_sim_draw()
        shp = (1, 1, 32, 16)
        return (q.reshape(shp).to(device), k.reshape(shp).to(device), v.reshape(shp).to(device))
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = _torch_dtype(w.dtype)
    q_rows = w.seq if w.q_chunks is None else len(w.q_chunks) * w.chunk

    def one(h, rows):
        out = torch.empty(w.batch, h, rows, w.d, dtype=dt, device=device)
        # draw in slices of at most 2^26 values to bound the fp32 staging buffer
        flat = out.view(-1, w.d)
        step = max(1, (1 << 26) // w.d)
        for r0 in range(0, flat.shape[0], step):
            r1 = min(flat.shape[0], r0 + step)
            flat[r0:r1] = torch.randn(r1 - r0, w.d, generator=g, device=device, dtype=torch.float32).to(dt)
        return out

    q = one(w.hq, q_rows)
    k = one(w.hkv, w.seq)
    v = one(w.hkv, w.seq)
    if w.q_scale != 1.0:
        q = (q.float() * w.q_scale).to(dt)
    return q, k, v


def uniform_draw(shape, seed, dtype=torch.float32, device="cpu", lo=-1.0, hi=1.0):
    """Plain seeded uniform tensor for unit tests of the elementwise entry points."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo).to(dtype)


def normal_draw(shape, seed, dtype=torch.float32, device="cpu", std=1.0):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)
