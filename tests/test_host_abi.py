"""Host-side checks of libringattn that need no GPU: the exported symbols, the
layout maps and the ring schedule against the oracle's independent
derivation (bit-exact), and argument validation (every rejected call returns
before any HIP call)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import layout as LY

ra = pytest.importorskip("exact_long_context_amd.ringattn",
                         reason="libringattn.so not built (run __graft_entry__.build())")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", ra.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ra_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(ra._lib, n) is not None
    assert set(ra.EXPORTED) == set(names)


def test_struct_layouts_match_header():
    # sizes fixed by the header's field lists (all naturally aligned)
    assert ctypes.sizeof(ra.ra_strides) == 24
    assert ctypes.sizeof(ra.ra_attn_desc) == 6 * 8 + 2 * 4 + 6 * 24 + 4 + 4
    assert ctypes.sizeof(ra.ra_ring_desc) == ctypes.sizeof(ra.ra_attn_desc) + 8 + 6 * 4
    assert ctypes.sizeof(ra.ra_task) == 6 * 4 + 8 + 2 * 4
    assert ra.ra_abi_version() == 3
    assert ra.ra_status_str(0) == "ok" and ra.ra_status_str(3) == "workspace too small"


@pytest.mark.parametrize("layout,S,N", [("contiguous", 96, 8), ("striped", 96, 8), ("zigzag", 96, 8),
                                        ("zigzag", 64, 32), ("striped", 4096, 16), ("contiguous", 7, 7),
                                        ("striped", 16, 16), ("zigzag", 1 << 20, 32)])
def test_layout_positions_bit_exact(layout, S, N):
    for c in sorted({0, 1, N // 2, N - 1}):
        got = ra.ra_layout_positions(layout, S, N, c)
        assert got.dtype == np.int64
        assert np.array_equal(got, LY.chunk_positions(layout, S, N, c))


def _rdesc(layout, S, N, causal, first=0, count=None, hq=2, hkv=1, d=128):
    import torch
    L = S // N
    q = torch.empty(1, hq, (count or N) * L, d, dtype=torch.bfloat16)
    k = torch.empty(1, hkv, S, d, dtype=torch.bfloat16)
    return ra.ring_desc(q, k, k, seq=S, n_chunks=N, layout=layout, causal=causal, q_chunk_first=first,
                        q_chunk_count=count or N)


@pytest.mark.parametrize("layout,S,N", [("contiguous", 64, 4), ("striped", 64, 4), ("zigzag", 64, 4),
                                        ("zigzag", 96, 6), ("striped", 48, 8), ("contiguous", 40, 5),
                                        ("contiguous", 4, 4), ("zigzag", 1 << 20, 32), ("striped", 131072, 16),
                                        ("contiguous", 32768, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_schedule_bit_exact(layout, S, N, causal):
    desc = _rdesc(layout, S, N, causal)
    L = S // N
    small = S <= 4096
    for i in sorted({0, 1 % N, N // 2, N - 1}):
        got = ra.ra_ring_schedule(desc, i)
        if small:
            ref = LY.ring_schedule(layout, S, N, i, causal)
        else:
            # full-size shapes: compare the kinds and offsets on the position
            # progressions without materialising pair counts
            ref = []
            for t, j in enumerate(LY.ring_order(N, i)):
                qp = LY.chunk_positions(layout, S, N, i)
                kp = LY.chunk_positions(layout, S, N, j)
                for (q0, ql) in LY.segments(layout, S, N, i):
                    for (k0, kl) in LY.segments(layout, S, N, j):
                        a, b = qp[q0:q0 + ql], kp[k0:k0 + kl]
                        ref.append(dict(step=t, kv_chunk=j, q_row0=q0, q_len=ql, kv_row0=k0, kv_len=kl,
                                        kind=LY.classify(a, b, causal), delta=LY.delta_of(a, b) if causal else 0))
        assert len(got) == len(ref)
        for g, r in zip(got, ref):
            for key in ("step", "kv_chunk", "q_row0", "q_len", "kv_row0", "kv_len", "kind"):
                assert g[key] == r[key], (key, g, r)
            if L >= 2 or not causal:
                assert g["delta"] == r["delta"], (g, r)
            else:
                # one-row segments: any offset with the same sign rule describes the same mask
                assert (g["delta"] >= 0) == (r["delta"] >= 0)


def test_schedule_capacity_and_range_errors():
    desc = _rdesc("zigzag", 64, 4, True)
    n = ctypes.c_int32(0)
    tasks = (ra.ra_task * 3)()
    st = ra._lib.ra_ring_schedule(ctypes.byref(desc), 0, tasks, 3, ctypes.byref(n))
    assert st == ra.RA_ERR_INVALID_ARG and n.value == 16
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_schedule(desc, 4)
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_schedule(desc, -1)


# ---------------------------------------------------------------------------
# Validation: every case below must fail before any HIP call (no GPU here).
# Fake device pointers are aligned non-null integers; they are never used.
# Where a GPU is present these tests are skipped: a regression in a check (or
# in a no-launch early exit) would otherwise hand the made-up addresses to a
# kernel.
# ---------------------------------------------------------------------------

P = 1 << 20  # fake aligned pointer


def _gpu_present() -> bool:
    import torch
    return torch.cuda.device_count() > 0   # counts devices without initialising HIP


pytestmark = pytest.mark.skipif(_gpu_present(), reason="fake device pointers: host validation is checked "
                                                       "where no GPU is present")


def _adesc(**kw):
    d = ra.ra_attn_desc()
    B, hq, hkv, lq, lk, dd = kw.get("B", 1), kw.get("hq", 2), kw.get("hkv", 1), kw.get("lq", 64), kw.get("lk", 64), \
        kw.get("d", 128)
    d.batch, d.hq, d.hkv, d.lq, d.lk, d.d = B, hq, hkv, lq, lk, dd
    d.in_dtype = kw.get("in_dtype", ra.RA_BF16)
    d.out_dtype = kw.get("out_dtype", ra.RA_BF16)
    d.q = ra.ra_strides(hq * lq * dd, lq * dd, dd)
    d.k = d.v = ra.ra_strides(hkv * lk * dd, lk * dd, dd)
    d.out = ra.ra_strides(hq * lq * dd, lq * dd, dd)
    d.ml = ra.ra_strides(hq * lq, lq, 1)
    d.o = ra.ra_strides(hq * lq * dd, lq * dd, dd)
    d.scale = 0.0
    d.reserved = 0
    for k, v in kw.items():
        if k in ("q_s", "k_s", "out_s", "o_s", "ml_s"):
            getattr(d, k[:-2]).s = v
        elif k == "reserved":
            d.reserved = v
    return d


def _chunk(desc, q=P, k=P, v=P, m=P, l=P, o=P, delta=0, causal=0):
    return ra._lib.ra_chunk_fwd(ctypes.byref(desc), q, k, v, m, l, o, delta, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), ra.RA_ERR_INVALID_ARG),
    (dict(lq=0), ra.RA_ERR_INVALID_ARG),
    (dict(lk=-1), ra.RA_ERR_INVALID_ARG),
    (dict(d=64), ra.RA_ERR_UNSUPPORTED),
    (dict(d=96, in_dtype=ra.RA_F32), ra.RA_ERR_UNSUPPORTED),
    (dict(in_dtype=7), ra.RA_ERR_INVALID_ARG),
    (dict(out_dtype=9), ra.RA_ERR_INVALID_ARG),
    (dict(q_s=100), ra.RA_ERR_INVALID_ARG),
    (dict(k_s=-128), ra.RA_ERR_INVALID_ARG),
    (dict(o_s=130), ra.RA_ERR_INVALID_ARG),
    (dict(ml_s=2), ra.RA_ERR_INVALID_ARG),
    (dict(reserved=1), ra.RA_ERR_INVALID_ARG),
])
def test_chunk_fwd_rejects_bad_descriptors(kw, status):
    assert _chunk(_adesc(**kw)) == status
    assert ra.ra_last_error() != ""


def test_chunk_fwd_rejects_null_and_misaligned_pointers():
    d = _adesc()
    assert _chunk(d, q=None) == ra.RA_ERR_INVALID_ARG
    assert _chunk(d, o=None) == ra.RA_ERR_INVALID_ARG
    assert _chunk(d, k=P + 2) == ra.RA_ERR_INVALID_ARG
    assert _chunk(d, causal=2) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_chunk_fwd(None, P, P, P, P, P, P, 0, 0, None) == ra.RA_ERR_INVALID_ARG


def test_fully_hidden_chunk_is_a_no_op():
    # a causal offset below -(lq - 1) hides every key: returns OK without launching
    d = _adesc(lq=64)
    assert _chunk(d, delta=-64, causal=1) == ra.RA_OK


def test_finalize_merge_state_validation():
    d = _adesc()
    assert ra._lib.ra_finalize(ctypes.byref(d), P, P, P, None, None, None) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_finalize(ctypes.byref(d), P, P, P + 4, P, None, None) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_merge(ctypes.byref(d), P, P, None, P, P, P, None) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_merge(ctypes.byref(_adesc(hq=3, hkv=2)), P, P, P, P, P, P, None) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_state_init(ctypes.byref(d), P, None, P, None) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_state_init(ctypes.byref(_adesc(d=48, in_dtype=ra.RA_F32)), P, P, P, None) == \
        ra.RA_ERR_UNSUPPORTED


def _ring_desc(layout="zigzag", S=256, N=4, causal=1, first=0, count=4, lq=None, lk=None, kv_splits=0, **kw):
    r = ra.ra_ring_desc()
    L = S // N if N > 0 else 0
    r.attn = _adesc(lq=lq if lq is not None else max(L, 1), lk=lk if lk is not None else max(L, 1), **kw)
    r.seq, r.n_chunks = S, N
    r.layout = ra.LAYOUTS.get(layout, 9) if isinstance(layout, str) else layout
    r.causal, r.q_chunk_first, r.q_chunk_count, r.kv_splits = causal, first, count, kv_splits
    return r


def _ring(ws=0, wsp=None, **kw):
    r = _ring_desc(**kw)
    return ra._lib.ra_ring_fwd(ctypes.byref(r), P, P, P, P, None, wsp, ws, None)


@pytest.mark.parametrize("kw", [
    dict(S=250, N=4), dict(N=0), dict(layout=9), dict(S=12, N=4, count=4),  # odd L for zig-zag
    dict(causal=2), dict(first=3, count=2), dict(first=-1), dict(count=0), dict(lq=32), dict(lk=128),
    dict(kv_splits=-1), dict(kv_splits=ra.RA_MAX_KV_SPLITS + 1), dict(hq=4, hkv=3),
    dict(S=1 << 32, N=1, lq=1, lk=1),
])
def test_ring_fwd_rejects_bad_descriptors(kw):
    assert _ring(**kw) == ra.RA_ERR_INVALID_ARG


def test_ring_split_kv_workspace():
    # partial o (d floats) and lse (1 float) per split and (b, query head, row)
    for S, count in ((0, 4), (1, 4), (2, 4), (5, 1), (ra.RA_MAX_KV_SPLITS, 2)):
        r = _ring_desc(S=256, N=4, count=count, B=2, hq=4, hkv=2, kv_splits=S)
        want = 0 if S <= 1 else S * 2 * 4 * (count * 64) * (128 + 1) * 4
        assert ra.ra_ring_workspace_bytes(r) == want
    need = ra.ra_ring_workspace_bytes(_ring_desc(kv_splits=3))
    assert _ring(kv_splits=3, ws=need - 1, wsp=P) == ra.RA_ERR_WORKSPACE
    assert _ring(kv_splits=3, ws=need, wsp=None) == ra.RA_ERR_INVALID_ARG
    assert _ring(kv_splits=3, ws=need, wsp=P + 8) == ra.RA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(layout="zigzag", S=1026, N=513, count=1),       # 1026 KV segments
    dict(layout="contiguous", S=2050, N=1025, count=1),  # 1025 KV segments
    dict(layout="contiguous", S=256, N=4, k_s=1 << 24),  # K rows span 8 GiB
])
def test_ring_fwd_rejects_unsupported_bf16_extents(kw):
    assert _ring(**kw) == ra.RA_ERR_UNSUPPORTED


def test_ring_fwd_rejects_null_pointers_and_workspace():
    r = ra.ra_ring_desc()
    r.attn = _adesc(lq=64, lk=64)
    r.seq, r.n_chunks, r.layout, r.causal, r.q_chunk_first, r.q_chunk_count = 256, 4, 0, 1, 0, 4
    assert ra._lib.ra_ring_fwd(ctypes.byref(r), None, P, P, P, None, None, 0, None) == ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_ring_fwd(ctypes.byref(r), P, P, P, P + 8, None, None, 0, None) == ra.RA_ERR_INVALID_ARG
    assert ra.ra_ring_workspace_bytes(r) == 0


def test_permute_and_positions_validation():
    f = ra._lib.ra_permute
    assert f(0, 1, 1, 1, 10, 3, 8, ra.RA_BF16, P, P, None) == ra.RA_ERR_INVALID_ARG   # S % N
    assert f(2, 1, 1, 1, 12, 4, 8, ra.RA_BF16, P, P, None) == ra.RA_ERR_INVALID_ARG   # odd L zig-zag
    assert f(5, 1, 1, 1, 16, 4, 8, ra.RA_BF16, P, P, None) == ra.RA_ERR_INVALID_ARG   # layout
    assert f(0, 3, 1, 1, 16, 4, 8, ra.RA_BF16, P, P, None) == ra.RA_ERR_INVALID_ARG   # direction
    assert f(0, 1, 1, 1, 16, 4, 8, 4, P, P, None) == ra.RA_ERR_INVALID_ARG            # dtype
    assert f(0, 1, 1, 1, 16, 4, 8, ra.RA_F32, P + 2, P, None) == ra.RA_ERR_INVALID_ARG  # alignment
    assert f(0, 1, 1, 1, 16, 4, 8, ra.RA_F32, None, P, None) == ra.RA_ERR_INVALID_ARG
    g = ra._lib.ra_permute_strided
    ok = (0, 1, 2, 3, 16, 4, 8, ra.RA_F32, P, 3 * 16 * 8, 16 * 8, 8, P, 3 * 16 * 8, 16 * 8, 8, None)

    def with_(**kw):
        names = ["layout", "dir", "B", "H", "S", "N", "d", "dtype", "src", "ssb", "ssh", "sss",
                 "dst", "dsb", "dsh", "dss", "stream"]
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return g(*a)
    for bad in (dict(sss=-8), dict(dsh=-1), dict(ssb=-128), dict(src=None), dict(dst=None),
                dict(src=P + 2), dict(dst=P + 6), dict(S=10, N=3), dict(layout=7), dict(dir=2),
                dict(dtype=9), dict(B=0), dict(d=0), dict(layout=2, S=12, N=4)):
        assert with_(**bad) == ra.RA_ERR_INVALID_ARG, bad
    with pytest.raises(ra.RingAttnError):
        ra.ra_layout_positions("zigzag", 12, 4, 0)
    with pytest.raises(ra.RingAttnError):
        ra.ra_layout_positions("striped", 16, 4, 4)


def test_ring_kv_splits_hint():
    """More KV ranges when there are few query tiles, none when the query
    tiles already give every compute unit two workgroups; bounded by
    RA_MAX_KV_SPLITS and by seq / 256."""
    def hint(**kw):
        return ra.ra_ring_kv_splits_hint(_ring_desc(**kw))
    # 1M-token zig-zag share: 4096 workgroups, no split
    assert hint(S=1 << 20, N=32, count=1, hq=32, hkv=8) == 1
    # one 2048-row chunk of 8 MHA heads: 64 workgroups -> 16 ranges
    assert hint(layout="contiguous", S=8192, N=4, count=1, hq=8, hkv=8, causal=0) == 16
    # tiny sequences: at most one range per 256 keys
    assert hint(layout="contiguous", S=512, N=4, count=1, hq=1, hkv=1) == 2
    assert hint(layout="contiguous", S=64, N=4, count=1, hq=1, hkv=1) == 1
    # one 8192-row striped chunk of 8 MHA heads: 256 workgroups -> 4 ranges
    assert hint(layout="striped", S=1 << 17, N=16, first=15, count=1, hq=8, hkv=8) == 4
    # the last 4096-row contiguous chunk of 32 MHA heads: 512 workgroups, no split
    assert hint(layout="contiguous", S=1 << 15, N=8, first=7, count=1, hq=32, hkv=32) == 1
    assert 1 <= hint(layout="striped", S=1 << 17, N=16, count=1, hq=1, hkv=1) <= ra.RA_MAX_KV_SPLITS
    r = _ring_desc(kv_splits=-3)
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_kv_splits_hint(r)



def _step(step, qp=P, kp=P, vp=P, mp=P, lp=P, op=P, **kw):
    r = _ring_desc(**kw)
    return ra._lib.ra_ring_step(ctypes.byref(r), step, qp, kp, vp, mp, lp, op, None)


def test_ring_step_validation():
    one = dict(count=1)
    assert _step(0, count=2) == ra.RA_ERR_INVALID_ARG          # one query chunk per call
    assert _step(-1, **one) == ra.RA_ERR_INVALID_ARG
    assert _step(4, **one) == ra.RA_ERR_INVALID_ARG            # N = 4 steps
    assert _step(0, kp=None, **one) == ra.RA_ERR_INVALID_ARG
    assert _step(0, mp=None, **one) == ra.RA_ERR_INVALID_ARG
    assert _step(0, op=P + 4, **one) == ra.RA_ERR_INVALID_ARG
    assert _step(0, layout=9, **one) == ra.RA_ERR_INVALID_ARG
    assert _step(0, d=64, **one) == ra.RA_ERR_UNSUPPORTED
    assert ra._lib.ra_ring_step(None, 0, P, P, P, P, P, P, None) == ra.RA_ERR_INVALID_ARG


def test_ring_step_wholly_future_is_a_no_op():
    # contiguous causal, query chunk 1 of 4: steps 2 and 3 bring KV chunks 3
    # and 2, wholly after it; the call returns OK without launching anything
    for t in (2, 3):
        assert _step(t, layout="contiguous", first=1, count=1) == ra.RA_OK


def _bwd(r, **ptrs):
    p = dict(q=P, k=P, v=P, out=P, dout=P, lse=P, dq=P, dk=P, dv=P, ws=P)
    p.update(ptrs)
    nws = ra.ra_ring_bwd_workspace_bytes(r)
    return ra._lib.ra_ring_bwd(ctypes.byref(r), p["q"], p["k"], p["v"], p["out"], p["dout"], p["lse"], p["dq"],
                               p["dk"], p["dv"], p["ws"], nws, None)


def test_ring_bwd_validation():
    r = _ring_desc()
    assert ra.ra_ring_bwd_workspace_bytes(r) == 2 * 1 * 2 * 256 * 4
    assert _bwd(_ring_desc(d=64, in_dtype=ra.RA_F32)) == ra.RA_ERR_UNSUPPORTED
    assert _bwd(r, dout=None) == ra.RA_ERR_INVALID_ARG
    assert _bwd(r, ws=None) == ra.RA_ERR_INVALID_ARG
    assert _bwd(r, dq=P + 4) == ra.RA_ERR_INVALID_ARG
    # dout is bf16 and shares the strides of out: an fp32 out whose row stride
    # is 4 mod 8 elements would misalign its 16-byte pieces
    r32 = _ring_desc(out_dtype=ra.RA_F32, out_s=132)
    assert _bwd(r32) == ra.RA_ERR_INVALID_ARG
    assert "multiples of 8" in ra.ra_last_error()
    rs = _ring_desc()
    assert ra._lib.ra_ring_bwd(ctypes.byref(rs), P, P, P, P, P, P, P, P, P, P, 8, None) == ra.RA_ERR_WORKSPACE


def test_ring_bwd_noalloc_validation():
    # the workspace it brings holds 2^21 (batch x query head x query row); beyond that it refuses
    small = _ring_desc(S=1 << 16, N=4, count=4, hq=32, hkv=8)          # 32 x 65536 rows: 16 MiB, fits
    assert ra.ra_ring_bwd_workspace_bytes(small) == ra.RA_BWD_NOALLOC_MAX_BYTES
    big = _ring_desc(S=1 << 16, N=4, count=4, B=2, hq=32, hkv=8)       # twice that
    assert ra._lib.ra_ring_bwd_noalloc(ctypes.byref(big), P, P, P, P, P, P, P, P, P, None) == \
        ra.RA_ERR_UNSUPPORTED
    assert "ra_ring_bwd_noalloc" in ra.ra_last_error()
    assert ra._lib.ra_ring_bwd_noalloc(ctypes.byref(_ring_desc(d=64, in_dtype=ra.RA_F32)), P, P, P, P, P, P, P, P,
                                       P, None) == ra.RA_ERR_UNSUPPORTED
    assert ra._lib.ra_ring_bwd_noalloc(ctypes.byref(_ring_desc()), P, P, P, P, None, P, P, P, P, None) == \
        ra.RA_ERR_INVALID_ARG
    assert ra._lib.ra_ring_bwd_noalloc(ctypes.byref(_ring_desc(out_dtype=ra.RA_F32, out_s=132)), P, P, P, P, P, P,
                                       P, P, P, None) == ra.RA_ERR_INVALID_ARG
