"""Successful calls of every entry point at the full workload shapes, against
a host-only build of the C ABI whose launchers are stand-ins (see
launch_stubs.cpp): validation, the launch planning, the schedule and the
layout maps run under AddressSanitizer / UndefinedBehaviorSanitizer with made-up
device pointers that nothing dereferences.  Run only by
tests/test_host_sanitizers.py, against that build; against the real library
it skips itself (it would hand made-up pointers to kernels)."""
import ctypes

import numpy as np
import pytest

ra = pytest.importorskip("exact_long_context_amd.ringattn")

try:
    LAUNCHES = ctypes.c_int.in_dll(ra._lib, "ra_hostcheck_launches")
    LAST = ctypes.c_longlong.in_dll(ra._lib, "ra_hostcheck_last_work")
    LAST_XCD = ctypes.c_int.in_dll(ra._lib, "ra_hostcheck_last_xcd")
except ValueError:
    pytest.skip("needs the host-only build with stand-in launchers", allow_module_level=True)

P = 1 << 20  # made-up aligned device pointer


def _desc(layout, S, N, hq, hkv, causal=1, first=0, count=1, kv_splits=0, out_dtype=None, in_dtype=None, d=128):
    L = S // N
    r = ra.ra_ring_desc()
    a = r.attn
    a.batch, a.hq, a.hkv, a.lq, a.lk, a.d = 1, hq, hkv, L, L, d
    a.in_dtype = ra.RA_BF16 if in_dtype is None else in_dtype
    a.out_dtype = a.in_dtype if out_dtype is None else out_dtype
    rows = count * L
    a.q = ra.ra_strides(hq * rows * d, rows * d, d)
    a.k = a.v = ra.ra_strides(hkv * S * d, S * d, d)
    a.out = ra.ra_strides(hq * rows * d, rows * d, d)
    a.ml = ra.ra_strides(hq * rows, rows, 1)
    a.o = ra.ra_strides(hq * rows * d, rows * d, d)
    r.seq, r.n_chunks, r.layout, r.causal = S, N, ra.LAYOUTS[layout], causal
    r.q_chunk_first, r.q_chunk_count, r.kv_splits = first, count, kv_splits
    return r


def _calls():
    return LAUNCHES.value


# workgroup-to-XCD order: 1 = one KV stream per XCD (8 streams or a multiple),
# 2 = the streams two at a time over all XCDs (two streams' K and V fit in
# 128 MiB, all of them do not), 3 = blocks of 32 neighbouring workgroups per
# XCD (streams not a multiple of 8, workgroups a multiple of 256), 0 = none
@pytest.mark.parametrize("name,args,work,xcd", [
    ("zigzag_1m_gqa", ("zigzag", 1 << 20, 32, 32, 8), 4096, 1),       # 8 streams x 2 segments x 256 tiles
    ("causal_contig_32k", ("contiguous", 1 << 15, 8, 32, 32, 1, 0, 8), 4096, 1),
    ("causal_striped_128k", ("striped", 1 << 17, 16, 8, 8, 1, 0, 16), 4096, 2),   # 8 streams of 64 MiB
    ("mha_8k", ("contiguous", 8192, 4, 8, 8, 0, 0, 4), 256, 1),
    ("usp_1m_share", ("zigzag", 1 << 20, 4, 4, 1), 4096, 3),        # 1 stream x 2 segments x 2048 tiles
    ("one stream, 4 x 16 tiles", ("contiguous", 4096, 4, 4, 1, 0, 0, 4), 64, 0),   # not a multiple of 256
])
def test_ring_fwd_plans(name, args, work, xcd):
    r = _desc(*args)
    n0 = _calls()
    assert ra._lib.ra_ring_fwd(ctypes.byref(r), P, P, P, P, P, None, 0, None) == ra.RA_OK
    assert _calls() == n0 + 1 and LAST.value == work and LAST_XCD.value == xcd


def test_split_kv_plans_two_launches():
    r = _desc("striped", 1 << 17, 16, 8, 8, first=15, kv_splits=4)
    nws = ra.ra_ring_workspace_bytes(r)
    assert nws == 4 * 8 * 8192 * 129 * 4
    n0 = _calls()
    assert ra._lib.ra_ring_fwd(ctypes.byref(r), P, P, P, P, P, P, nws, None) == ra.RA_OK
    assert _calls() == n0 + 2 and LAST.value == 8 * 8192   # the merge runs over every query row


def test_backward_plans_three_launches():
    r = _desc("zigzag", 1 << 20, 32, 32, 8)
    nws = ra.ra_ring_bwd_workspace_bytes(r)
    assert nws == 2 * 32 * 32768 * 4
    n0 = _calls()
    assert ra._lib.ra_ring_bwd(ctypes.byref(r), P, P, P, P, P, P, P, P, P, P, nws, None) == ra.RA_OK
    # prep, dQ, dK/dV (8 KV heads x 64 segments x 64 tiles of 256 keys)
    assert _calls() == n0 + 3 and LAST.value == 8 * 64 * 64


def test_backward_without_allocation_plans_three_launches():
    r = _desc("zigzag", 1 << 20, 32, 32, 8)
    n0 = _calls()
    assert ra._lib.ra_ring_bwd_noalloc(ctypes.byref(r), P, P, P, P, P, P, P, P, P, None) == ra.RA_OK
    assert _calls() == n0 + 3 and LAST.value == 8 * 64 * 64
    big = _desc("zigzag", 1 << 20, 32, 32, 8, count=3)   # 3 x 2^20 query rows x heads: 24 MiB
    assert ra._lib.ra_ring_bwd_noalloc(ctypes.byref(big), P, P, P, P, P, P, P, P, P, None) == ra.RA_ERR_UNSUPPORTED
    assert _calls() == n0 + 3


def test_step_chunk_and_row_kernels():
    r = _desc("zigzag", 1 << 20, 32, 32, 8)
    n0 = _calls()
    for t in range(32):
        assert ra._lib.ra_ring_step(ctypes.byref(r), t, P, P, P, P, P, P, None) == ra.RA_OK
    assert _calls() == n0 + 32
    a = r.attn
    assert ra._lib.ra_chunk_fwd(ctypes.byref(a), P, P, P, P, P, P, -5, 1, None) == ra.RA_OK
    assert ra._lib.ra_state_init(ctypes.byref(a), P, P, P, None) == ra.RA_OK
    assert ra._lib.ra_finalize(ctypes.byref(a), P, P, P, P, P, None) == ra.RA_OK
    assert ra._lib.ra_merge(ctypes.byref(a), P, P, P, P, P, P, None) == ra.RA_OK
    assert ra._lib.ra_permute(2, 1, 1, 8, 1 << 20, 32, 128, ra.RA_BF16, P, P + (1 << 30), None) == ra.RA_OK
    assert LAST.value == 8 << 20
    # [B, S, H, d] source read through strides, into a chunk-major destination
    S, H, d = 1 << 20, 8, 128
    assert ra._lib.ra_permute_strided(2, 1, 1, H, S, 32, d, ra.RA_BF16, P, S * H * d, d, H * d,
                                      P + (1 << 30), H * S * d, S * d, d, None) == ra.RA_OK
    assert LAST.value == H * S
    f = _desc("contiguous", 32, 4, 1, 1, causal=0, count=4, in_dtype=ra.RA_F32, d=16)
    assert ra._lib.ra_ring_fwd(ctypes.byref(f), P, P, P, P, P, None, 0, None) == ra.RA_OK


def test_schedule_and_positions_at_full_size():
    r = _desc("zigzag", 1 << 20, 32, 32, 8)
    tasks = ra.ra_ring_schedule(r, 0)
    assert len(tasks) == 32 * 4
    pos = ra.ra_layout_positions("zigzag", 1 << 20, 32, 31)
    assert pos[0] == 31 * 16384 and pos[-1] == 32 * 16384 + 16383
    for lay in ("contiguous", "striped"):
        p = np.concatenate([ra.ra_layout_positions(lay, 1 << 17, 16, c) for c in range(16)])
        assert np.array_equal(np.sort(p), np.arange(1 << 17))
