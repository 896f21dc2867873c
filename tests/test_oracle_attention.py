"""Pins for the float64 oracle's attention routines (CPU only).

Each check ties the oracle to something other than itself: a value the pages
print, a library routine, a closed form or brute force.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import synthetic
from oracle import attention as A
from oracle import layout as LY

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = v
    return vals


# ---------------------------------------------------------------------------
# The pages' own experiment
# ---------------------------------------------------------------------------

def test_glossary_four_device_simulation():
    """The glossary page's four-device experiment (Ultralytics glossary page
    "Ring Attention", section "How Ring Attention works") on its own draw, in
    fp32: device i holds query block i and, at step t, key/value block
    (i - t) mod 4; it adds the unnormalized exponentials of its scaled scores
    to a numerator and a denominator.  The page reports that the result
    matches full softmax attention at atol 1e-5; the oracle must agree with
    the simulated devices and with the fp32 full softmax at that tolerance."""
    g = _read_golden("glossary_four_device_simulation.txt")
    nd, blk, dim, atol = int(g["n_devices"]), int(g["block"]), int(g["dim"]), float(g["atol"])
    q, k, v = synthetic.tiny_sim_draw()
    assert q.shape == (nd * blk, dim)
    # which KV block each device holds at each step (the ring order), as one table
    visit = (torch.arange(nd)[:, None] - torch.arange(nd)[None, :]) % nd          # [device, step]
    q_dev = q.view(nd, blk, dim)                                                   # [device, row, dim]
    k_held, v_held = k.view(nd, blk, dim)[visit], v.view(nd, blk, dim)[visit]    # [device, step, key, dim]
    # every device's step-wise weights at once: 8 x 8 score blocks, unnormalized
    w_steps = torch.exp(torch.einsum("irc,itkc->itrk", q_dev, k_held) / math.sqrt(dim))
    numer = torch.einsum("itrk,itkc->irc", w_steps, v_held)                       # summed over steps
    denom = w_steps.sum(dim=(1, 3)).unsqueeze(-1)
    sim = (numer / denom).reshape(nd * blk, dim)
    full32 = torch.softmax(q @ k.T / math.sqrt(dim), dim=-1) @ v
    verdict = torch.allclose(sim, full32, atol=atol)
    assert str(verdict) == g["verdict"]
    assert tuple(w_steps.shape[2:]) == tuple(int(x) for x in g["score_block"].split("x"))

    shp = (1, 1, nd * blk, dim)
    ref, lse = A.attention_reference(q.reshape(shp), k.reshape(shp), v.reshape(shp))
    assert np.max(np.abs(ref[0, 0] - sim.double().numpy())) <= atol
    assert np.max(np.abs(ref[0, 0] - full32.double().numpy())) <= atol

    # the oracle's own ring loop on the same draw: chunks in ring order
    pos = [LY.chunk_positions("contiguous", nd * blk, nd, c) for c in range(nd)]
    qc = [q.reshape(shp)[:, :, c * blk:(c + 1) * blk] for c in range(nd)]
    kc = [k.reshape(shp)[:, :, c * blk:(c + 1) * blk] for c in range(nd)]
    vc = [v.reshape(shp)[:, :, c * blk:(c + 1) * blk] for c in range(nd)]
    ring = A.ring_attention(qc, kc, vc, pos, query_chunks=list(range(nd)), causal=False)
    ring_out = np.concatenate([o for o, _ in ring], axis=2)
    assert np.max(np.abs(ring_out[0, 0] - sim.double().numpy())) <= atol
    assert np.max(np.abs(ring_out - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# Library routine: torch float64 scaled_dot_product_attention
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, mask=None, causal=False, gqa=False):
    import torch.nn.functional as F
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                          attn_mask=None if mask is None else torch.from_numpy(mask),
                                          is_causal=causal, enable_gqa=gqa).numpy()


@pytest.mark.parametrize("hq,hkv,lq,lk,d,causal", [
    (2, 2, 37, 37, 16, False), (2, 2, 37, 37, 16, True), (4, 2, 29, 29, 32, True),
    (8, 2, 40, 40, 8, False), (3, 3, 17, 53, 16, False), (4, 1, 33, 33, 24, True)])
def test_reference_matches_torch_sdpa(hq, hkv, lq, lk, d, causal):
    rng = np.random.default_rng(hq * 1000 + lq)
    q = rng.standard_normal((2, hq, lq, d))
    k = rng.standard_normal((2, hkv, lk, d))
    v = rng.standard_normal((2, hkv, lk, d + 3))
    out, _ = A.attention_reference(q, k, v, causal=causal)
    ref = _sdpa(q, k, v, causal=causal, gqa=hq != hkv)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("layout", LY.LAYOUTS)
def test_reference_position_mask_matches_sdpa(layout):
    S, N, d = 48, 4, 16
    rng = np.random.default_rng(7)
    pos = LY.all_positions(layout, S, N)
    q = rng.standard_normal((1, 2, S, d))
    k = rng.standard_normal((1, 2, S, d))
    v = rng.standard_normal((1, 2, S, d))
    out, _ = A.attention_reference(q, k, v, causal=True, q_pos=pos, k_pos=pos)
    mask = pos[None, :] <= pos[:, None]
    ref = _sdpa(q, k, v, mask=mask)
    assert np.max(np.abs(out - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_first_causal_row_is_its_own_value():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 1, 9, 8)) for _ in range(3))
    out, lse = A.attention_reference(q, k, v, causal=True)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0])
    assert lse[0, 0, 0] == pytest.approx(float(q[0, 0, 0] @ k[0, 0, 0]) / math.sqrt(8), abs=1e-15)


def test_identical_keys_average_visible_values():
    rng = np.random.default_rng(2)
    L, d = 11, 6
    q = rng.standard_normal((1, 1, L, d))
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), L, axis=2)
    v = rng.standard_normal((1, 1, L, d))
    out, _ = A.attention_reference(q, k, v, causal=True)
    for t in range(L):
        assert np.allclose(out[0, 0, t], v[0, 0, :t + 1].mean(axis=0), atol=1e-14, rtol=0)
    out_nc, _ = A.attention_reference(q, k, v, causal=False)
    assert np.allclose(out_nc[0, 0], v[0, 0].mean(axis=0), atol=1e-14, rtol=0)


def test_one_hot_values_return_probabilities():
    rng = np.random.default_rng(3)
    Lq, Lk, d = 7, 13, 5
    q = rng.standard_normal((1, 1, Lq, d))
    k = rng.standard_normal((1, 1, Lk, d))
    v = np.eye(Lk)[None, None]
    out, lse = A.attention_reference(q, k, v)
    s = q[0, 0] @ k[0, 0].T / math.sqrt(d)
    assert np.max(np.abs(out[0, 0] - scipy.special.softmax(s, axis=1))) <= 1e-15
    assert np.max(np.abs(lse[0, 0] - scipy.special.logsumexp(s, axis=1))) <= 1e-13


def test_score_shift_leaves_output_and_shifts_lse():
    rng = np.random.default_rng(4)
    d, c, sc = 8, 37.25, 0.5
    q = rng.standard_normal((1, 1, 6, d))
    k = rng.standard_normal((1, 1, 9, d))
    v = rng.standard_normal((1, 1, 9, d))
    out, lse = A.attention_reference(q, k, v, scale=sc)
    q2 = np.concatenate([q, np.full((1, 1, 6, 1), c / sc)], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 1, 9, 1))], axis=-1)
    out2, lse2 = A.attention_reference(q2, k2, v, scale=sc)
    assert np.max(np.abs(out2 - out)) <= 1e-13
    assert np.max(np.abs(lse2 - (lse + c))) <= 1e-12


def _brute(q, k, v, qpos, kpos, causal, scale):
    """Pure-Python loops with math.exp: tiny cases only."""
    Lq, d = len(q), len(q[0])
    out, lse = [], []
    for t in range(Lq):
        sc = []
        for u in range(len(k)):
            if causal and kpos[u] > qpos[t]:
                continue
            sc.append((sum(q[t][e] * k[u][e] for e in range(d)) * scale, u))
        if not sc:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        mx = max(s for s, _ in sc)
        den = sum(math.exp(s - mx) for s, _ in sc)
        out.append([sum(math.exp(s - mx) * v[u][e] for s, u in sc) / den for e in range(len(v[0]))])
        lse.append(mx + math.log(den))
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_reference_matches_brute_force(causal, seed):
    rng = np.random.default_rng(100 + seed)
    Lq, Lk, d, dv = 5, 12, 4, 3          # Lq != Lk and d != dv catch transposed operands
    q = rng.standard_normal((Lq, d)) * 2
    k = rng.standard_normal((Lk, d)) * 2
    v = rng.standard_normal((Lk, dv))
    qpos = rng.permutation(12)[:Lq]
    kpos = rng.permutation(12)
    scale = 0.7
    bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), qpos.tolist(), kpos.tolist(), causal, scale)
    out, lse = A.attention_reference(q[None, None], k[None, None], v[None, None], scale=scale,
                                     causal=causal, q_pos=qpos, k_pos=kpos)
    assert np.max(np.abs(out[0, 0] - np.array(bo))) <= 1e-13
    assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(np.array(bl)))
    fin = ~np.isinf(np.array(bl))
    assert np.max(np.abs(lse[0, 0][fin] - np.array(bl)[fin]), initial=0) <= 1e-13


def test_unseen_row_gives_zero_and_neg_inf():
    q = np.ones((1, 1, 2, 4))
    k = np.ones((1, 1, 3, 4))
    v = np.ones((1, 1, 3, 4))
    out, lse = A.attention_reference(q, k, v, causal=True, q_pos=[0, 5], k_pos=[3, 4, 5])
    assert np.all(out[0, 0, 0] == 0) and lse[0, 0, 0] == -np.inf
    assert np.allclose(out[0, 0, 1], 1.0)


# ---------------------------------------------------------------------------
# Log-sum-exp associativity and the merge
# ---------------------------------------------------------------------------

def test_lecture_lse_notebook_check():
    g = _read_golden("lecture013_lse_check.txt")
    rng = np.random.default_rng(5)
    x = rng.standard_normal(int(g["length"])) * 3
    x1, x2 = np.array_split(x, int(g["split"]))
    m1, m2 = x1.max(), x2.max()
    m = max(m1, m2)
    l1 = math.exp(m1 - m) * np.exp(x1 - m1).sum()
    l2 = math.exp(m2 - m) * np.exp(x2 - m2).sum()
    s1 = scipy.special.softmax(x1)
    s2 = scipy.special.softmax(x2)
    combined = np.concatenate([s1 * (l1 / (l1 + l2)), s2 * (l2 / (l1 + l2))])
    assert (np.max(np.abs(combined - scipy.special.softmax(x))) <= 1e-15) == (g["expect_equal_to_full_softmax"] == "True")
    # the oracle's merge does the same reweighting through lse values
    d = 1
    lse, o = A.lse_merge(np.array([scipy.special.logsumexp(x1)]), np.zeros((1, d)),
                         np.array([scipy.special.logsumexp(x2)]), np.zeros((1, d)))
    assert abs(lse[0] - scipy.special.logsumexp(x)) <= 1e-14


from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(-1000, 1000, allow_nan=False), min_size=2, max_size=40), st.integers(1, 39), st.data())
def test_lse_split_identity(xs, cut, data):
    x = np.array(xs)
    cut = min(cut, len(x) - 1)
    # some entries may be -inf (masked keys)
    ninf = data.draw(st.lists(st.integers(0, len(x) - 1), max_size=3))
    x[ninf] = -np.inf
    x1, x2 = x[:cut], x[cut:]
    lse, _ = A.lse_merge(np.array([scipy.special.logsumexp(x1)]), np.zeros((1, 1)),
                         np.array([scipy.special.logsumexp(x2)]), np.zeros((1, 1)))
    ref = scipy.special.logsumexp(x)
    if np.isinf(ref):
        assert lse[0] == -np.inf
    else:
        assert abs(lse[0] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_merge_weights_match_library_softmax():
    rng = np.random.default_rng(6)
    la, lb = rng.standard_normal(50) * 20, rng.standard_normal(50) * 20
    oa, ob = rng.standard_normal((50, 4)), rng.standard_normal((50, 4))
    lse, o = A.lse_merge(la, oa, lb, ob)
    w = scipy.special.softmax(np.stack([la, lb], axis=1), axis=1)
    assert np.max(np.abs(o - (w[:, :1] * oa + w[:, 1:] * ob))) <= 1e-14
    assert np.max(np.abs(lse - scipy.special.logsumexp(np.stack([la, lb], 1), axis=1))) <= 1e-13


def test_merge_identity_commutative_associative():
    rng = np.random.default_rng(8)
    n, d = 64, 5
    parts = [(rng.standard_normal(n) * 30, rng.standard_normal((n, d))) for _ in range(3)]
    empty = (np.full(n, -np.inf), np.zeros((n, d)))
    a, b, c = parts
    l1, o1 = A.lse_merge(*a, *empty)
    assert np.array_equal(l1, a[0]) and np.max(np.abs(o1 - a[1])) == 0
    lab, oab = A.lse_merge(*a, *b)
    lba, oba = A.lse_merge(*b, *a)
    assert np.max(np.abs(lab - lba)) <= 1e-12 and np.max(np.abs(oab - oba)) <= 1e-12
    left = A.lse_merge(*A.lse_merge(*a, *b), *c)
    right = A.lse_merge(*a, *A.lse_merge(*b, *c))
    assert np.max(np.abs(left[0] - right[0])) <= 1e-12 and np.max(np.abs(left[1] - right[1])) <= 1e-12
    le, oe = A.lse_merge(*empty, *empty)
    assert np.all(le == -np.inf) and np.all(oe == 0)


def test_merge_of_disjoint_key_sets_equals_joint_attention():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 2, 10, 8))
    k = rng.standard_normal((1, 2, 30, 8))
    v = rng.standard_normal((1, 2, 30, 8))
    perm = rng.permutation(30)
    a_idx, b_idx = perm[:11], perm[11:]
    oa, la = A.attention_reference(q, k[:, :, a_idx], v[:, :, a_idx])
    ob, lb = A.attention_reference(q, k[:, :, b_idx], v[:, :, b_idx])
    lse, o = A.lse_merge(la, oa, lb, ob)
    ref_o, ref_l = _sdpa(q, k, v), scipy.special.logsumexp(q @ k.transpose(0, 1, 3, 2) / math.sqrt(8), axis=-1)
    assert np.max(np.abs(o - ref_o)) <= 1e-12 and np.max(np.abs(lse - ref_l)) <= 1e-12
