"""Planted mistakes in copies of the oracle must be caught by the pins.

Each mutation edits the source text of one oracle module (a dropped term, a
wrong sign or index, a transposed operand), loads the edited copy under a
fresh name and runs the pin tests against it with the module swapped in.  At
least one pin must fail for every mutation.  The real oracle is untouched.
"""
import os
import types

import pytest

import tests.test_oracle_attention as TA
import tests.test_oracle_ring as TR

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _load(fname, old, new):
    src = open(os.path.join(ORACLE, fname)).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_" + fname[:-3])
    mod.__dict__["__name__"] = mod.__name__
    exec(compile(src, f"<mutant {fname}>", "exec"), mod.__dict__)
    return mod


def _pins(A, LY):
    """Run the pins with the given modules; return the number that fail."""
    saved = (TA.A, TA.LY, TR.A, TR.LY)
    TA.A, TA.LY, TR.A, TR.LY = A, LY, A, LY
    calls = [
        lambda: TA.test_glossary_four_device_simulation(),
        lambda: TA.test_reference_matches_torch_sdpa(4, 2, 29, 29, 32, True),
        lambda: TA.test_reference_matches_torch_sdpa(3, 3, 17, 53, 16, False),
        lambda: TA.test_reference_position_mask_matches_sdpa("zigzag"),
        lambda: TA.test_reference_matches_brute_force(True, 0),
        lambda: TA.test_first_causal_row_is_its_own_value(),
        lambda: TA.test_merge_weights_match_library_softmax(),
        lambda: TA.test_merge_of_disjoint_key_sets_equals_joint_attention(),
        lambda: TR.test_ring_equals_definition_and_merge_route("striped", True, 4, 2),
        lambda: TR.test_ring_equals_definition_and_merge_route("zigzag", True, 2, 2),
        lambda: TR.test_chunk_update_with_schedule_deltas_equals_definition("zigzag"),
        lambda: TR.test_chunk_update_noncausal_order_invariance(),
        lambda: TR.test_chunk_update_fully_masked_rows_stay_empty(),
        lambda: TR.test_layout_closed_forms(),
        lambda: TR.test_schedule_delta_and_kind_match_brute_force("zigzag", 64, 4),
        lambda: TR.test_schedule_delta_and_kind_match_brute_force("contiguous", 4, 4),
        lambda: TR.test_schedule_delta_and_kind_match_brute_force("striped", 64, 4),
        lambda: TR.test_visible_pair_closed_forms(64, 4),
        lambda: TR.test_ring_order_matches_pass_to_next_device(4),
    ]
    failed = 0
    try:
        for c in calls:
            try:
                c()
            except Exception:
                failed += 1
    finally:
        TA.A, TA.LY, TR.A, TR.LY = saved
    return failed


MUTATIONS = [
    # attention.py
    ("attention.py", "s = (q[b, h, r0:r1] @ K.T) * scale", "s = (q[b, h, r0:r1] @ K.T)"),
    ("attention.py", "kp[None, :] <= qp[r0:r1, None]", "kp[None, :] < qp[r0:r1, None]"),
    ("attention.py", "return h // (hq // hkv)", "return h % hkv"),
    ("attention.py", "num = p @ V", "num = p @ K"),
    ("attention.py", "l[b, h] = np.where(live, alpha * l[b, h] + p.sum(axis=1), l[b, h])",
     "l[b, h] = np.where(live, l[b, h] + p.sum(axis=1), l[b, h])"),
    ("attention.py", "hide = (kcol - prow > delta)", "hide = (prow - kcol > delta)"),
    ("attention.py", "a = np.where(old > NEG_INF, np.exp(np.where(old > NEG_INF, old, 0.0) - mn), 0.0)",
     "a = np.where(old > NEG_INF, np.exp(mn - np.where(old > NEG_INF, old, 0.0)), 0.0)"),
    ("attention.py", "for t in range(N):\n            j = (i - t) % N\n            kj", "for t in range(N - 1):\n            j = (i - t) % N\n            kj"),
    ("attention.py", "lse = np.where(seen, m + np.log(ls), NEG_INF)", "lse = np.where(seen, m * np.log(ls), NEG_INF)"),
    ("attention.py", "o = wa[..., None] * oa + wb[..., None] * ob", "o = wa[..., None] * oa + wa[..., None] * ob"),
    # layout.py
    ("layout.py", "return rows * N + c", "return rows * N + (N - 1 - c)"),
    ("layout.py", "late = (2 * N - 1 - c) * s", "late = (2 * N - 2 - c) * s + 0 * c"),
    ("layout.py", "return int((int(qpos[0]) - int(kpos[0])) // g)", "return int((int(kpos[0]) - int(qpos[0])) // g)"),
    ("layout.py", "if kpos.min() > qpos.max():", "if kpos.min() > qpos.min():"),
    ("layout.py", "if kpos.max() <= qpos.min():", "if kpos.max() < qpos.min():"),
    ("layout.py", "return [(i - t) % N for t in range(N)]", "return [(i + t) % N for t in range(N)]"),
]


def test_unmutated_oracle_passes_all_pins():
    import oracle.attention as A
    import oracle.layout as LY
    assert _pins(A, LY) == 0


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_mutation_is_caught(fname, old, new):
    import oracle.attention as A
    import oracle.layout as LY
    mut = _load(fname, old, new)
    failed = _pins(mut, LY) if fname == "attention.py" else _pins(A, mut)
    assert failed >= 1, f"no pin caught the mutation {old!r} -> {new!r}"


# ---------------------------------------------------------------------------
# backward.py
# ---------------------------------------------------------------------------

import tests.test_oracle_backward as TB  # noqa: E402


def _load_backward(old, new):
    src = open(os.path.join(ORACLE, "backward.py")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_mutant_backward")
    exec(compile(src, "<mutant backward.py>", "exec"), mod.__dict__)
    return mod


def _pins_backward(BW):
    saved = TB.BW
    TB.BW = BW
    calls = [
        lambda: TB.test_gradient_matches_finite_differences(True, 4, 2),
        lambda: TB.test_gradient_matches_finite_differences(False, 1, 1),
        lambda: TB.test_key_shift_invariance_and_value_sum(True),
        lambda: TB.test_single_key_and_uniform_rows(),
        lambda: TB.test_ring_order_equals_definition("zigzag", True, [2]),
        lambda: TB.test_ring_order_equals_definition("striped", False, [0, 1, 2, 3]),
    ]
    failed = 0
    try:
        for c in calls:
            try:
                c()
            except Exception:
                failed += 1
    finally:
        TB.BW = saved
    return failed


BACKWARD_MUTATIONS = [
    # a dropped term, a wrong sign, transposed operands, a missing scale, the
    # wrong head sum, a skipped ring step, a wrong lse use
    ("dS = P * (dP - D[:, None]) * scale", "dS = P * dP * scale"),
    ("dS = P * (dP - D[:, None]) * scale", "dS = P * (D[:, None] - dP) * scale"),
    ("dvv[b, g] += P.T @ dout[b, h]", "dvv[b, g] += P.T @ q[b, h]"),
    ("dq[b, h] = dS @ K", "dq[b, h] = dS @ V"),
    ("dk[b, g] += dS.T @ q[b, h]", "dk[b, g] = dS.T @ q[b, h]"),
    ("dP = dout[b, h] @ V.T", "dP = dout[b, h] @ K.T"),
    ("D = (dout[b, h] * out).sum(axis=1)", "D = (dout[b, h] * out).sum(axis=0).mean() + 0 * out[:, 0]"),
    ("dS = P * (dP - D[b, h][:, None]) * sc", "dS = P * (dP - D[b, h][:, None])"),
    ("for t in range(N):\n            j = (i - t) % N\n            kpos", "for t in range(N - 1):\n            j = (i - t) % N\n            kpos"),
    ("np.exp(s - np.where(fin, lse, 0.0)[:, None])", "np.exp(s + np.where(fin, lse, 0.0)[:, None])"),
    ("dk[j][b, g] += dS.T @ qi[b, h]", "dk[j][b, g] += dS.T @ doi[b, h]"),
]


def test_unmutated_backward_passes_all_pins():
    import oracle.backward as BW
    assert _pins_backward(BW) == 0


@pytest.mark.parametrize("old,new", BACKWARD_MUTATIONS, ids=[f"backward:{i}" for i in range(len(BACKWARD_MUTATIONS))])
def test_backward_mutation_is_caught(old, new):
    failed = _pins_backward(_load_backward(old, new))
    assert failed >= 1, f"no pin caught the mutation {old!r} -> {new!r}"
