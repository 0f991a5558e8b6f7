"""Pins of the CPU oracle to the pages' worked examples and to their closed forms.

Each example comes from tests/golden/page_examples.json (printed page values,
with the page and example cited there). Every example is also checked
against its closed form, written out by hand below with math.exp, to 1e-12.
"""
import math

import numpy as np
import pytest

from oracle import attention as orc
from exact_io_aware_17_amd import workloads

E = math.exp
INF = float("inf")


def _f(x):
    if isinstance(x, str):
        return float(x)
    if isinstance(x, list):
        return [_f(y) for y in x]
    return float(x)


def _close(got, want, tol):
    got = np.atleast_1d(np.asarray(got, dtype=np.float64))
    want = np.atleast_1d(np.asarray(want, dtype=np.float64))
    assert got.shape == want.shape, (got, want)
    assert np.all(np.abs(got - want) <= tol), (got, want, tol)


def _weights(scores):
    """Softmax weights read through the oracle: identity values make O the weights."""
    n = len(scores)
    o, _, _, _ = orc.softmax_row_output(scores, np.eye(n))
    return o


# Closed forms of each row example, derived by hand from the definition.
def _closed_row(eid):
    if eid == "safe_softmax_3552":
        l = E(-2) + 1 + 1 + E(-3)
        return {"m": 5, "l": l, "O": (10 * E(-2) + 20 + 30 + 40 * E(-3)) / l,
                "p": [E(-2) / l, 1 / l, 1 / l, E(-3) / l]}
    if eid == "all_equal_5555":
        return {"m": 5, "l": 4.0, "O": 25.0}
    if eid == "overflow_800_801":
        l = 1 + E(-1)
        return {"m": 801, "l": l, "O": (10 * E(-1) + 20) / l, "p": [E(-1) / l, 1 / l]}
    if eid == "cell_D_causal":
        l = 1 + E(-1)
        return {"m": 2, "l": l, "O": (10 + 20 * E(-1)) / l, "p": [1 / l, E(-1) / l, 0, 0]}
    if eid == "cell_D2_fully_masked":
        return {"l": 0.0, "O": 0.0}
    if eid == "cell_E_single_block":
        l = 1 + E(-2) + E(-3)
        ot = 10 + 20 * E(-2) + 30 * E(-3)
        return {"m": 3, "l": l, "O_tilde": ot, "O": ot / l}
    if eid.startswith("cell_F_x"):
        x = float(eid[len("cell_F_x"):])
        return {"l": 1 + E(-x), "O": (10 + 20 * E(-x)) / (1 + E(-x))}
    raise KeyError(eid)


def test_row_examples_printed_and_closed_form(golden):
    for ex in golden["row_examples"]:
        s = _f(ex["scores"])
        vals = ex["values"]
        o, m, l, lse = orc.softmax_row_output(s, vals)
        got = {"m": m, "l": l, "O": o[0]}
        if "p" in ex["printed"]:
            got["p"] = _weights(s)
        if "O_tilde" in ex["printed"]:
            got["O_tilde"] = o[0] * l
        for key, want in ex["printed"].items():
            _close(got[key], want, ex["tol"][key])
        closed = _closed_row(ex["id"])
        for key, want in closed.items():
            _close(got[key] if key in got else None, want, 1e-12 * max(1.0, abs(np.max(want))))
        # The streaming recurrence gives the same row at any block size.
        for blk in (1, 2, len(s)):
            o2, m2, l2, _ = orc.online_row(s, vals, blk)
            _close(o2, o, 1e-12 * max(1.0, np.max(np.abs(o))))


def test_overflow_example_naive_exp_is_nan():
    """Exercises: the unshifted exponentials of 800 and 801 overflow (inf/inf = NaN)."""
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(np.array([800.0, 801.0]))
        naive = (e @ np.array([10.0, 20.0])) / e.sum()
    assert np.isinf(e).all() and np.isnan(naive)
    o, _, _, _ = orc.softmax_row_output([800.0, 801.0], [10.0, 20.0])
    assert np.isfinite(o).all()


def test_cell_F_is_monotone_toward_the_dominant_value():
    xs = [0, 1, 2, 4, 10, 30, 100]
    outs = [orc.softmax_row_output([x, 0.0], [10.0, 20.0])[0][0] for x in xs]
    assert all(a > b for a, b in zip(outs, outs[1:]) if b != 10.0)
    assert outs[-1] == 10.0


def _closed_two_block(eid):
    if eid == "equal_max_merge_3552":
        return {"m": 5, "l": E(-2) + 1 + 1 + E(-3), "l1": E(-2) + 1, "l2": 1 + E(-3)}
    if eid == "cell_A":
        l = 1 + E(-1) + 1 + E(-2)
        ot = 10 + 20 * E(-1) + 30 + 40 * E(-2)
        return {"m": 2, "l": l, "O_tilde": ot, "O": ot / l}
    if eid in ("cell_B", "cell_H_reverse"):
        l = E(-2) + E(-3) + 1 + E(-1)
        ot = 10 * E(-2) + 20 * E(-3) + 30 + 40 * E(-1)
        return {"m": 3, "l": l, "O_tilde": ot, "O": ot / l}
    if eid == "cell_C":
        return {"m": 5, "l": 4.0, "O_tilde": 100.0, "O": 25.0}
    if eid == "cell_D_blocks":
        l = 1 + E(-1)
        return {"m": 2, "l": l, "O": (10 + 20 * E(-1)) / l}
    if eid == "cell_D2_blocks":
        return {"l": 0.0, "O": 0.0}
    if eid == "two_d_example":
        w = np.array([E(-1), E(-3), 1.0, E(-2)])
        vals = np.array([[1, 0], [0, 1], [1, 1], [2, 0]], dtype=float)
        return {"m": 3, "l": w.sum(), "O": (w @ vals) / w.sum()}
    raise KeyError(eid)


def test_two_block_examples_printed_and_closed_form(golden):
    for ex in golden["two_block_examples"]:
        b1, b2 = _f(ex["blocks"][0]), _f(ex["blocks"][1])
        vals = np.asarray(ex["values"], dtype=float)
        if vals.ndim == 1:
            vals = vals[:, None]
        n1 = len(b1)
        st1 = orc.block_state(b1, vals[:n1])
        st2 = orc.block_state(b2, vals[n1:])
        m, l, ot = orc.merge(st1, st2)
        o, lse = orc.finalize((m, l, ot))
        got = {"m1": st1[0], "l1": st1[1], "O_tilde1": st1[2], "m2": st2[0], "l2": st2[1],
               "O_tilde2": st2[2], "m": m, "l": l, "O_tilde": ot, "O": o}
        if st1[0] != -INF:
            got["factor1"] = E(st1[0] - m) if m != -INF else 0.0
        if st2[0] != -INF:
            got["factor2"] = E(st2[0] - m) if m != -INF else 0.0
        for key, want in ex["printed"].items():
            _close(got[key], want, ex["tol"][key])
        for key, want in _closed_two_block(ex["id"]).items():
            _close(got[key], want, 1e-12 * max(1.0, float(np.max(np.abs(want)))))
        # The same numbers from the streaming form and from the plain definition.
        s_all = b1 + b2
        o_on, m_on, l_on, _ = orc.online_row(s_all, vals, n1)
        o_def, m_def, l_def, _ = orc.softmax_row_output(s_all, vals)
        _close(o_on, o, 1e-12 * max(1.0, float(np.max(np.abs(o)))))
        _close(o_def, o, 1e-12 * max(1.0, float(np.max(np.abs(o)))))


def test_two_d_direct_check(golden):
    ex = golden["two_d_direct"]
    o, m, l, _ = orc.softmax_row_output(ex["scores"], ex["values"])
    _close(l, ex["printed"]["l"], ex["tol"]["l"])
    _close(_weights(ex["scores"]), ex["printed"]["p"], ex["tol"]["p"])
    _close(o, ex["printed"]["O"], ex["tol"]["O"])


def test_state_merges(golden):
    for ex in golden["state_merges"]:
        states = [(float(m), float(l), np.asarray(o, dtype=float)) for m, l, o in ex["states"]]
        if ex["id"] == "unequal_max_states":
            m, l, ot = orc.merge(states[0], states[1])
            o, _ = orc.finalize((m, l, ot))
            got = {"m": m, "l": l, "O_tilde": ot, "O": o}
            closed_l = 1.8 + 3.0 * E(-4)
            closed = {"m": 6, "l": closed_l,
                      "O": (np.array([1.8, 0.9]) + E(-4) * np.array([6.0, 3.0])) / closed_l}
        else:
            s12 = orc.merge(states[0], states[1])
            s123 = orc.merge(s12, states[2])
            got = {"l_after_2": s12[1], "m": s123[0], "l": s123[1]}
            closed = {"l_after_2": 1.5 * E(-3) + 2.0,
                      "l": 1.5 * E(-3) + 2.0 + 1.2 * E(-2), "m": 7}
            # Any grouping and any order give the same state (associativity).
            for a, b, c in [(0, 1, 2), (2, 1, 0), (1, 2, 0), (2, 0, 1)]:
                alt = orc.merge(orc.merge(states[a], states[b]), states[c])
                alt2 = orc.merge(states[a], orc.merge(states[b], states[c]))
                for st in (alt, alt2):
                    assert st[0] == 7 and abs(st[1] - s123[1]) < 1e-14
        for key, want in ex["printed"].items():
            _close(got[key], want, ex["tol"][key])
        for key, want in closed.items():
            _close(got[key], want, 1e-12)


def test_red_team_mutation_is_caught(golden):
    """Dropping exp(m_old - m_new) changes Cell B's answer; the checks must see it."""
    ex = next(e for e in golden["two_block_examples"] if e["id"] == "cell_B")
    b1, b2 = ex["blocks"]
    vals = np.asarray(ex["values"], dtype=float)
    st1 = orc.block_state(b1, vals[:2])
    st2 = orc.block_state(b2, vals[2:])
    o_bad, _ = orc.finalize(orc.merge(st1, st2, rescale=False))
    assert abs(o_bad[0] - ex["printed"]["O"]) > 1.0
    o_bad2, _, _, _ = orc.online_row(b1 + b2, vals, 2, rescale=False)
    assert abs(o_bad2[0] - ex["printed"]["O"]) > 1.0
    # With equal maxima (Cell A) the factors are all 1, so the mutation is invisible there.
    exa = next(e for e in golden["two_block_examples"] if e["id"] == "cell_A")
    o_a, _, _, _ = orc.online_row(exa["blocks"][0] + exa["blocks"][1], exa["values"], 2,
                                   rescale=False)
    assert abs(o_a[0] - exa["printed"]["O"]) < 2e-4


def test_measurement_arithmetic(golden):
    for ex in golden["arithmetic"]:
        if ex["id"] == "score_matrix_2048":
            assert workloads.score_matrix_bytes(ex["N"], 4) == ex["bytes"]
        elif ex["id"] == "quadratic_share_4096_64":
            assert abs(workloads.quadratic_share(ex["N"], ex["d"]) - ex["share"]) <= ex["tol"]
        elif ex["id"] == "cell_G_flash_bytes":
            assert ex["floats_per_row"] * ex["N"] * ex["H"] * ex["L"] * 4 == ex["bytes"]
        elif ex["id"] == "cell_G_standard_bytes":
            per_head = workloads.score_matrix_bytes(ex["N"], 4)
            assert per_head == ex["bytes_per_head"]
            assert per_head * ex["H"] * ex["L"] == ex["gib_total"] * 2 ** 30
