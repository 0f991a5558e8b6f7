"""The pages' worked examples through the 16-bit matrix-core forward.

Each printed example (a row of scores against value vectors, or two blocks
of one) is embedded in Q, K, V so that the kernel that is timed (bf16 or
fp16 MFMA, lagged reference max, two normalisers) computes it: every query is
e_1, key j is s_j * e_1 (so its scaled score at scale 1 is s_j), and V holds
the example's values in its first columns. Keys that are not part of the
example get the score -1000, whose weight is exactly zero next to any of the
examples' scores, and zero values. Blocks of an example go to different
64-key blocks of the stream, so the merge between blocks runs in the kernel.

The outputs are compared with the printed values ("Exercises": the [3,5,5,2]
row, the equal-score row, the block merges, the 2-D example; "Worked
examples": Cells A-F and H), within the printed precision plus what 16-bit
arithmetic allows: the weights are rounded to the element type before P V
(moving O by at most u * max_j |v_j - O|, u the unit roundoff) and O is
rounded once more when written (u * |O|). The normaliser is checked through
lse = m + ln l, which the kernel forms from fp32 weights.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAD_SCORE = -1000.0
BLOCK = 64
UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def _exact(x, dtype) -> bool:
    return float(torch.tensor(float(x), dtype=dtype).double()) == float(x)


def _build(keys, N, d, dtype):
    """keys: list of (position, score, value vector). Returns q, k, v [1, 1, N, d]."""
    q = torch.zeros(1, 1, N, d, dtype=torch.float64)
    q[..., 0] = 1.0
    k = torch.zeros_like(q)
    k[..., 0] = PAD_SCORE
    v = torch.zeros_like(q)
    for pos, s, vec in keys:
        k[0, 0, pos, 0] = s
        v[0, 0, pos, :len(vec)] = torch.tensor(vec, dtype=torch.float64)
    return (t.to(dtype).to(DEV) for t in (q, k, v))


def _vecs(values):
    return [[float(x)] if not isinstance(x, list) else [float(y) for y in x] for x in values]


def _closed_form(scores, vecs):
    """O and lse of one row by the definition (fp64)."""
    s = np.array(scores, dtype=np.float64)
    m = s.max()
    p = np.exp(s - m)
    o = (p[:, None] * np.array(vecs)).sum(0) / p.sum()
    return o, m + math.log(p.sum())


def _check_row(o_row, lse_row, printed_o, o_tol, vecs, dtype, exact_o, exact_lse):
    u = UNIT[dtype]
    got = o_row[:len(exact_o)].double().cpu().numpy()
    spread = max(float(np.max(np.abs(np.array(vec) - exact_o))) for vec in vecs)
    tol = o_tol + u * spread + u * float(np.max(np.abs(exact_o))) + 1e-6
    want = np.atleast_1d(np.array(printed_o, dtype=np.float64))
    err = float(np.max(np.abs(got - want)))
    say(f"   O {got.tolist()} printed {want.tolist()} err {err:.3g} tol {tol:.3g}; "
        f"lse {float(lse_row):.7f} exact {exact_lse:.7f}")
    assert err <= tol
    # Normaliser: lse from fp32 weights, to fp32 accuracy.
    assert abs(float(lse_row) - exact_lse) <= 2e-6 * max(1.0, abs(exact_lse))


def _check_l(lse_val, m, ex):
    """The printed normaliser l = exp(lse - m): lse is fp32, so l carries
    lse's rounding, a few units of 2^-24 |lse| relative (3.8e-4 at lse = 801)."""
    lse_f = float(lse_val)
    l_gpu = math.exp(lse_f - m)
    tol = ex["tol"]["l"] + l_gpu * 8 * 2.0 ** -24 * max(1.0, abs(lse_f))
    say(f"   l {l_gpu:.7f} printed {ex['printed']['l']} tol {tol:.3g}")
    assert abs(l_gpu - ex["printed"]["l"]) <= tol


DTYPES = [torch.bfloat16, torch.float16]
DIMS = [64, 128]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", DIMS)
def test_row_examples(golden, dtype, d):
    for ex in golden["row_examples"]:
        if any(isinstance(s, str) for s in ex["scores"]):
            continue  # the masked rows run in test_masked_cells
        vecs = _vecs(ex["values"])
        if not all(_exact(s, dtype) for s in ex["scores"]) or \
                not all(_exact(x, dtype) for vec in vecs for x in vec):
            say(f"page example {ex['id']}: not exact in {dtype}, skipped")
            continue
        say(f"page example {ex['id']} ({dtype}, d={d})")
        keys = [(j, float(s), vec) for j, (s, vec) in enumerate(zip(ex["scores"], vecs))]
        q, k, v = _build(keys, 2 * BLOCK, d, dtype)
        o, lse = fa.fwd(q, k, v, scale=1.0)
        torch.cuda.synchronize()
        # Every query row is e_1, so every row is the example's row.
        assert torch.equal(o[0, 0], o[0, 0, :1].expand_as(o[0, 0]))
        exact_o, exact_lse = _closed_form(ex["scores"], vecs)
        _check_row(o[0, 0, 0], lse[0, 0, 0], ex["printed"]["O"], ex["tol"]["O"], vecs, dtype,
                   exact_o, exact_lse)
        if "l" in ex["printed"]:
            _check_l(lse[0, 0, 0], max(ex["scores"]), ex)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", DIMS)
def test_two_block_examples(golden, dtype, d):
    """The block merges: block 1 of an example in the first 64-key block of
    the stream, block 2 in the second (a block printed as all -inf gets
    scores of zero weight)."""
    for ex in golden["two_block_examples"]:
        blocks = ex["blocks"]
        if all(s == "-inf" for blk in blocks for s in blk):
            continue  # Cell D2's all-masked blocks run in test_masked_cells
        vecs = _vecs(ex["values"])
        keys, scores, used = [], [], []
        j = 0
        for bi, blk in enumerate(blocks):
            for pos, s in enumerate(blk):
                if s != "-inf":
                    keys.append((bi * BLOCK + pos, float(s), vecs[j]))
                    scores.append(float(s))
                    used.append(vecs[j])
                j += 1
        if not all(_exact(s, dtype) for s in scores) or \
                not all(_exact(x, dtype) for vec in used for x in vec):
            continue
        say(f"page example {ex['id']} ({dtype}, d={d})")
        q, k, v = _build(keys, 2 * BLOCK, d, dtype)
        o, lse = fa.fwd(q, k, v, scale=1.0)
        torch.cuda.synchronize()
        exact_o, exact_lse = _closed_form(scores, used)
        if "O" in ex["printed"]:
            _check_row(o[0, 0, 5], lse[0, 0, 5], ex["printed"]["O"], ex["tol"]["O"], used, dtype,
                       exact_o, exact_lse)
        else:  # the equal-max merge prints the sums only
            assert abs(float(lse[0, 0, 5]) - exact_lse) <= 2e-6 * max(1.0, abs(exact_lse))
        _check_l(lse[0, 0, 5], ex["printed"]["m"], ex)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", DIMS)
def test_two_d_direct(golden, dtype, d):
    ex = golden["two_d_direct"]
    vecs = _vecs(ex["values"])
    keys = [(j, float(s), vec) for j, (s, vec) in enumerate(zip(ex["scores"], vecs))]
    q, k, v = _build(keys, 2 * BLOCK, d, dtype)
    o, lse = fa.fwd(q, k, v, scale=1.0)
    torch.cuda.synchronize()
    exact_o, exact_lse = _closed_form(ex["scores"], vecs)
    _check_row(o[0, 0, 3], lse[0, 0, 3], ex["printed"]["O"], ex["tol"]["O"], vecs, dtype,
               exact_o, exact_lse)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("x", [10.0, 100.0])
def test_lag_rescale_on_cell_f(golden, dtype, d, x):
    """Cell F's row [x, 0] with its keys in two blocks, the 0 first: the
    reference max then jumps by x natural units. The kernel moves its
    reference when a block's max exceeds it by more than its lag, 8 log2
    units (5.55 natural units) for fp16 and 32 (22.2) for bf16: x = 10 runs
    the rescale branch (factor e^-10) in fp16, x = 100 in both."""
    ex = {e["id"]: e for e in golden["row_examples"]}[f"cell_F_x{int(x)}"]
    keys = [(0, 0.0, [20.0]), (BLOCK + 7, x, [10.0])]
    q, k, v = _build(keys, 2 * BLOCK, d, dtype)
    o, lse = fa.fwd(q, k, v, scale=1.0)
    torch.cuda.synchronize()
    exact_o, exact_lse = _closed_form([x, 0.0], [[10.0], [20.0]])
    say(f"Cell F x={x} ({dtype}, d={d})")
    _check_row(o[0, 0, 9], lse[0, 0, 9], ex["printed"]["O"], ex["tol"]["O"], [[10.0], [20.0]],
               dtype, exact_o, exact_lse)
    # ln(1 + e^-x) in lse: 4.54e-5 at x = 10, far above fp32 resolution at 10.
    assert abs(float(lse[0, 0, 9]) - exact_lse) <= 2e-6 * abs(exact_lse)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", DIMS)
def test_masked_cells(golden, dtype, d):
    """Cell D (query at position 1 of [2, 1, 4, 3]: keys 2 and 3 in its
    future) through the causal mask, and Cell D2 (every key hidden) through
    kv_len 0 and through the strict mask's first row: O = 0, lse = -inf."""
    ex = {e["id"]: e for e in golden["row_examples"]}["cell_D_causal"]
    vals = [10.0, 20.0, 30.0, 40.0]
    keys = [(j, s, [vals[j]]) for j, s in enumerate([2.0, 1.0, 4.0, 3.0])]
    q, k, v = _build(keys, 2 * BLOCK, d, dtype)
    o, lse = fa.fwd(q, k, v, causal=True, scale=1.0)
    torch.cuda.synchronize()
    exact_o, exact_lse = _closed_form([2.0, 1.0], [[10.0], [20.0]])
    say(f"Cell D ({dtype}, d={d})")
    _check_row(o[0, 0, 1], lse[0, 0, 1], ex["printed"]["O"], ex["tol"]["O"], [[10.0], [20.0]],
               dtype, exact_o, exact_lse)
    # Row 0 sees key 0 alone: O = V_0 exactly.
    assert float(o[0, 0, 0, 0]) == 10.0
    # Cell D2: nothing visible.
    o, lse = fa.fwd(q, k, v, causal=True, scale=1.0,
                    kv_lens=torch.zeros(1, dtype=torch.int32, device=DEV))
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()
    o, lse = fa.fwd(q, k, v, causal="strict", scale=1.0)
    assert torch.all(o[0, 0, 0] == 0).item() and bool(torch.isneginf(lse[0, 0, 0]))
    assert float(o[0, 0, 1, 0]) == 10.0  # strict row 1 sees key 0 alone
