"""GPU parity of fa_fwd / fa_fwd_f32 against the fp64 oracle (through the C-ABI)."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa
from exact_io_aware_17_amd import workloads as W
from oracle import attention as orc

from _parity import (BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F32_LSE, F32_O,
                     INF, check_lse, check_o, oracle_fwd, say, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(w: W.Workload, kv_lens=None):
    x = W.make_inputs(w)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    kv = x.get("kv_lens") if kv_lens is None else kv_lens
    kvd = None if kv is None else kv.to(DEV)
    say(f"case {w.name} B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} "
        f"kv_lens={None if kv is None else kv.tolist()}")
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale, kv_lens=kvd)
    torch.cuda.synchronize()
    return x, q, k, v, kv, o, lse


def _full_check(w, kv_lens=None):
    x, q, k, v, kv, o, lse = _run(w, kv_lens)
    o_ref, lse_ref = oracle_fwd(x["q"], x["k"], x["v"], w.scale, w.causal, kv)
    if w.dtype == "f32":
        check_o(to64(o), o_ref, F32_O)
        check_lse(to64(lse), lse_ref, F32_LSE)
    else:
        check_o(to64(o), o_ref, BF16_O_MAX, BF16_O_MEAN)
        check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)
    return x, o, lse


# ---- the five workloads at their own sizes (workload 4 sampled) ----

def test_workload1_fp32_full():
    _full_check(W.BY_ID[1])


def test_workload2_bf16_full():
    _full_check(W.BY_ID[2])


def test_workload3_causal_large_logits_full():
    _full_check(W.BY_ID[3])


def test_workload5_forward_full():
    _full_check(W.BY_ID[5])


def test_workload4_padded_whole_heads():
    """The padded N = 16384 workload: every row of two seeded heads per batch
    against the oracle (max-abs and mean-abs), the closed-form rows of every
    head of the kv_len 0 and 1 batches, and finiteness of every output."""
    w = W.BY_ID[4]
    x, q, k, v, kv, o, lse = _run(w)
    kvl = kv.tolist()
    assert kvl[0] == 0 and kvl[1] == 1
    # Every output element is finite; lse is -inf exactly on the empty batch.
    assert torch.all(torch.isfinite(o)).item()
    assert torch.all(torch.isneginf(lse[0])).item()
    assert torch.all(torch.isfinite(lse[1:])).item()
    # Closed-form rows on every head: kv_len 0 -> O = 0, lse = -inf ("Worked
    # examples", Cell D2); kv_len 1 -> O = V_0 exactly, lse = that key's score.
    assert torch.all(o[0] == 0).item()
    assert torch.equal(o[1], v[1, :, :1, :].expand_as(o[1]))
    s0 = (q[1].float() @ k[1, :, 0, :].float().unsqueeze(-1)).squeeze(-1) * w.scale
    assert torch.max(torch.abs(lse[1] - s0)).item() < 1e-2
    # Whole heads against the oracle: head 0 and a seeded second head of every
    # batch, all N rows, in row chunks (the oracle materialises each chunk's
    # scores against all keys).
    rng = np.random.default_rng(4)
    N = w.N
    chunk = 4096
    for b in range(w.B):
        heads = [(b, 0), (b, int(rng.integers(1, w.H)))]
        for (bb, hh) in heads:
            say(f"   batch {bb} (kv_len {kvl[bb]}) head {hh}: all {N} rows")
            o_g = to64(o[bb, hh])
            lse_g = to64(lse[bb, hh])
            o_ref = np.empty_like(o_g)
            lse_ref = np.empty_like(lse_g)
            qh, kh, vh = (to64(x[n][bb:bb + 1, hh:hh + 1]) for n in ("q", "k", "v"))
            for r0 in range(0, N, chunk):
                rows = list(range(r0, min(N, r0 + chunk)))
                orf, lrf = orc.attn_fwd_naive(qh, kh, vh, w.scale, True, [kvl[bb]], rows=rows)
                o_ref[r0:r0 + len(rows)] = orf[0, 0]
                lse_ref[r0:r0 + len(rows)] = lrf[0, 0]
            check_o(o_g, o_ref, BF16_O_MAX, BF16_O_MEAN)
            check_lse(lse_g, lse_ref, BF16_LSE_ABS, BF16_LSE_REL)


# ---- edge cases at oracle-friendly sizes ----

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 77, 200, 333])
def test_ragged_shapes(dtype, d, causal, N):
    w = W.Workload(90, f"ragged N={N}", 2, 3, N, d, dtype, causal)
    _full_check(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_key_padding_with_empty_and_single_rows(dtype, causal):
    w = W.Workload(91, "padding", 5, 2, 300, 64, dtype, causal)
    kv = torch.tensor([0, 1, 150, 300, 64], dtype=torch.int32)
    x, o, lse = _full_check(w, kv_lens=kv)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    v = x["v"].to(DEV)
    assert torch.equal(o[1], v[1, :, :1, :].expand_as(o[1]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 77, 333])
def test_strict_causal(dtype, d, N):
    w = W.Workload(97, f"strict N={N}", 2, 3, N, d, dtype, "strict")
    x, o, lse = _full_check(w)
    # "Worked examples", Cell D2 through the strict mask: row 0 sees no key.
    assert torch.all(o[:, :, 0] == 0) and torch.all(torch.isneginf(lse[:, :, 0]))
    if N > 1:  # row 1 sees key 0 only
        assert torch.equal(o[:, :, 1], x["v"].to(DEV)[:, :, 0])


@pytest.mark.parametrize("causal", [True, "strict"])
def test_64_key_causal_instance_with_ragged_tail(causal):
    # Causal rows of at least 4096 keys on a small grid take the 64-key d = 128
    # instance (rolling transpose-read schedule); N = 4133 leaves a ragged last
    # block and kv_len 4100 a masked one.
    w = W.Workload(99, "64-key causal ragged", 2, 2, 4133, 128, "bf16", causal)
    assert fa.block_keys(w.B, w.H, w.N, w.d, causal) == 64
    _full_check(w, kv_lens=torch.tensor([4133, 4100], dtype=torch.int32))


def test_strict_causal_with_padding():
    w = W.Workload(98, "strict padded", 3, 2, 300, 128, "bf16", "strict")
    _full_check(w, kv_lens=torch.tensor([0, 1, 170], dtype=torch.int32))


def test_kv_lens_out_of_range_are_clamped():
    w = W.Workload(92, "clamp", 3, 1, 130, 64, "bf16", False)
    x = W.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = fa.fwd(q, k, v, kv_lens=torch.tensor([-5, 10**6, 130], dtype=torch.int32, device=DEV))
    o2, l2 = fa.fwd(q, k, v, kv_lens=torch.tensor([0, 130, 130], dtype=torch.int32, device=DEV))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hidden_keys_never_leak(dtype):
    """Cell D: overwriting hidden K/V rows with large finite values changes no bit."""
    w = W.Workload(93, "leak", 2, 2, 256, 128, dtype, True)
    x = W.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kv = torch.tensor([200, 97], dtype=torch.int32, device=DEV)
    o1, l1 = fa.fwd(q, k, v, causal=True, kv_lens=kv)
    k2, v2 = k.clone(), v.clone()
    k2[0, :, 200:] = 3000.0
    v2[0, :, 200:] = -3000.0
    k2[1, :, 97:] = -3000.0
    v2[1, :, 97:] = 3000.0
    o2, l2 = fa.fwd(q, k2, v2, causal=True, kv_lens=kv)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_first_row_is_v0_and_deterministic():
    w = W.BY_ID[5]
    x = W.make_inputs(W.with_shape(w, N=1024))
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    for _ in range(3):
        o2, lse2 = fa.fwd(q, k, v, causal=True)
        assert torch.equal(o, o2) and torch.equal(lse, lse2)


def _embed(scores, values, d, dtype):
    n = len(scores)
    q = torch.zeros(1, 1, n, d, dtype=torch.float64)
    q[0, 0, :, 0] = 1.0
    k = torch.zeros_like(q)
    k[0, 0, :, 0] = torch.tensor(scores, dtype=torch.float64)
    v = torch.zeros_like(q)
    vals = torch.tensor(values, dtype=torch.float64)
    if vals.dim() == 1:
        vals = vals[:, None]
    v[0, 0, :, : vals.shape[1]] = vals
    return q.to(dtype), k.to(dtype), v.to(dtype)


def test_page_examples_through_fp32_kernel(golden):
    """The pages' worked rows fed through fa_fwd_f32 (scale 1, one-hot embedding, d = 64)."""
    for ex in golden["row_examples"]:
        if any(isinstance(s, str) for s in ex["scores"]):
            continue
        say(f"page example {ex['id']}")
        q, k, v = (t.to(DEV) for t in _embed(ex["scores"], ex["values"], 64, torch.float32))
        n = len(ex["scores"])
        o, lse = fa.fwd(q, k, v, scale=1.0)
        # The last query row sees all keys in a non-causal call; every row has the same scores.
        got = o[0, 0, n - 1, 0].item()
        assert abs(got - ex["printed"]["O"]) <= ex["tol"]["O"] + 1e-5 * abs(got)
    # Cell D through the causal mask, Cell D2 through an empty key range.
    q, k, v = (t.to(DEV) for t in _embed([2.0, 1.0, 4.0, 3.0], [10.0, 20.0, 30.0, 40.0], 64,
                                          torch.float32))
    o, _ = fa.fwd(q, k, v, causal=True, scale=1.0)
    want = (10 + 20 * math.exp(-1)) / (1 + math.exp(-1))
    assert abs(o[0, 0, 1, 0].item() - want) < 1e-5
    o, lse = fa.fwd(q, k, v, causal=True, scale=1.0,
                    kv_lens=torch.zeros(1, dtype=torch.int32, device=DEV))
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # Overflow example: scores 800 and 801 stay finite through the max shift.
    q, k, v = (t.to(DEV) for t in _embed([800.0, 801.0], [10.0, 20.0], 64, torch.float32))
    o, lse = fa.fwd(q, k, v, scale=1.0)
    assert abs(o[0, 0, 1, 0].item() - 17.31058578630005) < 2e-5


def test_fp32_matches_bf16_path_on_bf16_exact_inputs():
    """Both paths compute the same attention; on bf16-exact inputs they agree to bf16 rounding."""
    w = W.Workload(94, "cross", 2, 2, 512, 128, "bf16", True)
    x = W.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o_b, l_b = fa.fwd(q, k, v, causal=True)
    o_f, l_f = fa.fwd(q.float(), k.float(), v.float(), causal=True)
    assert torch.max(torch.abs(o_b.float() - o_f)).item() < 2e-2
    assert torch.max(torch.abs(l_b - l_f)).item() < 1e-3
