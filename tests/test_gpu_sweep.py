"""Seeded sweep over combinations of the forward's and backward's options,
each case checked element by element against the fp64 oracle.

The other GPU tests take one feature at a time (grouped heads, key padding,
the strict mask, fp16, each head dimension, split-KV). Here a fixed seed
draws cases from the cross product of all of them at small, ragged sizes
(query and key counts that are not multiples of the 128-row tiles or the
64-key blocks, single query rows, more queries than keys, batches whose
key length is 0), so that options are also exercised together: for example
fp16 with grouped K/V heads, the strict mask, key padding and a split key
range at d = 96. The case list is fixed by the seed; its ids name every
option.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import (BF16_GRAD, BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F16_GRAD,
                     F16_O_MAX, F16_O_MEAN, F32_LSE, F32_O, check_lse, check_o, oracle_bwd,
                     oracle_fwd, say, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
ROWS = [1, 2, 31, 33, 64, 100, 127, 129, 200, 257, 300]


def _draw(rs, backward):
    d = int(rs.choice([32, 64, 96, 128, 256]))
    dt = str(rs.choice(["bf16", "f16"] if backward else ["bf16", "bf16", "f16", "f32"]))
    causal = [False, True, "strict"][int(rs.randint(3))]
    Hkv = int(rs.choice([1, 2, 4]))
    G = int(rs.choice([1, 2, 4]))
    B = int(rs.randint(1, 4))
    Nq = int(rs.choice(ROWS))
    Nk = Nq if rs.rand() < 0.5 else int(rs.randint(1, 601))
    kv = None
    if rs.rand() < 0.3:
        kv = [int(x) for x in rs.randint(0, Nk + 1, size=B)]
    split = dt != "f32" and not backward and rs.rand() < 0.35
    return (B, Hkv * G, Hkv, Nq, Nk, d, dt, causal, kv, split)


def _cases(n, seed, backward):
    rs = np.random.RandomState(seed)
    return [_draw(rs, backward) for _ in range(n)]


FWD_CASES = _cases(40, 20261203, backward=False)
BWD_CASES = _cases(16, 20261204, backward=True)


def _id(c):
    B, H, Hkv, Nq, Nk, d, dt, causal, kv, split = c
    tag = {False: "n", True: "c", "strict": "s"}[causal]
    return (f"B{B}H{H}g{Hkv}q{Nq}k{Nk}d{d}{dt}{tag}"
            f"{'' if kv is None else 'kv' + '-'.join(map(str, kv))}{'split' if split else ''}")


def _inputs(c, seed, backward):
    B, H, Hkv, Nq, Nk, d, dt, causal, kv, split = c
    g = torch.Generator().manual_seed(seed)
    dtype = DTYPES[dt]
    q = torch.randn(B, H, Nq, d, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    do = torch.randn(B, H, Nq, d, generator=g).to(dtype) if backward else None
    kvt = None if kv is None else torch.tensor(kv, dtype=torch.int32)
    return q, k, v, do, kvt


@pytest.mark.parametrize("case", FWD_CASES, ids=[_id(c) for c in FWD_CASES])
def test_forward_sweep(case):
    B, H, Hkv, Nq, Nk, d, dt, causal, kv, split = case
    say(f"case sweep-fwd {_id(case)}")
    q, k, v, _, kvt = _inputs(case, 7000 + FWD_CASES.index(case), False)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                    kv_lens=None if kvt is None else kvt.to(DEV), split=split)
    torch.cuda.synchronize()
    assert o.shape == q.shape and o.dtype == q.dtype and lse.shape == (B, H, Nq)
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kvt)
    if dt == "f32":
        check_o(to64(o), o_ref, F32_O)
        check_lse(to64(lse), lse_ref, F32_LSE)
    else:
        o_max, o_mean = (BF16_O_MAX, BF16_O_MEAN) if dt == "bf16" else (F16_O_MAX, F16_O_MEAN)
        check_o(to64(o), o_ref, o_max, o_mean)
        check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)


@pytest.mark.parametrize("case", BWD_CASES, ids=[_id(c) for c in BWD_CASES])
def test_backward_sweep(case):
    B, H, Hkv, Nq, Nk, d, dt, causal, kv, _ = case
    say(f"case sweep-bwd {_id(case)}")
    q, k, v, do, kvt = _inputs(case, 8000 + BWD_CASES.index(case), True)
    scale = fa.default_scale(d)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    kvd = None if kvt is None else kvt.to(DEV)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, kv_lens=kvd)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_bwd(q, k, v, do, scale, causal, kvt)
    # The flat bound, widened by the 16-bit output's own half-ulp of |ref|
    # (2^-9 for bf16, 2^-11 for fp16, doubled for the fp32 accumulation).
    flat, rel = (BF16_GRAD, 2.0 ** -8) if dt == "bf16" else (F16_GRAD, 2.0 ** -10)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to64(got)
        assert np.all(np.isfinite(gh)), name
        err = np.abs(gh - ref)
        say(f"   {name} max-abs {err.max():.3e} (|ref| max {np.abs(ref).max():.3g})")
        assert np.all(err <= flat + rel * np.abs(ref)), f"{name} max-abs {err.max():.3g}"


def test_sweep_covers_every_option():
    """The seed draws every head dimension, type, mask, group size, padded
    and split case, and query and key counts on both sides of a tile."""
    cs = FWD_CASES + BWD_CASES
    assert {c[5] for c in cs} == {32, 64, 96, 128, 256}
    assert {c[6] for c in FWD_CASES} == {"bf16", "f16", "f32"}
    assert {c[6] for c in BWD_CASES} == {"bf16", "f16"}
    assert {str(c[7]) for c in cs} == {"False", "True", "strict"}
    assert {c[1] // c[2] for c in cs} == {1, 2, 4}
    assert any(c[8] is not None and 0 in c[8] for c in cs)
    assert any(c[9] for c in FWD_CASES)
    assert any(c[3] > c[4] for c in cs) and any(c[3] < c[4] for c in cs)
    assert any(c[3] == 1 for c in cs) and any(c[3] > 128 for c in cs)
