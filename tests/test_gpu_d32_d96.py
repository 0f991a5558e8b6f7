"""GPU parity at head dimensions 32 and 96 against the fp64 oracle, through
the C-ABI.

Rows of 64 and 192 bytes do not split into whole rows per 1 KB DMA, so these
sizes load K/V (and Q/dO in the backward) with DMAs dealt round-robin over
the waves, and permute the 16-byte chunks of a row per row (an XOR at d = 32,
a rotation of the 12 chunks at d = 96). The cases cover bf16, fp16 and fp32,
ragged tiles, masks, padding, grouped K/V heads, Nq != Nk and split-KV.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import BF16_GRAD, BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F16_GRAD, \
    F16_O_MAX, F16_O_MEAN, F32_LSE, F32_O, check_lse, check_o, oracle_bwd, oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.bfloat16: (BF16_O_MAX, BF16_O_MEAN, BF16_LSE_ABS, BF16_LSE_REL),
       torch.float16: (F16_O_MAX, F16_O_MEAN, BF16_LSE_ABS, BF16_LSE_REL),
       torch.float32: (F32_O, None, F32_LSE, 0.0)}
NAME = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}

# (dtype, d, B, H, Hkv, Nq, Nk, causal, kv_lens)
FWD_CASES = [
    (torch.bfloat16, 32, 2, 4, 4, 300, 300, True, None),
    (torch.bfloat16, 32, 1, 4, 4, 257, 257, False, [100]),
    (torch.bfloat16, 32, 1, 2, 2, 4096, 4096, True, None),   # split-KV plan
    (torch.float16, 32, 1, 8, 2, 200, 700, True, None),
    (torch.float32, 32, 1, 2, 2, 200, 200, "strict", None),
    (torch.bfloat16, 96, 2, 4, 4, 300, 300, True, None),
    (torch.bfloat16, 96, 2, 2, 2, 257, 257, False, [100, 0]),
    (torch.bfloat16, 96, 1, 2, 2, 4096, 4096, True, None),   # split-KV plan
    (torch.bfloat16, 96, 1, 4, 2, 1, 4096, True, None),      # decode
    (torch.float16, 96, 1, 4, 4, 384, 384, "strict", None),
    (torch.float16, 96, 1, 4, 1, 130, 1000, False, None),
    (torch.float32, 96, 1, 4, 2, 64, 300, True, [250]),
]


def _ids(c):
    dt, d, B, H, Hkv, Nq, Nk, causal, kv = c
    tag = {False: "", True: "c", "strict": "s"}[causal]
    return f"{NAME[dt]}d{d}B{B}H{H}g{Hkv}q{Nq}k{Nk}{tag}{'' if kv is None else 'kv'}"


def _inputs(dtype, d, B, H, Hkv, Nq, Nk, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    do = torch.randn(B, H, Nq, d, generator=g).to(dtype)
    return q, k, v, do


@pytest.mark.parametrize("case", FWD_CASES, ids=[_ids(c) for c in FWD_CASES])
def test_forward_matches_oracle(case):
    dtype, d, B, H, Hkv, Nq, Nk, causal, kvl = case
    say(f"case d{d}-fwd {NAME[dtype]} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
        f"kv={kvl}")
    q, k, v, _ = _inputs(dtype, d, B, H, Hkv, Nq, Nk, 3300 + d + Nq + Nk)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = fa.default_scale(d)
    runs = [fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)]
    if dtype != torch.float32:
        runs.append(fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd, split=True))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    omax, omean, labs, lrel = TOL[dtype]
    for o, lse in runs:
        check_o(to64(o), o_ref, omax, omean)
        check_lse(to64(lse), lse_ref, labs, lrel)


@pytest.mark.parametrize("d", [32, 96])
def test_split_plan(d):
    assert fa.split_workspace_bytes(1, 2, 4096, d, True) > 0


# (dtype, d, B, H, Hkv, Nq, Nk, causal, kv_lens)
BWD_CASES = [
    (torch.bfloat16, 32, 2, 2, 2, 160, 160, True, None),
    (torch.bfloat16, 32, 1, 4, 2, 96, 300, True, None),
    (torch.float16, 32, 1, 2, 2, 257, 257, False, [150]),
    (torch.bfloat16, 96, 2, 2, 2, 160, 160, True, None),
    (torch.bfloat16, 96, 1, 4, 2, 96, 300, True, None),
    (torch.bfloat16, 96, 2, 2, 2, 200, 200, "strict", [200, 77]),
    (torch.float16, 96, 1, 2, 2, 257, 257, False, [150]),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[_ids(c) for c in BWD_CASES])
def test_backward_matches_oracle(case):
    dtype, d, B, H, Hkv, Nq, Nk, causal, kvl = case
    say(f"case d{d}-bwd {NAME[dtype]} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
        f"kv={kvl}")
    q, k, v, do = _inputs(dtype, d, B, H, Hkv, Nq, Nk, 3400 + d + Nq + Nk)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, kv_lens=kvd)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_bwd(q, k, v, do, scale, causal, kv)
    tol, rel = (BF16_GRAD, 2.0 ** -8) if dtype == torch.bfloat16 else (F16_GRAD, 2.0 ** -10)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to64(g)
        assert np.all(np.isfinite(gh)), name
        err = np.abs(gh - r)
        say(f"   {name} max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
            f"(|ref| max {np.abs(r).max():.3g})")
        assert np.all(err <= tol + rel * np.abs(r)), f"{name} max-abs {err.max():.3g}"
