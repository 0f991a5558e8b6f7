"""GPU parity at head dimension 256 against the fp64 oracle, through the C-ABI.

At d = 256 the forward runs one workgroup per compute unit (its Q^T
fragments and output accumulators need more than half the register file) and
the backward computes dV and dK in two passes of the key-tile kernel. The
cases cover bf16, fp16 and fp32, causal / strict / padded masks, grouped K/V
heads, Nq != Nk and split-KV.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import BF16_GRAD, BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F16_GRAD, \
    F16_O_MAX, F16_O_MEAN, F32_LSE, F32_O, check_lse, check_o, oracle_bwd, oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 256
TOL = {torch.bfloat16: (BF16_O_MAX, BF16_O_MEAN, BF16_LSE_ABS, BF16_LSE_REL),
       torch.float16: (F16_O_MAX, F16_O_MEAN, BF16_LSE_ABS, BF16_LSE_REL),
       torch.float32: (F32_O, None, F32_LSE, 0.0)}
NAME = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}

# (dtype, B, H, Hkv, Nq, Nk, causal, kv_lens)
FWD_CASES = [
    (torch.bfloat16, 1, 4, 4, 300, 300, True, None),
    (torch.bfloat16, 2, 2, 2, 257, 257, False, [100, 0]),
    (torch.bfloat16, 1, 8, 2, 200, 700, True, None),
    (torch.bfloat16, 1, 2, 2, 2048, 2048, True, None),   # few heads: split-KV plan
    (torch.bfloat16, 1, 4, 2, 1, 4096, True, None),      # decode
    (torch.float16, 1, 4, 4, 384, 384, "strict", None),
    (torch.float16, 1, 4, 1, 130, 1000, False, None),
    (torch.float32, 1, 2, 2, 200, 200, True, None),
    (torch.float32, 1, 4, 2, 64, 300, True, [250]),
]


def _ids(c):
    dt, B, H, Hkv, Nq, Nk, causal, kv = c
    tag = {False: "", True: "c", "strict": "s"}[causal]
    return f"{NAME[dt]}B{B}H{H}g{Hkv}q{Nq}k{Nk}{tag}{'' if kv is None else 'kv'}"


def _inputs(dtype, B, H, Hkv, Nq, Nk, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Nk, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Nk, D, generator=g).to(dtype)
    do = torch.randn(B, H, Nq, D, generator=g).to(dtype)
    return q, k, v, do


@pytest.mark.parametrize("case", FWD_CASES, ids=[_ids(c) for c in FWD_CASES])
def test_forward_d256_matches_oracle(case):
    dtype, B, H, Hkv, Nq, Nk, causal, kvl = case
    say(f"case d256-fwd {NAME[dtype]} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
        f"kv={kvl}")
    q, k, v, _ = _inputs(dtype, B, H, Hkv, Nq, Nk, 3100 + Nq + Nk)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = fa.default_scale(D)
    runs = [fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)]
    if dtype != torch.float32:
        runs.append(fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd, split=True))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    omax, omean, labs, lrel = TOL[dtype]
    for o, lse in runs:
        check_o(to64(o), o_ref, omax, omean)
        check_lse(to64(lse), lse_ref, labs, lrel)


def test_split_plan_at_d256():
    assert fa.split_workspace_bytes(1, 2, 2048, D, True) > 0
    assert fa.split_workspace_bytes(1, 4, 1, D, True, 2, 4096) > 0


# (dtype, B, H, Hkv, Nq, Nk, causal, kv_lens)
BWD_CASES = [
    (torch.bfloat16, 1, 2, 2, 160, 160, True, None),
    (torch.bfloat16, 1, 4, 2, 96, 300, True, None),
    (torch.bfloat16, 2, 2, 2, 200, 200, "strict", [200, 77]),
    (torch.float16, 1, 2, 2, 200, 200, False, [150]),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[_ids(c) for c in BWD_CASES])
def test_backward_d256_matches_oracle(case):
    dtype, B, H, Hkv, Nq, Nk, causal, kvl = case
    say(f"case d256-bwd {NAME[dtype]} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
        f"kv={kvl}")
    q, k, v, do = _inputs(dtype, B, H, Hkv, Nq, Nk, 3200 + Nq + Nk)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    scale = fa.default_scale(D)
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
