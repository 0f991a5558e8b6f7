"""GPU parity of the fp16 path (fa_fwd_ex / fa_bwd_ex with FA_DTYPE_F16)
against the fp64 oracle, through the C-ABI.

The fp16 kernels are the bf16 kernels with the fp16 matrix instruction and
fp16 rounding of P, O, dS and the gradients. The oracle receives the same
fp16 inputs, upcast exactly.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import BF16_LSE_ABS, BF16_LSE_REL, F16_GRAD, F16_O_MAX, F16_O_MEAN, check_lse, \
    check_o, oracle_bwd, oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, H, Hkv, Nq, Nk, d, causal, kv_lens, q_mult)
FWD_CASES = [
    (2, 4, 4, 300, 300, 128, True, None, 1.0),
    (1, 4, 4, 257, 257, 64, False, None, 1.0),
    (2, 8, 2, 200, 700, 128, True, None, 1.0),      # grouped heads, continuation
    (2, 4, 4, 320, 320, 128, "strict", [0, 200], 1.0),
    (1, 4, 2, 1, 4096, 128, True, None, 1.0),        # decode (split-KV plan)
    (1, 4, 4, 1024, 1024, 64, True, None, 8.0),      # scores up to about +-60
    (1, 4, 4, 2048, 2048, 128, True, None, 1.0),
]


def _ids(c):
    B, H, Hkv, Nq, Nk, d, causal, kv, qm = c
    tag = {False: "", True: "c", "strict": "s"}[causal]
    return f"B{B}H{H}g{Hkv}q{Nq}k{Nk}d{d}{tag}{'' if kv is None else 'kv'}{'' if qm == 1 else 'x8'}"


def _inputs(B, H, Hkv, Nq, Nk, d, seed, q_mult=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, H, Nq, d, generator=g) * q_mult).to(torch.float16)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.float16)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.float16)
    do = torch.randn(B, H, Nq, d, generator=g).to(torch.float16)
    return q, k, v, do


@pytest.mark.parametrize("case", FWD_CASES, ids=[_ids(c) for c in FWD_CASES])
def test_forward_f16_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, causal, kvl, qm = case
    say(f"case f16-fwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} kv={kvl} "
        f"q_mult={qm}")
    q, k, v, _ = _inputs(B, H, Hkv, Nq, Nk, d, 2700 + Nq + Nk + d, qm)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = fa.default_scale(d)
    o_u, lse_u = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    o_s, lse_s = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd, split=True)
    torch.cuda.synchronize()
    assert o_u.dtype == torch.float16
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    for o, lse in ((o_u, lse_u), (o_s, lse_s)):
        check_o(to64(o), o_ref, F16_O_MAX, F16_O_MEAN)
        check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)


def test_decode_f16_is_split():
    assert fa.split_workspace_bytes(1, 4, 1, 128, True, 2, 4096, torch.float16) > 0


# (B, H, Hkv, Nq, Nk, d, causal, kv_lens)
BWD_CASES = [
    (2, 4, 4, 160, 160, 128, True, None),
    (1, 2, 2, 257, 257, 64, False, [100]),
    (1, 4, 2, 96, 300, 128, True, None),
    (2, 2, 2, 200, 200, 64, "strict", None),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[_ids(c + (1.0,)) for c in BWD_CASES])
def test_backward_f16_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, causal, kvl = case
    say(f"case f16-bwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} kv={kvl}")
    q, k, v, do = _inputs(B, H, Hkv, Nq, Nk, d, 2800 + Nq + Nk + d)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, kv_lens=kvd)
    torch.cuda.synchronize()
    assert dq.dtype == dk.dtype == dv.dtype == torch.float16
    rq, rk, rv = oracle_bwd(q, k, v, do, scale, causal, kv)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to64(g)
        assert np.all(np.isfinite(gh)), name
        err = np.abs(gh - r)
        say(f"   {name} max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
            f"(|ref| max {np.abs(r).max():.3g})")
        # Above |ref| = 16 the fp16 output's own half-ulp reaches 2^-7 |ref| / 2.
        assert np.all(err <= F16_GRAD + 2.0 ** -10 * np.abs(r)), f"{name} max-abs {err.max():.3g}"


def test_f16_and_bf16_agree_on_shared_inputs():
    """Inputs exactly representable in both types (multiples of 1/16 in
    [-2, 2]): both paths see the same Q, K, V and differ only by the rounding
    of P and O, so they agree within the bf16 bound."""
    B, H, N, d = 1, 4, 384, 128
    g = torch.Generator().manual_seed(2900)
    q, k, v = (torch.randint(-32, 33, (B, H, N, d), generator=g).float() / 16 for _ in range(3))
    o16, l16 = fa.fwd(q.half().to(DEV), k.half().to(DEV), v.half().to(DEV), causal=True)
    ob, lb = fa.fwd(q.bfloat16().to(DEV), k.bfloat16().to(DEV), v.bfloat16().to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(o16.float() - ob.float())).item() <= 2e-2
    assert torch.max(torch.abs(l16 - lb)).item() <= 2e-3
