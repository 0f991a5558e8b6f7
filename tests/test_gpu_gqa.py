"""GPU parity of the grouped-head and Nq != Nk entry points (fa_fwd_ex,
fa_fwd_f32_ex, fa_bwd_ex) against the fp64 oracle, through the C-ABI.

Query head h reads K/V head h // (H / Hkv); under the causal masks the Nq
queries are the last Nq of the Nk key positions (query i sees key j iff
j <= i + Nk - Nq, or < for the strict mask). The cases cover grouped and
single K/V heads, continuations (Nq < Nk), more queries than keys (whole
query tiles with no visible key), one-query decode over a long cache with the
split-KV plan, key padding, and ragged tails of query and key tiles.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import BF16_GRAD, BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F32_LSE, \
    F32_O, check_lse, check_o, oracle_bwd, oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, H, Hkv, Nq, Nk, d, causal, kv_lens)
CASES = [
    (2, 8, 2, 300, 300, 128, True, None),      # grouped, ragged tiles
    (1, 8, 1, 257, 257, 64, False, None),      # one K/V head for all
    (2, 4, 4, 200, 700, 128, True, None),      # continuation after 500 cached keys
    (2, 4, 2, 700, 200, 64, True, None),       # first 500 queries see no key
    (1, 4, 2, 1, 4096, 128, True, None),       # decode: one query per head
    (2, 32, 4, 1, 5000, 64, False, [4000, 1]),  # decode, 8 heads per K/V head, padded keys
    (1, 8, 2, 1, 3000, 128, "strict", None),   # strict decode (hides the last key)
    (1, 256, 1, 1, 700, 128, True, [700]),     # one K/V head for 256 query heads (two tiles)
    (2, 8, 2, 16, 2000, 128, False, [1500, 0]),  # short queries, padded keys, an empty batch
    (1, 4, 4, 130, 1000, 64, "strict", None),
    (1, 2, 1, 1000, 33, 128, "strict", [20]),  # Nq > Nk with padding
]


def _ids(c):
    B, H, Hkv, Nq, Nk, d, causal, kv = c
    tag = {False: "", True: "c", "strict": "s"}[causal]
    return f"B{B}H{H}g{Hkv}q{Nq}k{Nk}d{d}{tag}{'' if kv is None else 'kv'}"


def _inputs(B, H, Hkv, Nq, Nk, d, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    do = torch.randn(B, H, Nq, d, generator=g).to(dtype)
    return q, k, v, do


def _kv(kvl):
    return None if kvl is None else torch.tensor(kvl, dtype=torch.int32)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_forward_bf16_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, causal, kvl = case
    say(f"case gqa-fwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} kv={kvl}")
    q, k, v, _ = _inputs(B, H, Hkv, Nq, Nk, d, 2100 + Nq + Nk + d)
    kv = _kv(kvl)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = fa.default_scale(d)
    o_u, lse_u = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    o_s, lse_s = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd, split=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    for o, lse in ((o_u, lse_u), (o_s, lse_s)):
        check_o(to64(o), o_ref, BF16_O_MAX, BF16_O_MEAN)
        check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)
    empty = lse_ref == -np.inf
    assert np.all(to64(o_u)[empty] == 0.0)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_forward_f32_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, causal, kvl = case
    say(f"case gqa-f32 B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} kv={kvl}")
    q, k, v, _ = _inputs(B, H, Hkv, Nq, Nk, d, 2200 + Nq + Nk + d, torch.float32)
    kv = _kv(kvl)
    kvd = None if kv is None else kv.to(DEV)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, kv_lens=kvd)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    check_o(to64(o), o_ref, F32_O)
    check_lse(to64(lse), lse_ref, F32_LSE)


def test_decode_over_long_cache_is_split():
    B, H, Hkv, Nq, Nk, d = 2, 16, 2, 1, 32768, 128
    say(f"case gqa-decode B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d}")
    assert fa.split_workspace_bytes(B, H, Nq, d, True, Hkv, Nk) > 0
    q, k, v, _ = _inputs(B, H, Hkv, Nq, Nk, d, 2301)
    kv = torch.tensor([32768, 12345], dtype=torch.int32)
    qd, kd, vd, kvd = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    o_s, lse_s = fa.fwd(qd, kd, vd, causal=True, kv_lens=kvd, split=True)
    o_u, lse_u = fa.fwd(qd, kd, vd, causal=True, kv_lens=kvd)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, fa.default_scale(d), True, kv)
    for o, lse in ((o_s, lse_s), (o_u, lse_u)):
        check_o(to64(o), o_ref, BF16_O_MAX, BF16_O_MEAN)
        check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_equals_repeated_heads_bitwise(causal):
    """fa_fwd_ex on grouped K/V gives exactly fa_fwd's result on K/V with each
    head repeated H / Hkv times (same kernel, same per-head arithmetic)."""
    B, H, Hkv, N, d = 2, 8, 2, 384, 128
    say(f"case gqa-repeat causal={causal}")
    q, k, v, _ = _inputs(B, H, Hkv, N, N, d, 2400)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_g, lse_g = fa.fwd(qd, kd, vd, causal=causal)
    kr = kd.repeat_interleave(H // Hkv, dim=1).contiguous()
    vr = vd.repeat_interleave(H // Hkv, dim=1).contiguous()
    o_r, lse_r = fa.fwd(qd, kr, vr, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r) and torch.equal(lse_g, lse_r)


# (B, H, Hkv, Nq, Nk, d, causal, kv_lens)
BWD_CASES = [
    (2, 4, 2, 160, 160, 128, True, None),
    (1, 4, 1, 100, 100, 64, False, None),
    (2, 2, 2, 96, 300, 128, True, None),       # continuation: the prefix keys get gradients
    (1, 4, 2, 300, 96, 64, True, None),        # early queries see no key: dQ = 0 there
    (2, 4, 2, 64, 257, 64, "strict", [200, 257]),
    (1, 8, 2, 1, 700, 128, True, None),        # one query per head
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[_ids(c) for c in BWD_CASES])
def test_backward_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, causal, kvl = case
    say(f"case gqa-bwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} kv={kvl}")
    q, k, v, do = _inputs(B, H, Hkv, Nq, Nk, d, 2500 + Nq + Nk + d)
    kv = _kv(kvl)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, kv_lens=kvd)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    rq, rk, rv = oracle_bwd(q, k, v, do, scale, causal, kv)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to64(g)
        assert np.all(np.isfinite(gh)), name
        err = np.abs(gh - r)
        say(f"   {name} max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
            f"(|ref| max {np.abs(r).max():.3g})")
        # Above |ref| = 12.8 the bf16 output's own half-ulp exceeds 5e-2.
        assert np.all(err <= BF16_GRAD + 2.0 ** -8 * np.abs(r)), f"{name} max-abs {err.max():.3g}"


def test_backward_grouped_sums_repeated_heads():
    """dK, dV of a shared head are the sums of the per-head gradients that
    fa_bwd returns on repeated K/V (up to the bf16 rounding of each term)."""
    B, H, Hkv, N, d = 1, 8, 2, 256, 128
    say("case gqa-bwd-repeat")
    q, k, v, do = _inputs(B, H, Hkv, N, N, d, 2600)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    G = H // Hkv
    kr = kd.repeat_interleave(G, dim=1).contiguous()
    vr = vd.repeat_interleave(G, dim=1).contiguous()
    o, lse = fa.fwd(qd, kd, vd, causal=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=True)
    o_r, lse_r = fa.fwd(qd, kr, vr, causal=True)
    dq_r, dk_r, dv_r = fa.bwd(qd, kr, vr, o_r, lse_r, dod, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_r)
    for g, gr in ((dk, dk_r), (dv, dv_r)):
        summed = gr.float().view(B, Hkv, G, N, d).sum(dim=2)
        err = (g.float() - summed).abs().max().item()
        assert err <= 2e-2 + 2.0 ** -7 * summed.abs().max().item(), err
