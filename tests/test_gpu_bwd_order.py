"""GPU parity of the backward's head-sequential work order.

On grids of at least 16 rounds of resident workgroups each gradient kernel
runs every XCD's heads one after another instead of tile-major
(fa_bwd_tile_order). Only the assignment of tiles to workgroups changes, so
the gradients of a head must be bitwise those of a call on that head alone
(whose grid is tile-major), and they are compared with the fp64 oracle's on
the same inputs. Inputs are drawn on the device with a seeded generator (the
batched tensors are hundreds of MB); the heads checked are copied back.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import BF16_GRAD, oracle_bwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BOTH = fa.FA_BWD_DQ_HEAD_SEQUENTIAL | fa.FA_BWD_DKDV_HEAD_SEQUENTIAL

# (B, H, Hkv, N, d, causal, K/V heads checked as (b, kv head))
CASES = [
    (8, 32, 32, 4096, 128, True, [(0, 0), (3, 17), (7, 31)]),
    (8, 32, 32, 4096, 128, False, [(5, 9)]),
    (8, 32, 16, 4096, 256, True, [(2, 5)]),   # two query heads per K/V head; one workgroup per CU
]


def _ids(c):
    B, H, Hkv, N, d, causal, _ = c
    return f"B{B}H{H}g{Hkv}N{N}d{d}{'c' if causal else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_head_sequential_backward(case):
    B, H, Hkv, N, d, causal, heads = case
    order = fa.bwd_tile_order(B, H, N, d, Hkv=Hkv)
    say(f"case bwd order B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}: order {order}")
    assert order == BOTH
    g = torch.Generator(device=DEV).manual_seed(2100 + N + d + H)
    q = torch.randn(B, H, N, d, generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g, device=DEV).to(torch.bfloat16)
    do = torch.randn(B, H, N, d, generator=g, device=DEV).to(torch.bfloat16)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    G = H // Hkv
    for b, hk in heads:
        hs = slice(hk * G, (hk + 1) * G)
        qs, ks, vs, os_, ds = (t[b:b + 1, s].contiguous() for t, s in
                               ((q, hs), (k, slice(hk, hk + 1)), (v, slice(hk, hk + 1)),
                                (o, hs), (do, hs)))
        ls = lse[b:b + 1, hs].contiguous()
        assert fa.bwd_tile_order(1, G, N, d, Hkv=1) == 0  # a lone group: tile-major
        rq, rk, rv = fa.bwd(qs, ks, vs, os_, ls, ds, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(dq[b:b + 1, hs], rq)
        assert torch.equal(dk[b:b + 1, hk:hk + 1], rk)
        assert torch.equal(dv[b:b + 1, hk:hk + 1], rv)
        oq, ok, ov = oracle_bwd(qs.cpu(), ks.cpu(), vs.cpu(), ds.cpu(), scale, causal)
        for name, got, ref in (("dq", rq, oq), ("dk", rk, ok), ("dv", rv, ov)):
            err = np.abs(to64(got) - ref)
            say(f"   batch {b} K/V head {hk} {name} max-abs {err.max():.3e} "
                f"(|ref| max {np.abs(ref).max():.3g})")
            assert np.all(err <= BF16_GRAD + 2.0 ** -8 * np.abs(ref)), name


def test_small_grids_stay_tile_major():
    """The metric backward (2 rounds of workgroups) keeps the tile-major order."""
    assert fa.bwd_tile_order(2, 16, 4096, 128) == 0
