"""GPU parity of the forward's head-sequential tile order.

On grids of at least 16 rounds of resident workgroups, with B*H a multiple
of 8 and the causal tiles not paired, each XCD runs its heads one after
another instead of item-major (fa_fwd_tile_order,
FA_FWD_ORDER_HEAD_SEQUENTIAL). Only the assignment of tiles to workgroups
changes, so the output and lse of a head must be bitwise those of a call on
that head alone (a one-head grid runs item-major); both are also compared
with the fp64 oracle on the same inputs. The batched inputs (hundreds of MB
to a few GB) are drawn on the device with a seeded generator and the checked
heads are copied back. The cases cover causal, strict causal with key
padding, no mask, fp16 with grouped K/V heads at d = 64, Nq < Nk, and the
split-capable entry point (a workspace given, but a grid too large to split).
"""
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import (BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F16_O_MAX,
                     F16_O_MEAN, check_lse, check_o, oracle_fwd, say, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, H, Hkv, Nq, Nk, d, dtype, causal, padded, split, heads checked as (b, h))
CASES = [
    (16, 32, 32, 2048, 2048, 128, "bf16", True, False, False, [(0, 0), (7, 19), (15, 31)]),
    (8, 32, 32, 4096, 4096, 128, "bf16", False, False, False, [(3, 8)]),
    (16, 32, 32, 2048, 2048, 128, "bf16", "strict", True, False, [(2, 5), (9, 30)]),
    (128, 32, 8, 1024, 1024, 64, "f16", True, False, False, [(127, 13)]),  # more slots at d = 64
    (128, 16, 16, 512, 4096, 128, "bf16", True, False, False, [(100, 3)]),
    (16, 32, 32, 2048, 2048, 128, "bf16", True, False, True, [(4, 4)]),
]


def _ids(c):
    B, H, Hkv, Nq, Nk, d, dt, causal, padded, split, _ = c
    tag = {True: "c", "strict": "s", False: "n"}[causal]
    return (f"B{B}H{H}g{Hkv}q{Nq}k{Nk}d{d}{dt}{tag}"
            f"{'kv' if padded else ''}{'split' if split else ''}")


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_head_sequential_forward(case):
    B, H, Hkv, Nq, Nk, d, dt, causal, padded, split, heads = case
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    order = fa.tile_order(Nq, B * H, d, causal, Nk=Nk, dtype=dtype)
    say(f"case fwd order {_ids(case)}: order {order}")
    assert order == fa.FA_FWD_ORDER_HEAD_SEQUENTIAL
    g = torch.Generator(device=DEV).manual_seed(3100 + Nq + Nk + d + B)
    q = torch.randn(B, H, Nq, d, generator=g, device=DEV).to(dtype)
    k = torch.randn(B, Hkv, Nk, d, generator=g, device=DEV).to(dtype)
    v = torch.randn(B, Hkv, Nk, d, generator=g, device=DEV).to(dtype)
    kv = None
    if padded:
        kv = torch.randint(1, Nk + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
        kv[0] = Nk
    scale = fa.default_scale(d)
    ws = None
    if split:
        ws = torch.zeros(fa.split_workspace_bytes(B, H, Nq, d, causal, Nk=Nk),
                         dtype=torch.uint8, device=DEV)
        assert fa.schedule(Nq, B * H, causal, 256, 2, Nk=Nk, d=d)[0] == []  # no split plan
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale, kv_lens=kv, split=split, workspace=ws)
    torch.cuda.synchronize()
    G = H // Hkv
    o_max, o_mean = (BF16_O_MAX, BF16_O_MEAN) if dt == "bf16" else (F16_O_MAX, F16_O_MEAN)
    for b, h in heads:
        hk = h // G
        qs = q[b:b + 1, h:h + 1].contiguous()
        ks = k[b:b + 1, hk:hk + 1].contiguous()
        vs = v[b:b + 1, hk:hk + 1].contiguous()
        kvs = None if kv is None else kv[b:b + 1].contiguous()
        assert fa.tile_order(Nq, 1, d, causal, Nk=Nk, dtype=dtype) == fa.FA_FWD_ORDER_HEAVY_FIRST
        ro, rl = fa.fwd(qs, ks, vs, causal=causal, scale=scale, kv_lens=kvs)
        torch.cuda.synchronize()
        assert torch.equal(o[b:b + 1, h:h + 1], ro), (b, h)
        assert torch.equal(lse[b:b + 1, h:h + 1], rl), (b, h)
        o_ref, lse_ref = oracle_fwd(qs.cpu(), ks.cpu(), vs.cpu(), scale, causal,
                                    None if kvs is None else kvs.cpu())
        say(f"   batch {b} head {h}"
            f"{'' if kvs is None else f' ({int(kvs[0])} keys)'}: all {Nq} rows")
        check_o(to64(ro)[0, 0], o_ref[0, 0], o_max, o_mean)
        check_lse(to64(rl)[0, 0], lse_ref[0, 0], BF16_LSE_ABS, BF16_LSE_REL)


def test_metric_shape_stays_item_major():
    """B = 2, H = 16, N = 4096 causal (1024 workgroups, 2 rounds) keeps the
    item-major order, as do grids just under 16 rounds."""
    assert fa.tile_order(4096, 32, 128, True) == fa.FA_FWD_ORDER_HEAVY_FIRST
    assert fa.tile_order(2048, 8 * 63, 128, True) == fa.FA_FWD_ORDER_HEAVY_FIRST
