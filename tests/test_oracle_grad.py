"""Pins of the oracle's backward: central finite differences and float64 autograd."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, scale, causal, kv_lens):
    o, _ = orc.attn_fwd_naive(q, k, v, scale, causal, kv_lens)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal,kv_lens", [(False, None), (True, None), (True, [0, 11]),
                                            ("strict", None), ("strict", [3, 11])])
def test_backward_matches_finite_differences(causal, kv_lens):
    """N=16, d=4, central differences with h = 1e-6 on L = sum(dO * O)."""
    B, H, N, d = 2, 1, 16, 4
    q, k, v, do = (_rand((B, H, N, d), s) for s in (31, 32, 33, 34))
    scale = 0.5
    dq, dk, dv = orc.attn_bwd(q, k, v, do, scale, causal, kv_lens)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal, kv_lens)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal, kv_lens)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g) / np.maximum(1.0, np.abs(g))
        assert np.max(err) < 1e-7, (name, np.max(err))
    if kv_lens is not None and kv_lens[0] == 0:
        # A batch with no visible key has zero gradients everywhere.
        assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    B, H, N, d = 2, 2, 48, 8
    q, k, v, do = (_rand((B, H, N, d), s) for s in (41, 42, 43, 44))
    scale = 1.0 / math.sqrt(d)
    kv_lens = [48, 29]
    dq, dk, dv = orc.attn_bwd(q, k, v, do, scale, causal, kv_lens)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    idx = torch.arange(N)
    mask = torch.zeros(B, 1, N, N, dtype=torch.bool)
    for b in range(B):
        m = idx[None, :] < kv_lens[b]
        if causal:
            m = m & (idx[None, :] <= idx[:, None])
        mask[b, 0] = m
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    (o * torch.from_numpy(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [True, "strict"])
def test_backward_grouped_heads_unequal_lengths_finite_differences(causal):
    """Grouped K/V heads (H = 4, H_kv = 2) and N_q = 5 < N_k = 9, bottom-right."""
    B, H, Hkv, N, Nk, d = 1, 4, 2, 5, 9, 3
    q, do = _rand((B, H, N, d), 91), _rand((B, H, N, d), 94)
    k, v = _rand((B, Hkv, Nk, d), 92), _rand((B, Hkv, Nk, d), 93)
    scale = 0.5
    dq, dk, dv = orc.attn_bwd(q, k, v, do, scale, causal, [8])
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal, [8])
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal, [8])
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g) / np.maximum(1.0, np.abs(g))
        assert np.max(err) < 1e-7, (name, np.max(err))
    assert np.all(dk[:, :, 8:] == 0) and np.all(dv[:, :, 8:] == 0)  # padded keys
