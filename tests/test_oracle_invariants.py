"""Pins of the Q/K/V-level oracle against brute force, a library routine,
closed-form rows and the invariances the pages state."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc

INF = float("inf")


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * scale


def _brute(q, k, v, scale, causal, kv_lens):
    """Pure-Python loops with math.exp: the definition on tiny inputs.

    K/V may have fewer heads (query head h reads K/V head h // (H / H_kv))
    and N_k keys; query i then sits at key position i + N_k - N.
    """
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        kvl = Nk if kv_lens is None else min(int(kv_lens[b]), Nk)
        for h in range(H):
            hk = h // (H // Hkv)
            for i in range(N):
                pos = i + Nk - N
                if causal == "strict":
                    keys = [j for j in range(Nk) if j < kvl and j < pos]
                else:
                    keys = [j for j in range(Nk) if j < kvl and (not causal or j <= pos)]
                if not keys:
                    o[b, h, i] = 0.0
                    lse[b, h, i] = -INF
                    continue
                sc = {}
                for j in keys:
                    acc = 0.0
                    for t in range(d):
                        acc += float(q[b, h, i, t]) * float(k[b, hk, j, t])
                    sc[j] = scale * acc
                m = max(sc.values())
                w = {j: math.exp(sc[j] - m) for j in keys}
                tot = sum(w.values())
                for c in range(v.shape[3]):
                    o[b, h, i, c] = sum(w[j] * float(v[b, hk, j, c]) for j in keys) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


@pytest.mark.parametrize("causal", [False, True, "strict"])
@pytest.mark.parametrize("kv_lens", [None, [0, 1, 5, 8]])
def test_naive_matches_brute_force(causal, kv_lens):
    B, H, N, d = 4, 2, 8, 4
    q, k, v = _rand((B, H, N, d), 1), _rand((B, H, N, d), 2), _rand((B, H, N, d), 3)
    o, lse = orc.attn_fwd_naive(q, k, v, 0.5, causal, kv_lens)
    ob, lseb = _brute(q, k, v, 0.5, causal, kv_lens)
    assert np.max(np.abs(o - ob)) < 1e-13
    fin = np.isfinite(lseb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - lseb[fin])) < 1e-13
    assert np.all(lse[~fin] == -INF)


@pytest.mark.parametrize("causal", [False, True])
def test_naive_matches_torch_sdpa_fp64(causal):
    """Library routine: PyTorch's math-path attention and logsumexp in float64 on the CPU."""
    B, H, N, d = 2, 3, 67, 16
    q, k, v = _rand((B, H, N, d), 4), _rand((B, H, N, d), 5), _rand((B, H, N, d), 6)
    scale = 1.0 / math.sqrt(d)
    kv_lens = [67, 40]
    o, lse = orc.attn_fwd_naive(q, k, v, scale, causal, kv_lens)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    idx = torch.arange(N)
    mask = torch.zeros(B, 1, N, N, dtype=torch.bool)
    for b in range(B):
        m = idx[None, :] < kv_lens[b]
        if causal:
            m = m & (idx[None, :] <= idx[:, None])
        mask[b, 0] = m
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    s = (tq @ tk.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, -INF)
    ref_lse = torch.logsumexp(s, dim=-1)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
    assert np.max(np.abs(lse - ref_lse.numpy())) < 1e-12


@pytest.mark.parametrize("block", [1, 7, 32, 50])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_matches_naive_at_any_block_size(block, causal):
    B, H, N, d = 3, 2, 50, 8
    q, k, v = _rand((B, H, N, d), 7, 2.0), _rand((B, H, N, d), 8), _rand((B, H, N, d), 9)
    kv_lens = [50, 0, 23]
    o, lse = orc.attn_fwd_naive(q, k, v, 0.3, causal, kv_lens)
    ot, lset = orc.attn_fwd_tiled(q, k, v, 0.3, causal, kv_lens, block=block)
    assert np.max(np.abs(o - ot)) < 1e-12
    assert np.array_equal(np.isfinite(lse), np.isfinite(lset))
    fin = np.isfinite(lse)
    assert np.max(np.abs(lse[fin] - lset[fin])) < 1e-12


def test_block_order_is_free():
    """Cell H and the associativity answers: streaming blocks in any order gives the same output."""
    B, H, N, d = 1, 2, 64, 8
    q, k, v = _rand((B, H, N, d), 10, 3.0), _rand((B, H, N, d), 11), _rand((B, H, N, d), 12)
    o, lse = orc.attn_fwd_tiled(q, k, v, 0.4, False, None, block=8)
    rng = np.random.default_rng(13)
    for order in (list(range(7, -1, -1)), list(rng.permutation(8))):
        o2, lse2 = orc.attn_fwd_tiled(q, k, v, 0.4, False, None, block=8, order=order)
        assert np.max(np.abs(o - o2)) < 1e-12
        assert np.max(np.abs(lse - lse2)) < 1e-12


def test_mutation_without_rescale_is_detected():
    """The red-team change (c forced to 1) must break agreement with the definition."""
    B, H, N, d = 1, 1, 64, 8
    q, k, v = _rand((B, H, N, d), 14, 3.0), _rand((B, H, N, d), 15), _rand((B, H, N, d), 16)
    o, _ = orc.attn_fwd_naive(q, k, v, 0.4)
    o_bad, _ = orc.attn_fwd_tiled(q, k, v, 0.4, block=8, rescale=False)
    assert np.max(np.abs(o - o_bad)) > 1e-2


def test_masked_keys_never_leak():
    """Cell D: hidden keys contribute exactly nothing; overwriting them changes no bit."""
    B, H, N, d = 2, 2, 40, 8
    q, k, v = _rand((B, H, N, d), 17), _rand((B, H, N, d), 18), _rand((B, H, N, d), 19)
    kv_lens = [30, 13]
    o, lse = orc.attn_fwd_naive(q, k, v, 0.35, True, kv_lens)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, :, kv_lens[b]:] = 1e30
        v2[b, :, kv_lens[b]:] = -1e30
    o2, lse2 = orc.attn_fwd_naive(q, k2, v2, 0.35, True, kv_lens)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_closed_form_rows():
    B, H, N, d = 3, 2, 24, 8
    q, k, v = _rand((B, H, N, d), 20), _rand((B, H, N, d), 21), _rand((B, H, N, d), 22)
    scale = 0.3
    o, lse = orc.attn_fwd_naive(q, k, v, scale, True, [24, 1, 0])
    # Causal row 0 sees only key 0: O_0 = V_0 exactly and lse_0 = s_00.
    assert np.array_equal(o[0, :, 0], v[0, :, 0])
    s00 = scale * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0])
    assert np.max(np.abs(lse[0, :, 0] - s00)) < 1e-14
    # kv_len = 1: every row sees only key 0.
    assert np.array_equal(o[1], np.broadcast_to(v[1, :, :1], o[1].shape))
    s_i0 = scale * np.einsum("hnd,hd->hn", q[1], k[1, :, 0])
    assert np.max(np.abs(lse[1] - s_i0)) < 1e-14
    # kv_len = 0: the guard (Cell D2) gives O = 0 and lse = -inf.
    assert np.all(o[2] == 0.0) and np.all(lse[2] == -INF)
    # Q = 0: every visible key has the same score, so the output is their mean (Cell C).
    oz, _ = orc.attn_fwd_naive(np.zeros_like(q), k, v, scale, True, None)
    means = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.max(np.abs(oz - means)) < 1e-13


def test_one_hot_limit():
    """Cell F through Q/K/V: one key whose score dominates pulls the output onto its value row."""
    N, d = 16, 4
    k = _rand((1, 1, N, d), 23)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)   # unit keys: the target's own score is the max
    v = _rand((1, 1, N, d), 24)
    target = 9
    errs = []
    for gain in (1.0, 10.0, 100.0, 1000.0):
        q = gain * k[:, :, target:target + 1]
        o, _ = orc.attn_fwd_naive(q, k[:, :, :N], v, 1.0, False, None)
        errs.append(np.max(np.abs(o[0, 0, 0] - v[0, 0, target])))
    assert errs[-1] < 1e-12 and all(a >= b for a, b in zip(errs, errs[1:]))


def _embed(scores, values, d=4):
    """q = e1, k_j = s_j e1, v_j = values_j in the leading coordinates: scores are exactly s_j."""
    n = len(scores)
    vals = np.atleast_2d(np.asarray(values, dtype=float))
    if vals.shape[0] == 1 and n > 1:
        vals = vals.T
    q = np.zeros((1, 1, n, d))
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, n, d))
    k[0, 0, :, 0] = scores
    v = np.zeros((1, 1, n, d))
    v[0, 0, :, : vals.shape[1]] = vals
    return q, k, v


def test_page_examples_through_qkv(golden):
    """The worked rows fed through the full attention (scale 1, one-hot embedding)."""
    for ex in golden["row_examples"]:
        if any(isinstance(s, str) for s in ex["scores"]):
            continue
        q, k, v = _embed(ex["scores"], ex["values"])
        o, _ = orc.attn_fwd_naive(q, k, v, 1.0)
        want, _, _, _ = orc.softmax_row_output(ex["scores"], ex["values"])
        assert np.max(np.abs(o[0, 0, 0, : want.shape[0]] - want)) < 1e-12
        assert abs(o[0, 0, 0, 0] - ex["printed"]["O"]) <= ex["tol"]["O"]
    # Cell D through the causal mask: query 1 of scores [2, 1, 4, 3].
    q, k, v = _embed([2.0, 1.0, 4.0, 3.0], [10.0, 20.0, 30.0, 40.0])
    o, _ = orc.attn_fwd_naive(q, k, v, 1.0, causal=True)
    assert abs(o[0, 0, 1, 0] - (10 + 20 * math.exp(-1)) / (1 + math.exp(-1))) < 1e-12
    # Cell D2 through key padding: no visible key at all.
    o, lse = orc.attn_fwd_naive(q, k, v, 1.0, causal=True, kv_lens=[0])
    assert np.all(o == 0.0) and np.all(lse == -INF)


def test_strict_causal_first_row_is_the_guard():
    # "Worked examples", Cell D2: with the strict mask the first query sees no
    # key at all, and the guard returns O = 0, lse = -inf.
    q, k, v = _rand((2, 3, 9, 5), 31), _rand((2, 3, 9, 5), 32), _rand((2, 3, 9, 5), 33)
    o, lse = orc.attn_fwd_naive(q, k, v, 0.4, "strict")
    assert np.all(o[:, :, 0] == 0.0) and np.all(lse[:, :, 0] == -INF)
    assert np.all(np.isfinite(lse[:, :, 1:]))
    # Row 1 sees key 0 only: O = V_0, lse = its score.
    assert np.max(np.abs(o[:, :, 1] - v[:, :, 0])) < 1e-15
    s10 = 0.4 * np.sum(q[:, :, 1] * k[:, :, 0], axis=-1)
    assert np.max(np.abs(lse[:, :, 1] - s10)) < 1e-14


@pytest.mark.parametrize("kv_lens", [None, [7, 3]])
def test_strict_causal_is_causal_shifted_by_one(kv_lens):
    # Query i under j < i is query i placed at position i-1 under j <= i-1:
    # drop the first query and the last key/value.
    B, H, N, d = 2, 2, 12, 4
    q, k, v = _rand((B, H, N, d), 41), _rand((B, H, N, d), 42), _rand((B, H, N, d), 43)
    o, lse = orc.attn_fwd_naive(q, k, v, 0.7, "strict", kv_lens)
    kv2 = None if kv_lens is None else [min(x, N - 1) for x in kv_lens]
    o2, lse2 = orc.attn_fwd_naive(q[:, :, 1:], k[:, :, :-1], v[:, :, :-1], 0.7, True, kv2)
    assert np.max(np.abs(o[:, :, 1:] - o2)) < 1e-13
    fin = np.isfinite(lse2)
    assert np.array_equal(fin, np.isfinite(lse[:, :, 1:]))
    assert np.max(np.abs(lse[:, :, 1:][fin] - lse2[fin])) < 1e-13


def test_unknown_mask_is_rejected():
    with pytest.raises(ValueError):
        orc.visible(4, 4, "diagonal", 4)


@pytest.mark.parametrize("causal", [False, True, "strict"])
@pytest.mark.parametrize("H,Hkv,N,Nk", [(4, 2, 5, 9), (3, 1, 8, 8), (2, 2, 1, 7), (4, 4, 6, 3)])
def test_grouped_heads_and_unequal_lengths_match_brute_force(causal, H, Hkv, N, Nk):
    B, d = 2, 3
    q = _rand((B, H, N, d), 51)
    k, v = _rand((B, Hkv, Nk, d), 52), _rand((B, Hkv, Nk, d), 53)
    for kv_lens in (None, [Nk, max(Nk - 2, 0)]):
        o, lse = orc.attn_fwd_naive(q, k, v, 0.6, causal, kv_lens)
        ob, lseb = _brute(q, k, v, 0.6, causal, kv_lens)
        assert np.max(np.abs(o - ob)) < 1e-13
        fin = np.isfinite(lseb)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.max(np.abs(lse[fin] - lseb[fin]), initial=0.0) < 1e-13


@pytest.mark.parametrize("Hkv", [1, 2, 3])
def test_grouped_heads_equal_repeated_kv(Hkv):
    # H_kv < H is the same attention as H heads of K/V, each group's K/V head
    # repeated for its query heads.
    B, H, N, d = 2, 6, 20, 8
    q = _rand((B, H, N, d), 61)
    k, v, do = _rand((B, Hkv, N, d), 62), _rand((B, Hkv, N, d), 63), _rand((B, H, N, d), 64)
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    for causal in (False, True):
        o, lse = orc.attn_fwd_naive(q, k, v, 0.35, causal, [20, 13])
        o2, lse2 = orc.attn_fwd_naive(q, kr, vr, 0.35, causal, [20, 13])
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
        dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.35, causal, [20, 13])
        dq2, dk2, dv2 = orc.attn_bwd(q, kr, vr, do, 0.35, causal, [20, 13])
        assert np.max(np.abs(dq - dq2)) < 1e-13
        G = H // Hkv
        assert np.max(np.abs(dk - dk2.reshape(B, Hkv, G, N, d).sum(axis=2))) < 1e-12
        assert np.max(np.abs(dv - dv2.reshape(B, Hkv, G, N, d).sum(axis=2))) < 1e-12


@pytest.mark.parametrize("causal", [True, "strict"])
def test_fewer_queries_are_the_last_rows_of_the_square_case(causal):
    # Bottom-right alignment: N_q queries against N_k keys are the last N_q
    # rows of the square causal computation whose last rows are those queries.
    B, H, Nk, Nq, d = 2, 2, 30, 7, 6
    k, v = _rand((B, H, Nk, d), 71), _rand((B, H, Nk, d), 72)
    q_full = _rand((B, H, Nk, d), 73)
    q = q_full[:, :, Nk - Nq:]
    o, lse = orc.attn_fwd_naive(q, k, v, 0.5, causal, [30, 25])
    of, lsef = orc.attn_fwd_naive(q_full, k, v, 0.5, causal, [30, 25])
    assert np.array_equal(o, of[:, :, Nk - Nq:]) and np.array_equal(lse, lsef[:, :, Nk - Nq:])
    ot, lset = orc.attn_fwd_tiled(q, k, v, 0.5, causal, [30, 25], block=4)
    assert np.max(np.abs(ot - o)) < 1e-12
    fin = np.isfinite(lse)
    assert np.max(np.abs(lset[fin] - lse[fin])) < 1e-12


def test_single_query_sees_every_key_under_the_causal_mask():
    # Decoding: one query against N_k keys is aligned to the last position.
    q, k, v = _rand((1, 2, 1, 8), 81), _rand((1, 2, 50, 8), 82), _rand((1, 2, 50, 8), 83)
    o, lse = orc.attn_fwd_naive(q, k, v, 0.3, True)
    o2, lse2 = orc.attn_fwd_naive(q, k, v, 0.3, False)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_kv_heads_must_divide_query_heads():
    with pytest.raises(ValueError):
        orc.attn_fwd_naive(_rand((1, 3, 4, 2), 1), _rand((1, 2, 4, 2), 2), _rand((1, 2, 4, 2), 3), 1.0)
