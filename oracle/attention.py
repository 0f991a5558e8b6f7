"""Exact-attention oracle: plain, slow, fp64, CPU only.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module. The GPU library never does, and this
module imports nothing from it: the two share no code.

What is computed (sources are the five pages on exact, IO-aware attention):

* Scores S = scale * Q K^T, one row per query and one column per key
  ("Foundations", sections 4 and 9: the dot product of a query row with every
  key, and the 1/sqrt(d_k) divisor applied to the scores).
* Masked scores are -inf, so their exponential is exactly 0
  ("Worked examples", Cell D: future keys masked to -inf).
* Safe softmax: subtract the row max m before exponentiating, then divide by
  the row sum l ("Foundations", sections 7 and 8).
* A row whose keys are all masked has l = 0; it returns O = 0 and
  logsumexp = -inf ("Worked examples", Cell D2, the guard, first convention).
* The output row is O_i = sum_j softmax(S_i)_j V_j and the saved statistic is
  lse_i = m_i + ln l_i.

Readings taken where the pages leave a step open (each is listed with the
design notes of this repository):

* causal means key j is visible to query i iff j <= i + (N_k - N_q): with
  N_q = N_k that is j <= i, and with fewer queries than keys the queries are
  the last N_q positions (bottom-right alignment, as when new queries attend
  to a longer cache); the strict variant (j < i + (N_k - N_q)), which the
  pages use in Cell D2 to produce a row with no visible key, is selected with
  causal="strict";
* grouped heads: K and V may have H_kv heads, a divisor of the H query
  heads; query head h reads K/V head h // (H / H_kv) (H_kv = H is the
  pages' per-head attention, H_kv = 1 a single shared K/V head);
* key padding kv_lens[b] hides keys j >= kv_lens[b] for every query of batch
  b; queries are never dropped;
* the merge of two states whose maxima are both -inf keeps the empty state
  (-inf, 0, 0) instead of forming exp(-inf - (-inf)) = NaN;
* the backward pass is the textbook derivative of the definition above; the
  pages only say that S and P are recomputed from Q, K, V rather than stored
  ("Question bank": backward recomputation at about 1.2x the FLOPs).

Every function works in float64 on numpy arrays and materialises the full
score row or matrix it needs: there is no blocking or fusion beyond what the
named algorithm itself states.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# Score-level core: one row of scores against value vectors.
# --------------------------------------------------------------------------

def softmax_row_output(scores: Sequence[float], values) -> Tuple[np.ndarray, float, float, float]:
    """Plain safe softmax over ONE row of scores, then the weighted sum of values.

    ``scores``: length-n row (entries may be -inf for masked keys).
    ``values``: n value vectors, shape (n,) or (n, dv).
    Returns (O, m, l, lse): output vector, row max, row sum of exp(s - m), and
    logsumexp. Follows "Foundations" sections 7-8 (exponentiate after the max
    shift, divide by the sum) and the fully-masked guard of "Worked examples",
    Cell D2 (l = 0 -> O = 0, lse = -inf).
    """
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    if vals.ndim == 1:
        vals = vals[:, None]
    m = float(np.max(s)) if s.size else NEG_INF
    if m == NEG_INF:
        return np.zeros(vals.shape[1]), NEG_INF, 0.0, NEG_INF
    p = np.exp(s - m)
    l = float(np.sum(p))
    o = (p @ vals) / l
    return o, m, l, m + math.log(l)


# --------------------------------------------------------------------------
# Block states and the two-block merge.
# --------------------------------------------------------------------------

def block_state(scores: Sequence[float], values) -> Tuple[float, float, np.ndarray]:
    """State (m, l, O~) of one block of scores, measured against the block's own max.

    O~ is the unnormalised output sum_j exp(s_j - m) v_j ("Worked examples",
    the recipe before the scenario matrix, and Cells A and B: each block is
    max-shifted independently before any merge). An all-masked block gives
    the empty state (-inf, 0, 0) ("Worked examples", Cell D, block 2).
    """
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    if vals.ndim == 1:
        vals = vals[:, None]
    m = float(np.max(s)) if s.size else NEG_INF
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros(vals.shape[1])
    p = np.exp(s - m)
    return m, float(np.sum(p)), p @ vals


def merge(a: Tuple[float, float, np.ndarray], b: Tuple[float, float, np.ndarray],
          rescale: bool = True) -> Tuple[float, float, np.ndarray]:
    """Merge two block states re-referenced to the common max.

    m_new = max(m1, m2); each side is multiplied by exp(m_b - m_new) before the
    sums are added ("Exercises", the two-block merges; "Question bank", the
    rescale-before-adding answer). When both maxima are -inf the result stays
    the empty state (reading of "Worked examples", Cell D2, where the pages
    say every term is zero).

    ``rescale=False`` drops the exp(m_old - m_new) factors (both set to 1).
    That is the deliberate mistake of the interactive explainer's "red team";
    it exists only so the tests can show that they detect it.
    """
    m1, l1, o1 = a
    m2, l2, o2 = b
    m_new = max(m1, m2)
    if m_new == NEG_INF:
        return NEG_INF, 0.0, np.zeros_like(np.asarray(o1, dtype=np.float64))
    if rescale:
        f1 = 0.0 if m1 == NEG_INF else math.exp(m1 - m_new)
        f2 = 0.0 if m2 == NEG_INF else math.exp(m2 - m_new)
    else:
        f1 = 1.0
        f2 = 1.0
    return m_new, f1 * l1 + f2 * l2, f1 * np.asarray(o1) + f2 * np.asarray(o2)


def finalize(state: Tuple[float, float, np.ndarray]) -> Tuple[np.ndarray, float]:
    """Divide once by the complete normaliser; guard l = 0.

    ("Worked examples", the "why divide only at the end" recall card and
    Cell D2's guard.) Returns (O, lse).
    """
    m, l, o = state
    if l == 0.0:
        return np.zeros_like(np.asarray(o, dtype=np.float64)), NEG_INF
    return np.asarray(o) / l, m + math.log(l)


def online_row(scores: Sequence[float], values, block: int,
               order: Optional[Iterable[int]] = None,
               rescale: bool = True) -> Tuple[np.ndarray, float, float, float]:
    """Streaming (online) softmax over one score row, ``block`` keys at a time.

    Carries (m, l, acc) and, for each new block with block max m',
    sets m_new = max(m, m'), c = exp(m - m_new), l <- l*c + sum exp(s - m_new),
    acc <- acc*c + sum exp(s - m_new) v, and divides acc by l once at the end
    (the interactive explainer's recurrence). A block whose m_new is -inf is
    skipped, so the state stays empty (reading of Cell D2).
    ``order`` lists block indices in the order they are streamed (default:
    ascending); ``rescale=False`` forces c = 1 (the red-team mutation).
    Returns (O, m, l, lse).
    """
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    if vals.ndim == 1:
        vals = vals[:, None]
    n = s.shape[0]
    nblocks = (n + block - 1) // block
    blocks = range(nblocks) if order is None else list(order)
    m = NEG_INF
    l = 0.0
    acc = np.zeros(vals.shape[1])
    for bi in blocks:
        lo, hi = bi * block, min(n, (bi + 1) * block)
        sb = s[lo:hi]
        m_blk = float(np.max(sb)) if sb.size else NEG_INF
        m_new = max(m, m_blk)
        if m_new == NEG_INF:
            continue
        c = (0.0 if m == NEG_INF else math.exp(m - m_new)) if rescale else 1.0
        p = np.exp(sb - m_new)
        l = l * c + float(np.sum(p))
        acc = acc * c + p @ vals[lo:hi]
        m = m_new
    if l == 0.0:
        return np.zeros(vals.shape[1]), NEG_INF, 0.0, NEG_INF
    return acc / l, m, l, m + math.log(l)


# --------------------------------------------------------------------------
# Q/K/V level: the full attention, materialising S.
# --------------------------------------------------------------------------

def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible(n_rows: int, n_keys: int, causal, kv_len: int,
            rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [len(rows), n_keys]: key j visible to query i.

    causal is False (no mask), True (j <= i + off) or "strict"
    (j < i + off), with off = n_keys - n_rows: query i sits at key position
    i + off (bottom-right alignment; off = 0 when there are as many queries
    as keys). Visible iff the causal condition holds and j < kv_len. Causal
    masking follows "Worked examples", Cell D (keys in the query's future
    are hidden); the strict form, which also hides the query's own position,
    is the variant of Cell D2; the key-padding length is this repository's
    reading for batched, padded inputs (keys only are padded).
    """
    if causal not in (False, True, "strict"):
        raise ValueError("causal must be False, True or 'strict'")
    if rows is None:
        rows = np.arange(n_rows)
    i = np.asarray(rows)[:, None] + (n_keys - n_rows)
    j = np.arange(n_keys)[None, :]
    vis = j < kv_len
    if causal == "strict":
        vis = vis & (j < i)
    elif causal:
        vis = vis & (j <= i)
    return vis


def _kv_head(h: int, H: int, Hkv: int) -> int:
    """K/V head read by query head h when K and V have Hkv of the H heads."""
    if Hkv <= 0 or H % Hkv:
        raise ValueError("the number of K/V heads must divide the number of query heads")
    return h // (H // Hkv)


def _kv_len(kv_lens, b: int, n: int) -> int:
    if kv_lens is None:
        return n
    return int(min(max(int(kv_lens[b]), 0), n))


def attn_fwd_naive(q, k, v, scale: float, causal: bool = False, kv_lens=None,
                   rows: Optional[Sequence[int]] = None,
                   heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Standard attention by its definition, with the full score matrix.

    q: [B, H, N, d]; k, v: [B, H_kv, N_k, d] with H_kv dividing H (any float
    dtype; upcast to float64 losslessly).
    scale: the caller's scale (tests pass the float32 value the GPU receives).
    causal: False, True or "strict" (see ``visible``: bottom-right aligned
    when N_k != N).
    kv_lens: None or per-batch valid key counts (clamped to [0, N_k]).
    rows: optional query indices to compute (rows are independent, so this is
    the same definition restricted to those rows).
    heads: optional list of (b, h) to compute; others are left as NaN.
    Returns (O [B, H, R, d], lse [B, H, R]) in float64, R = len(rows) or N.

    For each (b, h): S = scale * Q K^T; S_ij = -inf where hidden;
    m_i = max_j S_ij; if m_i = -inf then O_i = 0, lse_i = -inf; otherwise
    P_ij = exp(S_ij - m_i), l_i = sum_j P_ij, O_i = (P V)_i / l_i and
    lse_i = m_i + ln l_i ("Foundations", sections 4, 7, 8, 9; "Worked
    examples", Cells D and D2).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    alpha = float(scale)
    row_idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    dv = v.shape[3]
    o_out = np.full((B, H, R, dv), np.nan)
    lse_out = np.full((B, H, R), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        kvl = _kv_len(kv_lens, b, Nk)
        hk = _kv_head(h, H, Hkv)
        vis = visible(N, Nk, causal, kvl, row_idx)
        s = alpha * (q[b, h, row_idx] @ k[b, hk].T)
        s = np.where(vis, s, NEG_INF)
        m = np.max(s, axis=1)
        empty = m == NEG_INF
        m_safe = np.where(empty, 0.0, m)
        p = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 on hidden keys
        l = np.sum(p, axis=1)
        num = p @ v[b, hk]
        with np.errstate(invalid="ignore", divide="ignore"):
            o = num / l[:, None]
            lse = m + np.log(l)
        o[empty] = 0.0
        lse[empty] = NEG_INF
        o_out[b, h] = o
        lse_out[b, h] = lse
    return o_out, lse_out


def attn_fwd_tiled(q, k, v, scale: float, causal: bool = False, kv_lens=None,
                   block: int = 32, order: Optional[Sequence[int]] = None,
                   rescale: bool = True):
    """The same attention computed by streaming KV blocks with the online recurrence.

    Every query row streams its score row in blocks of ``block`` keys through
    ``online_row`` (the interactive explainer's recurrence). ``order`` permutes
    the block order (block order is free: "Worked examples", Cell H).
    Returns (O [B, H, N, d], lse [B, H, N]) in float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    alpha = float(scale)
    o_out = np.zeros((B, H, N, v.shape[3]))
    lse_out = np.zeros((B, H, N))
    for b in range(B):
        kvl = _kv_len(kv_lens, b, Nk)
        for h in range(H):
            hk = _kv_head(h, H, Hkv)
            vis = visible(N, Nk, causal, kvl)
            s_all = alpha * (q[b, h] @ k[b, hk].T)
            s_all = np.where(vis, s_all, NEG_INF)
            for i in range(N):
                o, _, _, lse = online_row(s_all[i], v[b, hk], block, order, rescale)
                o_out[b, h, i] = o
                lse_out[b, h, i] = lse
    return o_out, lse_out


def attn_bwd(q, k, v, do, scale: float, causal: bool = False, kv_lens=None):
    """Gradients of L = sum(dO * O) with P recomputed from the saved logsumexp.

    The pages state only that the backward pass recomputes S and P from Q, K,
    V instead of storing them ("Question bank"); the formulas are the textbook
    derivative of the forward definition:
        P_ij = exp(S_ij - lse_i)   (0 where hidden or where lse_i = -inf)
        D_i  = sum_k dO_ik O_ik
        dV   = P^T dO
        dP   = dO V^T
        dS   = P * (dP - D)
        dQ   = scale * dS K
        dK   = scale * dS^T Q
    With grouped K/V heads (H_kv < H), dK and dV of a K/V head sum the
    contributions of every query head that reads it.
    O and lse come from this module's own forward. Returns (dq, dk, dv) float64.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    alpha = float(scale)
    o, lse = attn_fwd_naive(q, k, v, scale, causal, kv_lens)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        kvl = _kv_len(kv_lens, b, Nk)
        vis = visible(N, Nk, causal, kvl)
        for h in range(H):
            hk = _kv_head(h, H, Hkv)
            s = alpha * (q[b, h] @ k[b, hk].T)
            lse_bh = lse[b, h]
            empty = lse_bh == NEG_INF
            shift = np.where(empty, 0.0, lse_bh)
            p = np.exp(s - shift[:, None])
            p = np.where(vis & ~empty[:, None], p, 0.0)
            D = np.sum(do[b, h] * o[b, h], axis=1)
            dv[b, hk] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            ds = p * (dp - D[:, None])
            dq[b, h] = alpha * (ds @ k[b, hk])
            dk[b, hk] += alpha * (ds.T @ q[b, h])
    return dq, dk, dv

