"""fp64 softmax attention, LSE merge and backward — the oracle (test infrastructure).

Notation: a query chunk holds ``nq`` rows with global positions ``qpos``; a
KV chunk holds ``nk`` keys with global positions ``kpos``.  Tensors are
tokens-major: q [nq, hq, d], k and v [nk, hkv, d].  Query head h reads KV
head h // (hq // hkv) (contiguous GQA groups; the GQA paper is only named in
the TASP citation map, the grouping is the plain reading).

The definition (Attention Is All You Need, named in the TASP citation map;
exactness is required by the TASP abstract, where every query chunk attends
to every KV chunk):

    allowed(i, j)  NONE:        always
                   CAUSAL:      kpos[j] <= qpos[i]
                   DOC_CAUSAL:  CAUSAL and doc(qpos[i]) == doc(kpos[j])
                                (HSAP abstract / methodology: causal attention
                                on packed sequences with no cross-document
                                attention)
    s_ij   = scale * <q_i, k_j>
    LSE_i  = ln sum_{allowed j} exp(s_ij)          (-inf if row i has no key)
    P_ij   = exp(s_ij - LSE_i) if allowed else 0
    O_i    = sum_j P_ij v_j                         (0 if row i has no key)

A ring step evaluates this with the keys restricted to one KV chunk and
returns (O, LSE) as its partial result; merging partials with weights
exp(LSE_part - LSE_total) gives the attention over the union of the keys
(the blockwise exact attention of FlashAttention / Self-attention Does Not
Need O(n^2) Memory, both named in the TASP citation map).
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL = 0, 1, 2


def doc_of(pos: np.ndarray, cu_seqlens: np.ndarray) -> np.ndarray:
    """Document index t with cu[t] <= pos < cu[t+1] (cu is ascending, cu[0] = 0)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    t = np.searchsorted(cu, pos, side="right") - 1
    if np.any(t < 0) or np.any(pos >= cu[-1]):
        raise ValueError("position outside the packed buffer")
    return t


def allowed_mask(qpos: np.ndarray, kpos: np.ndarray, mask: int,
                 cu_seqlens: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [nq, nk]: may query row i attend to key j."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    if mask == MASK_NONE:
        return np.ones((qpos.size, kpos.size), dtype=bool)
    causal = kpos[None, :] <= qpos[:, None]
    if mask == MASK_CAUSAL:
        return causal
    if mask == MASK_DOC_CAUSAL:
        if cu_seqlens is None:
            raise ValueError("document mask needs cu_seqlens")
        same_doc = doc_of(qpos, cu_seqlens)[:, None] == doc_of(kpos, cu_seqlens)[None, :]
        return causal & same_doc
    raise ValueError(f"unknown mask {mask}")


def count_pairs(qpos, kpos, mask, cu_seqlens=None, row_block: int = 2048) -> int:
    """Number of allowed (query row, key) pairs, per head."""
    qpos = np.asarray(qpos, dtype=np.int64)
    total = 0
    for i0 in range(0, qpos.size, row_block):
        total += int(allowed_mask(qpos[i0:i0 + row_block], kpos, mask, cu_seqlens).sum())
    return total


def _check_shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [tokens, heads, d]")
    nq, hq, d = q.shape
    nk, hkv, dk = k.shape
    if v.shape[:2] != k.shape[:2] or dk != d:
        raise ValueError("k and v must have the same tokens and heads, and k's width must match q's")
    if hkv == 0 or hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    return nq, hq, d, nk, hkv, hq // hkv


def _head_probs(s: np.ndarray, allow: np.ndarray):
    """Row-wise masked softmax of one head's scores: (P, LSE), empty rows -> (0, -inf)."""
    has_key = allow.any(axis=1)
    s_masked = np.where(allow, s, -np.inf)
    m = np.where(has_key, s_masked.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(allow, np.exp(s_masked - m[:, None]), 0.0)
    l = e.sum(axis=1)
    lse = np.where(has_key, m + np.log(np.where(has_key, l, 1.0)), -np.inf)
    p = np.where(has_key[:, None], e / np.where(has_key, l, 1.0)[:, None], 0.0)
    return p, lse


def attention(q, k, v, qpos, kpos, mask: int, scale: float,
              cu_seqlens=None, row_block: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of the query rows against the given keys.

    Returns O [nq, hq, dv] and LSE [hq, nq], both float64.  Query rows are
    independent, so they are computed ``row_block`` at a time.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, hq, d, nk, hkv, group = _check_shapes(q, k, v)
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    o = np.zeros((nq, hq, v.shape[2]))
    lse = np.full((hq, nq), -np.inf)
    for i0 in range(0, nq, row_block):
        i1 = min(nq, i0 + row_block)
        allow = allowed_mask(qpos[i0:i1], kpos, mask, cu_seqlens)
        for h in range(hq):
            g = h // group
            s = scale * (q[i0:i1, h, :] @ k[:, g, :].T)
            p, lse[h, i0:i1] = _head_probs(s, allow)
            o[i0:i1, h, :] = p @ v[:, g, :]
    return o, lse


def merge(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """LSE-weighted merge of two partial results over disjoint key sets.

    LSE = ln(e^{LSE_a} + e^{LSE_b});  O = e^{LSE_a - LSE} O_a + e^{LSE_b - LSE} O_b.
    A partial with LSE = -inf (no keys) has weight 0; two empty partials give
    (0, -inf).  o_* are [nq, hq, d], lse_* are [hq, nq].
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    empty = np.isneginf(lse)
    safe = np.where(empty, 0.0, lse)
    w_a = np.where(empty, 0.0, np.exp(lse_a - safe))   # [hq, nq]
    w_b = np.where(empty, 0.0, np.exp(lse_b - safe))
    o = w_a.T[:, :, None] * o_a + w_b.T[:, :, None] * o_b
    return o, lse


def merge_many(parts: Iterable[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Fold ``merge`` over a sequence of (O, LSE) partials, in the given order."""
    it = iter(parts)
    o, lse = next(it)
    for o_b, lse_b in it:
        o, lse = merge(o, lse, o_b, lse_b)
    return np.asarray(o, dtype=np.float64), np.asarray(lse, dtype=np.float64)


def _score_grad(p: np.ndarray, dp: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """dS_ij = P_ij (dP_ij - delta_i): the softmax Jacobian applied to dP."""
    return p * (dp - delta[:, None])


def attention_backward(q, k, v, do, qpos, kpos, mask: int, scale: float,
                       cu_seqlens=None, row_block: int = 1024):
    """Gradients of L = sum_{i,h,c} dO[i,h,c] * O[i,h,c] with respect to q, k, v.

    The keys are all keys the query rows can see; dO is the upstream gradient
    on these rows (zero on every other row of the sequence).  With
    delta_i = sum_c dO_ic O_ic:
        dP_ij = <dO_i, v_j>
        dS_ij = P_ij (dP_ij - delta_i)
        dQ_i  = scale * sum_j dS_ij k_j
        dK_j  = scale * sum_{i, h in group(g)} dS_ij q_i
        dV_j  = sum_{i, h in group(g)} P_ij dO_i
    Returns dq [nq,hq,d], dk [nk,hkv,d], dv [nk,hkv,dv], delta [hq,nq],
    O [nq,hq,dv] and LSE [hq,nq], all float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nq, hq, d, nk, hkv, group = _check_shapes(q, k, v)
    if do.shape != (nq, hq, v.shape[2]):
        raise ValueError("dO must be [nq, hq, dv]")
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    dq = np.zeros((nq, hq, d))
    dk = np.zeros((nk, hkv, d))
    dv = np.zeros(v.shape)
    o = np.zeros((nq, hq, v.shape[2]))
    lse = np.full((hq, nq), -np.inf)
    delta = np.zeros((hq, nq))
    for i0 in range(0, nq, row_block):
        i1 = min(nq, i0 + row_block)
        allow = allowed_mask(qpos[i0:i1], kpos, mask, cu_seqlens)
        for h in range(hq):
            g = h // group
            s = scale * (q[i0:i1, h, :] @ k[:, g, :].T)
            p, lse[h, i0:i1] = _head_probs(s, allow)
            o_h = p @ v[:, g, :]
            o[i0:i1, h, :] = o_h
            do_h = do[i0:i1, h, :]
            dlt = (do_h * o_h).sum(axis=1)
            delta[h, i0:i1] = dlt
            dp = do_h @ v[:, g, :].T
            ds = _score_grad(p, dp, dlt)
            dq[i0:i1, h, :] = scale * (ds @ k[:, g, :])
            dk[:, g, :] += scale * (ds.T @ q[i0:i1, h, :])
            dv[:, g, :] += p.T @ do_h
    return dq, dk, dv, delta, o, lse


def attention_backward_sampled(q, k, v, do, qpos, kpos, mask: int, scale: float, cu_seqlens=None,
                               rows=None, keys=None, heads=None, row_block: int = 512):
    """The gradients of ``attention_backward`` on a sample of its outputs.

    dq for query rows ``rows``, dk and dv for keys ``keys``, for the query
    heads ``heads`` (dk / dv of a KV head sum only the listed heads of its
    group, so pass whole groups to get the full dk / dv).  The softmax
    statistics (LSE, O and delta) of every query row are computed first,
    exactly as in the full backward; then only the sampled rows of dS and
    the sampled columns of P and dS are formed.
    Returns dq [len(rows), len(heads), d], dk and dv [len(keys), hkv, d]
    (zero for KV heads with no listed query head).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nq, hq, d, nk, hkv, group = _check_shapes(q, k, v)
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    rows = np.arange(nq) if rows is None else np.asarray(rows)
    keys = np.arange(nk) if keys is None else np.asarray(keys)
    heads = list(range(hq)) if heads is None else list(heads)
    dq = np.zeros((len(rows), len(heads), d))
    dk = np.zeros((len(keys), hkv, d))
    dv = np.zeros((len(keys), hkv, v.shape[2]))
    for hi, h in enumerate(heads):
        g = h // group
        lse = np.full(nq, -np.inf)
        delta = np.zeros(nq)
        for i0 in range(0, nq, row_block):
            i1 = min(nq, i0 + row_block)
            allow = allowed_mask(qpos[i0:i1], kpos, mask, cu_seqlens)
            s = scale * (q[i0:i1, h, :] @ k[:, g, :].T)
            p, lse[i0:i1] = _head_probs(s, allow)
            delta[i0:i1] = (do[i0:i1, h, :] * (p @ v[:, g, :])).sum(axis=1)
        # sampled rows of dS -> dq
        allow = allowed_mask(qpos[rows], kpos, mask, cu_seqlens)
        s = scale * (q[rows, h, :] @ k[:, g, :].T)
        p, _ = _head_probs(s, allow)
        ds = _score_grad(p, do[rows, h, :] @ v[:, g, :].T, delta[rows])
        dq[:, hi, :] = scale * (ds @ k[:, g, :])
        # sampled columns of P and dS -> dk, dv
        allow = allowed_mask(qpos, kpos[keys], mask, cu_seqlens)
        s = scale * (q[:, h, :] @ k[keys, g, :].T)
        has = ~np.isneginf(lse)
        p = np.where(allow & has[:, None], np.exp(s - np.where(has, lse, 0.0)[:, None]), 0.0)
        ds = _score_grad(p, do[:, h, :] @ v[keys, g, :].T, delta)
        dk[:, g, :] += scale * (ds.T @ q[:, h, :])
        dv[:, g, :] += p.T @ do[:, h, :]
    return dq, dk, dv
