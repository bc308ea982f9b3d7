"""Plain, slow, float64 CPU oracle for exact softmax attention (forward + backward).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

What it computes
----------------
Forward, for every batch b and query head h, with KV head ``kv = h // (H/Hkv)``:

    S  = s * Q[b,h] @ K[b,kv]^T                      (N x N, materialised)
    S[i, j] = -inf for j > i                          (causal only)
    m_i = max_j S_ij ;  P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i)
    O  = P @ V[b,kv] ;  LSE_i = m_i + log(sum_j exp(S_ij - m_i))

This is the materialised attention of the standard-attention code block in
the FA2-backward page ("FlashAttention V2深度解析", section
"Attention反向传播的「内存泄漏」难题": scores from Q K^T divided by sqrt(D),
a softmax, then a product with V), with the max-subtracted softmax of the
FA explainer page ("【词汇专栏】FlashAttention", section 2.2 在线Softmax,
``standard_softmax``).  The Ascend page ("FlashAttention 在昇腾NPU上到底快在哪",
section 三、增量 Softmax) and the explainer's FAQ state that the tiled/online
softmax reaches exactly this result up to rounding, so the oracle is the
definition itself, not a replay of any tiling.

Backward is the exact chain rule through that definition.  The softmax step
uses the explicit Jacobian ``J_i = diag(P_i) - P_i P_i^T`` (formed as an
N x N matrix per row for N <= 256) or, for larger N, the algebraically equal
contraction ``dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)``.  It deliberately does
not use ``rowsum(dO * O)``, so it shares no formula with the GPU's backward
preprocess.  The backward code block printed on the FA2-backward page
(section 改进1：IO感知的算子调度) keeps only the Jacobian's diagonal and
normalises per block; it is taken as a statement of intent (recompute P,
never store it), not as a formula.

Readings of points the pages leave open (each also listed in the design notes):
  * scale ``s`` is the float32 value handed to the library, upcast to float64;
  * LSE is the natural log of the sum of exp of the *scaled* scores, masked
    keys excluded;
  * causal is square: key j is visible to query i iff j <= i;
  * GQA maps query head h to KV head h // (H/Hkv); dK/dV sum over the group.

Pins: every function here is pinned by tests under ``tests/`` that do not
re-type these formulas: finite differences, closed forms, hand-derived worked
examples (``tests/golden``), exact identities and PyTorch float64 autograd.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

EXPLICIT_JACOBIAN_MAX_N = 256
_ROW_BLOCK = 512


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,H,N,d], k/v [B,Hkv,N,d]")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or H % k.shape[1]:
        raise ValueError("shape mismatch between q and k/v")
    return B, H, k.shape[1], N, d


def _scores(q_rows, k_all, s, rows, causal):
    """Scaled scores of the given query rows against all keys, causal mask applied."""
    S = s * (q_rows @ k_all.T)
    if causal:
        keys = np.arange(k_all.shape[0])
        S[keys[None, :] > rows[:, None]] = -np.inf
    return S


def _visible(rows, N, causal):
    """Number of leading keys any of these query rows can see.  Under the causal
    mask keys after the last row have probability exactly 0 for every row of the
    block, so leaving them out changes no value."""
    return int(np.max(rows)) + 1 if causal else N


def _softmax_rows(S):
    """Row softmax with max subtraction; returns P and the row log-sum-exp."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    Z = E.sum(axis=1, keepdims=True)
    return E / Z, (m + np.log(Z))[:, 0]


def softmax_vjp_explicit(P, dP):
    """dS_i = J_i^T dP_i with J_i = diag(P_i) - P_i P_i^T formed explicitly."""
    out = np.empty_like(P)
    for r in range(P.shape[0]):
        p = P[r]
        J = np.diag(p) - np.outer(p, p)
        out[r] = J.T @ dP[r]
    return out


def softmax_vjp_contracted(P, dP):
    """dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik): the same Jacobian, contracted."""
    return P * (dP - np.sum(P * dP, axis=1, keepdims=True))


def _softmax_vjp(P, dP, n_keys):
    if n_keys <= EXPLICIT_JACOBIAN_MAX_N:
        return softmax_vjp_explicit(P, dP)
    return softmax_vjp_contracted(P, dP)


def _row_sets(rows, B, H, N):
    if rows is None:
        full = np.arange(N)
        return lambda b, h: full
    rows = np.asarray(rows)
    if rows.ndim == 1:
        return lambda b, h: rows
    return lambda b, h: rows[b, h]


def _head_fwd(qh, kh, vh, s, causal, r_all):
    """O and LSE of one head on the query rows r_all."""
    N = kh.shape[0]
    O = np.empty((len(r_all), qh.shape[1])); LSE = np.empty(len(r_all))
    for a in range(0, len(r_all), _ROW_BLOCK):
        r = r_all[a:a + _ROW_BLOCK]
        n = _visible(r, N, causal)
        P, lse = _softmax_rows(_scores(qh[r], kh[:n], s, r, causal))
        O[a:a + len(r)] = P @ vh[:n]
        LSE[a:a + len(r)] = lse
    return O, LSE


def _head_bwd(qh, kh, vh, doh, s, causal, r_sel, kr):
    """One query head's share of the backward pass.

    Returns dQ on the rows r_sel (all rows when r_sel is None) and this head's
    contribution to dK/dV on the key rows kr.
    """
    N, d = kh.shape
    full_q = r_sel is None
    dQ = np.empty((N if full_q else len(r_sel), d))
    dK = np.zeros((len(kr), d)); dV = np.zeros((len(kr), d))
    if not full_q:
        for a in range(0, len(r_sel), _ROW_BLOCK):
            r = r_sel[a:a + _ROW_BLOCK]
            n = _visible(r, N, causal)
            P, _ = _softmax_rows(_scores(qh[r], kh[:n], s, r, causal))
            dP = doh[r] @ vh[:n].T
            dS = _softmax_vjp(P, dP, N)
            dQ[a:a + len(r)] = s * (dS @ kh[:n])
    # dK/dV need every query row that sees a selected key: under the causal mask
    # rows before the first selected key contribute exactly zero.
    start = int(kr.min()) if (causal and not full_q) else 0
    for a in range(start, N, _ROW_BLOCK):
        r = np.arange(a, min(a + _ROW_BLOCK, N))
        n = _visible(r, N, causal)
        P, _ = _softmax_rows(_scores(qh[r], kh[:n], s, r, causal))
        dP = doh[r] @ vh[:n].T
        dS = _softmax_vjp(P, dP, N)
        if full_q:
            dQ[r] = s * (dS @ kh[:n])
        sel = np.nonzero(kr < n)[0]
        dV[sel] += P[:, kr[sel]].T @ doh[r]
        dK[sel] += s * (dS[:, kr[sel]].T @ qh[r])
    return dQ, dK, dV


def _map_heads(fn, jobs, n_keys):
    """Runs independent per-head jobs, concurrently when there are several
    large ones.

    Heads share nothing, so running them on several threads changes no value;
    BLAS is limited to one thread per job while the pool is active.
    """
    workers = min(len(jobs), len(os.sched_getaffinity(0))) if n_keys >= 1024 else 1
    if workers <= 1:
        return [fn(*j) for j in jobs]
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(lambda j: fn(*j), jobs))


def attention_fwd_ref(q, k, v, scale, causal, rows=None):
    """Forward oracle.  Returns (O, LSE) in float64.

    ``rows``: None for every query row, else an index array shared by all
    heads ([R]) or one per head ([B, H, R]); outputs then hold those rows only.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    B, H, Hkv, N, d = _check(q, k, v)
    g = H // Hkv
    s = float(scale)
    pick = _row_sets(rows, B, H, N)
    R = len(pick(0, 0))
    heads = [(b, h) for b in range(B) for h in range(H)]
    res = _map_heads(_head_fwd, [(q[b, h], k[b, h // g], v[b, h // g], s, causal, pick(b, h)) for b, h in heads], N)
    O = np.empty((B, H, R, d)); LSE = np.empty((B, H, R))
    for (b, h), (o, lse) in zip(heads, res):
        O[b, h] = o
        LSE[b, h] = lse
    return O, LSE


def attention_bwd_ref(q, k, v, do, scale, causal, rows=None, key_rows=None):
    """Backward oracle.  Returns (dQ, dK, dV) in float64 for L = sum(dO * O).

    ``rows`` selects the query rows of dQ (as in ``attention_fwd_ref``);
    ``key_rows`` selects the key rows of dK/dV (None, [Rk] or [B, Hkv, Rk]).
    GQA: dK/dV of a KV head sum the contributions of its query heads, added in
    ascending head order.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    B, H, Hkv, N, d = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must match q")
    g = H // Hkv
    s = float(scale)
    qpick = _row_sets(rows, B, H, N)
    kpick = _row_sets(key_rows, B, Hkv, N)
    R = len(qpick(0, 0)); Rk = len(kpick(0, 0))
    heads = [(b, h) for b in range(B) for h in range(H)]
    jobs = [(q[b, h], k[b, h // g], v[b, h // g], do[b, h], s, causal,
             None if rows is None else qpick(b, h), kpick(b, h // g)) for b, h in heads]
    res = _map_heads(_head_bwd, jobs, N)
    dQ = np.empty((B, H, R, d))
    dK = np.zeros((B, Hkv, Rk, d)); dV = np.zeros((B, Hkv, Rk, d))
    for (b, h), (dq, dk, dv) in zip(heads, res):
        dQ[b, h] = dq
        dK[b, h // g] += dk
        dV[b, h // g] += dv
    return dQ, dK, dV


def attention_ref(q, k, v, do, scale, causal):
    """Full forward and backward: (O, LSE, dQ, dK, dV), all float64."""
    O, LSE = attention_fwd_ref(q, k, v, scale, causal)
    dQ, dK, dV = attention_bwd_ref(q, k, v, do, scale, causal)
    return O, LSE, dQ, dK, dV
