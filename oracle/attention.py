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
    O = np.empty((B, H, R, d)); LSE = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            kv = h // g
            r_all = pick(b, h)
            for a in range(0, R, _ROW_BLOCK):
                r = r_all[a:a + _ROW_BLOCK]
                n = _visible(r, N, causal)
                P, lse = _softmax_rows(_scores(q[b, h, r], k[b, kv, :n], s, r, causal))
                O[b, h, a:a + len(r)] = P @ v[b, kv, :n]
                LSE[b, h, a:a + len(r)] = lse
    return O, LSE


def attention_bwd_ref(q, k, v, do, scale, causal, rows=None, key_rows=None):
    """Backward oracle.  Returns (dQ, dK, dV) in float64 for L = sum(dO * O).

    ``rows`` selects the query rows of dQ (as in ``attention_fwd_ref``);
    ``key_rows`` selects the key rows of dK/dV (None, [Rk] or [B, Hkv, Rk]).
    dK/dV of a key need every query row that sees it, so those rows are all
    visited; under the causal mask rows i < min(selected keys) contribute
    exactly zero and are skipped.
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
    dQ = np.empty((B, H, R, d))
    dK = np.zeros((B, Hkv, Rk, d)); dV = np.zeros((B, Hkv, Rk, d))
    full_q = rows is None
    for b in range(B):
        for h in range(H):
            kv = h // g
            # dQ on the selected query rows.
            if not full_q:
                r_all = qpick(b, h)
                for a in range(0, R, _ROW_BLOCK):
                    r = r_all[a:a + _ROW_BLOCK]
                    n = _visible(r, N, causal)
                    P, _ = _softmax_rows(_scores(q[b, h, r], k[b, kv, :n], s, r, causal))
                    dP = do[b, h, r] @ v[b, kv, :n].T
                    dS = _softmax_vjp(P, dP, N)
                    dQ[b, h, a:a + len(r)] = s * (dS @ k[b, kv, :n])
            # dK/dV on the selected key rows (and dQ on all rows when full).
            kr = kpick(b, kv)
            start = int(kr.min()) if (causal and not full_q) else 0
            for a in range(start, N, _ROW_BLOCK):
                r = np.arange(a, min(a + _ROW_BLOCK, N))
                n = _visible(r, N, causal)
                P, _ = _softmax_rows(_scores(q[b, h, r], k[b, kv, :n], s, r, causal))
                dP = do[b, h, r] @ v[b, kv, :n].T
                dS = _softmax_vjp(P, dP, N)
                if full_q:
                    dQ[b, h, r] = s * (dS @ k[b, kv, :n])
                sel = np.nonzero(kr < n)[0]
                dV[b, kv, sel] += P[:, kr[sel]].T @ do[b, h, r]
                dK[b, kv, sel] += s * (dS[:, kr[sel]].T @ q[b, h, r])
    return dQ, dK, dV


def attention_ref(q, k, v, do, scale, causal):
    """Full forward and backward: (O, LSE, dQ, dK, dV), all float64."""
    O, LSE = attention_fwd_ref(q, k, v, scale, causal)
    dQ, dK, dV = attention_bwd_ref(q, k, v, do, scale, causal)
    return O, LSE, dQ, dK, dV
