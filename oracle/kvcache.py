"""Float64 CPU oracle for attention over a key/value cache: Nq query rows against
Nk >= 1 keys, key ranges ("splits") and the merge of per-range results.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

What it computes
----------------
For every batch b and query head h, with KV head ``kv = h // (H/Hkv)``,
Q[b,h] of Nq rows and K[b,kv], V[b,kv] of Nk rows:

    S = s * Q[b,h] @ K[b,kv]^T                        (Nq x Nk, materialised)
    causal: S[i, j] = -inf for j > i + (Nk - Nq)      (bottom-right alignment)
    P = row softmax of S ;  O = P @ V ;  LSE_i = log sum_j exp(S_ij)

The causal mask is aligned at the bottom right: the last query row sees every
key, as when a new chunk of Nq tokens attends to a cache holding Nk tokens of
which the chunk is the tail.  Nq == Nk gives the square mask of the training
shapes; Nq == 1 is decoding one token.  The pages name the key/value cache
reuse of inference ("FlashAttention 在昇腾NPU上到底快在哪", section 七) but fix no
alignment; bottom-right is the reading under which causal decoding sees the
whole cache.  Causal calls need Nq <= Nk so that every row sees a key.

A split is the same attention restricted to the keys [k0, k1): its O is
normalised over that range alone and its LSE is the log-sum-exp over that
range (-inf, with O = 0, for a row that sees none of those keys).  Merging
splits is the rescaling step of the incremental softmax ("FlashAttention 在昇腾
NPU上到底快在哪", section 三、增量 Softmax): with LSE = log sum_s exp(LSE_s),

    O = sum_s exp(LSE_s - LSE) O_s

which recovers the attention over the union of the ranges exactly.  The
multi-device "AllReduce of attention results" in "【词汇专栏】FlashAttention"
(section 3.2) becomes exact only with these weights.

Pins (``tests/test_oracle_kv.py``): the square special case against the
independently pinned square oracle, PyTorch's float64 SDPA with an explicit
mask, closed forms for constant scores, decode against the unmasked case, a
hand-derived two-split merge, and the merge of every split against the
unsplit result.
"""
from __future__ import annotations

import numpy as np


def _check(q, k, v, causal):
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,H,Nq,d], k/v [B,Hkv,Nk,d]")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or H % k.shape[1]:
        raise ValueError("shape mismatch between q and k/v")
    Nk = k.shape[2]
    if causal and Nq > Nk:
        raise ValueError("causal attention with bottom-right alignment needs Nq <= Nk")
    return B, H, k.shape[1], Nq, Nk, d


def _range_attention(qh, kh, vh, s, causal, Nq, k0, k1):
    """O, LSE of the rows of one head over the keys [k0, k1)."""
    Nk = kh.shape[0]
    keys = np.arange(k0, k1)
    S = s * (qh @ kh[k0:k1].T)
    if causal:
        last = np.arange(Nq) + (Nk - Nq)          # last visible key of each row
        S[keys[None, :] > last[:, None]] = -np.inf
    O = np.zeros((Nq, qh.shape[1]))
    LSE = np.full(Nq, -np.inf)
    m = S.max(axis=1) if S.shape[1] else np.full(Nq, -np.inf)
    seen = np.isfinite(m)
    if np.any(seen):
        E = np.exp(S[seen] - m[seen, None])
        Z = E.sum(axis=1)
        O[seen] = (E / Z[:, None]) @ vh[k0:k1]
        LSE[seen] = m[seen] + np.log(Z)
    return O, LSE


def attention_fwd_kv_ref(q, k, v, scale, causal, k0=0, k1=None):
    """O [B,H,Nq,d] and LSE [B,H,Nq] (float64) of attention over the keys [k0, k1)
    (all keys by default), with the bottom-right causal mask when ``causal``."""
    B, H, Hkv, Nq, Nk, d = _check(q, k, v, causal)
    k1 = Nk if k1 is None else k1
    if not 0 <= k0 <= k1 <= Nk:
        raise ValueError("key range out of bounds")
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = float(scale)
    g = H // Hkv
    O = np.empty((B, H, Nq, d)); LSE = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = _range_attention(q[b, h], k[b, h // g], v[b, h // g], s, causal, Nq, k0, k1)
    return O, LSE


def merge_ref(o_parts, lse_parts):
    """Merges per-range results: o_parts [S, ..., d], lse_parts [S, ...] (float64)
    into (O, LSE).  Rows with LSE_s = -inf in every range get O = 0, LSE = -inf."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    fin = np.isfinite(m)
    ms = np.where(fin, m, 0.0)
    w = np.exp(lse_parts - ms[None])                      # exp(-inf) = 0 for empty ranges
    Z = w.sum(axis=0)
    LSE = np.where(fin, ms + np.log(np.where(fin, Z, 1.0)), -np.inf)
    O = np.einsum("s...,s...d->...d", w, o_parts) / np.where(fin, Z, 1.0)[..., None]
    return O, LSE
