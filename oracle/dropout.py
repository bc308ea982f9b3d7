"""Float64 CPU oracle for attention with dropout on the probabilities, and the
counter-based generator that draws its mask.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

What the pages fix, and what is read into them
----------------------------------------------
"FlashAttention 在昇腾NPU上到底快在哪" (section 二) says that dropout is fused into
the attention operator together with the softmax; "【词汇专栏】FlashAttention"
(section 5.1) shows PyTorch's fused attention taking a ``dropout_p`` argument.
Neither page gives the generator, the keep rule or the scaling.  Readings:

* Dropout acts on the normalised probabilities, with inverted scaling (the
  meaning of ``dropout_p`` in PyTorch's fused attention):

      P = row softmax of s Q K^T (causal mask as without dropout)
      O = (P * M / keep) V,       LSE_i = log sum_j exp(S_ij)   (no mask in it)

  M is a 0/1 keep mask and ``keep`` the probability that an element is kept,
  so E[O] is the attention without dropout.

* The randomness is Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): a bijection of a 128-bit
  counter under a 64-bit key, ten rounds of two 32x32->64-bit products with
  the multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl
  constants 0x9E3779B9 and 0xBB67AE85 between rounds.

* Each call covers a 4 x 4 block of the score matrix of one (batch, head):
  query rows 4a..4a+3, key columns 4c..4c+3, with

      counter = (c, a, b*H + h, offset),   key = (seed mod 2^32, seed >> 32)

  Output word r belongs to query 4a + r, and its byte e (little-endian) to key
  4c + e.  So every element gets 8 random bits of its own, and the mask
  depends only on (seed, offset, b, h, i, j): not on tiling or launch shape.

* Keep rule: with t = round(256 * p_drop), an element is kept when its byte is
  >= t.  The drop rate is t / 256 exactly and keep = (256 - t) / 256;
  0 <= t <= 255 (p_drop < 255.5/256).  A rate is thus quantised to 1/256.

* Backward: the chain rule through O = Z V with Z = P * M / keep:
  dV = Z^T dO, dZ = dO V^T, dP = dZ * M / keep, dS = softmax-Jacobian(P) dP,
  dQ = s dS K, dK = s dS^T Q.  (Written out in full here; the contraction
  rowsum(P * dP) = rowsum(dO * O) is a kernel's business, not the oracle's;
  the Jacobian is formed explicitly for short rows, as in the square oracle.)

Pins (``tests/test_oracle_dropout.py``): Philox against the generator's
published known-answer vectors; the 4 x 4 block map against element-by-element
calls; the byte and keep-rate statistics; p_drop = 0 against the square oracle;
LSE independent of the mask; E[O] over seeds against the attention without
dropout; the gradients against central finite differences with the mask held
fixed.
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_vjp

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with ten rounds.  counter: uint32 [..., 4]; key: uint32 [..., 2]
    (broadcast against counter).  Returns uint32 [..., 4]."""
    c = np.asarray(counter, dtype=np.uint64)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint64), c.shape[:-1] + (2,))
    x0, x1, x2, x3 = (c[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = np.uint64(_M0) * x0          # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def drop_threshold(p_drop):
    """Byte threshold t and keep probability for a requested drop rate."""
    t = int(np.floor(256.0 * float(p_drop) + 0.5))
    if not (0.0 <= p_drop) or t > 255:
        raise ValueError("p_drop must satisfy 0 <= p_drop and round(256 p_drop) <= 255")
    return t, (256 - t) / 256.0


def random_bytes(B, H, Nq, Nk, seed, offset, bh=None):
    """The 8 random bits of every score element: uint8 [B, H, Nq, Nk].  With
    ``bh`` (B = H = 1 only) the single head drawn is head b*H + h = bh of a
    larger tensor."""
    if bh is not None and (B, H) != (1, 1):
        raise ValueError("bh selects one head: B and H must be 1")
    seed = int(seed)
    key = np.array([seed & _MASK32, (seed >> 32) & _MASK32], dtype=np.uint32)
    na, nc = (Nq + 3) // 4, (Nk + 3) // 4
    a, c = np.meshgrid(np.arange(na), np.arange(nc), indexing="ij")
    out = np.empty((B, H, 4 * na, 4 * nc), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            head = b * H + h if bh is None else int(bh)
            ctr = np.stack([c, a, np.full_like(a, head), np.full_like(a, int(offset))], axis=-1)
            words = philox4x32_10(ctr.astype(np.uint32), key)       # [na, nc, 4]: word r -> query 4a+r
            by = words.view(np.uint8).reshape(na, nc, 4, 4)          # [a, c, r, e] (little-endian bytes)
            out[b, h] = by.transpose(0, 2, 1, 3).reshape(4 * na, 4 * nc)
    return out[:, :, :Nq, :Nk]


def keep_mask(B, H, Nq, Nk, p_drop, seed, offset, bh=None):
    """0/1 keep mask (float64) and the keep probability."""
    t, keep = drop_threshold(p_drop)
    return (random_bytes(B, H, Nq, Nk, seed, offset, bh) >= t).astype(np.float64), keep


def _setup(q, k, v, causal):
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or H % Hkv:
        raise ValueError("expected q [B,H,N,d], k/v [B,Hkv,N,d] with H a multiple of Hkv")
    return B, H, Hkv, N, d


def _probs(q, k, scale, causal):
    """P [B,H,N,N] and LSE [B,H,N], float64, with GQA head mapping."""
    B, H, N, _ = q.shape
    g = H // k.shape[1]
    kk = np.repeat(k, g, axis=1)
    S = scale * np.einsum("bhid,bhjd->bhij", q, kk)
    if causal:
        S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def attention_fwd_dropout_ref(q, k, v, scale, causal, p_drop, seed, offset, bh=None):
    """O [B,H,N,d] and LSE [B,H,N] of attention with dropout on P.  ``bh``: the
    inputs are one head (B = H = 1), head b*H + h = bh of a larger tensor."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, Hkv, N, d = _setup(q, k, v, causal)
    M, keep = keep_mask(B, H, N, N, p_drop, seed, offset, bh)
    P, lse = _probs(q, k, scale, causal)
    Z = P * M / keep
    O = np.einsum("bhij,bhjd->bhid", Z, np.repeat(v, H // Hkv, axis=1))
    return O, lse


def attention_bwd_dropout_ref(q, k, v, do, scale, causal, p_drop, seed, offset, bh=None):
    """dQ, dK, dV of sum(O * dO) for the dropout forward above (GQA: K/V
    gradients summed over the query heads of each group; ``bh`` as there)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, Hkv, N, d = _setup(q, k, v, causal)
    g = H // Hkv
    M, keep = keep_mask(B, H, N, N, p_drop, seed, offset, bh)
    P, _ = _probs(q, k, scale, causal)
    kk, vv = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    Z = P * M / keep
    dv_h = np.einsum("bhij,bhid->bhjd", Z, do)
    dZ = np.einsum("bhid,bhjd->bhij", do, vv)
    dP = dZ * M / keep
    dS = np.empty_like(P)
    for b in range(B):
        for h in range(H):
            dS[b, h] = _softmax_vjp(P[b, h], dP[b, h], N)
    dq = scale * np.einsum("bhij,bhjd->bhid", dS, kk)
    dk_h = scale * np.einsum("bhij,bhid->bhjd", dS, q)
    dk = dk_h.reshape(B, Hkv, g, N, d).sum(axis=2)
    dv = dv_h.reshape(B, Hkv, g, N, d).sum(axis=2)
    return dq, dk, dv


__all__ = ["philox4x32_10", "drop_threshold", "random_bytes", "keep_mask",
           "attention_fwd_dropout_ref", "attention_bwd_dropout_ref"]
