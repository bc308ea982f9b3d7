"""Pins of the key/value-cache oracle (Nq x Nk attention, key ranges, merge).

None of these re-types the oracle's formulas: they compare it with the square
oracle (itself pinned in test_oracle.py), with PyTorch's float64 SDPA given an
explicit mask, with closed forms and with a hand-derived merge.
"""
import math

import numpy as np
import pytest

from oracle import attention_fwd_ref
from oracle.kvcache import attention_fwd_kv_ref, merge_ref


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_equals_square_oracle(causal):
    q, k, v = _rand((2, 4, 37, 16), 1), _rand((2, 2, 37, 16), 2), _rand((2, 2, 37, 16), 3)
    O, L = attention_fwd_kv_ref(q, k, v, 0.3, causal)
    O2, L2 = attention_fwd_ref(q, k, v, 0.3, causal)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk,causal", [(5, 23, True), (1, 40, True), (7, 7, True), (9, 30, False), (30, 9, False)])
def test_against_torch_sdpa_with_bottom_right_mask(Nq, Nk, causal):
    torch = pytest.importorskip("torch")
    B, H, Hkv, d, s = 1, 6, 3, 8, 0.4
    q, k, v = _rand((B, H, Nq, d), 4), _rand((B, Hkv, Nk, d), 5), _rand((B, Hkv, Nk, d), 6)
    O, L = attention_fwd_kv_ref(q, k, v, s, causal)
    g = H // Hkv
    kt = torch.from_numpy(np.repeat(k, g, axis=1))
    vt = torch.from_numpy(np.repeat(v, g, axis=1))
    qt = torch.from_numpy(q)
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=s)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    # LSE from the library's own logsumexp over the masked scores.
    S = s * torch.einsum("bhid,bhjd->bhij", qt, kt)
    if causal:
        S = S.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_constant_scores_closed_form():
    # K = 0: every visible key scores 0, so O is the mean of the visible V rows
    # and LSE = log(number of visible keys) = log(i + Nk - Nq + 1).
    Nq, Nk = 6, 11
    q = _rand((1, 2, Nq, 4), 7)
    k = np.zeros((1, 1, Nk, 4))
    v = _rand((1, 1, Nk, 4), 8)
    O, L = attention_fwd_kv_ref(q, k, v, 0.5, True)
    for i in range(Nq):
        n = i + Nk - Nq + 1
        np.testing.assert_allclose(O[0, :, i], np.broadcast_to(v[0, 0, :n].mean(axis=0), (2, 4)), atol=1e-14)
        np.testing.assert_allclose(L[0, :, i], math.log(n), atol=1e-14)


def test_decode_row_sees_the_whole_cache():
    q, k, v = _rand((3, 4, 1, 16), 9), _rand((3, 4, 50, 16), 10), _rand((3, 4, 50, 16), 11)
    Oc, Lc = attention_fwd_kv_ref(q, k, v, 0.25, True)
    On, Ln = attention_fwd_kv_ref(q, k, v, 0.25, False)
    np.testing.assert_array_equal(Oc, On)
    np.testing.assert_array_equal(Lc, Ln)


def test_merge_hand_derived():
    # Two ranges with LSE 0 and log 3 carry weights 1/4 and 3/4; the merged
    # LSE is log(1 + 3) = log 4.
    a = np.array([1.0, -2.0, 0.5]); b = np.array([3.0, 2.0, -1.5])
    O, L = merge_ref(np.stack([a, b]), np.array([0.0, math.log(3.0)]))
    np.testing.assert_allclose(O, 0.25 * a + 0.75 * b, atol=1e-15)
    np.testing.assert_allclose(L, math.log(4.0), atol=1e-15)
    # A range that saw no key (LSE -inf) contributes nothing.
    O2, L2 = merge_ref(np.stack([a, b, 9 * b]), np.array([0.0, math.log(3.0), -np.inf]))
    np.testing.assert_allclose(O2, O, atol=1e-15)
    np.testing.assert_allclose(L2, L, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_key_ranges_equals_unsplit(causal):
    Nq, Nk = 9, 70
    q, k, v = _rand((2, 4, Nq, 8), 12), _rand((2, 2, Nk, 8), 13), _rand((2, 2, Nk, 8), 14)
    cuts = [0, 16, 17, 40, 64, 70]
    parts = [attention_fwd_kv_ref(q, k, v, 0.35, causal, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    O, L = merge_ref(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    Of, Lf = attention_fwd_kv_ref(q, k, v, 0.35, causal)
    np.testing.assert_allclose(O, Of, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lf, rtol=0, atol=1e-13)


def test_range_with_no_visible_key():
    # Causal, Nq = Nk = 4: row 0 sees only key 0, so the range [2, 4) is empty for rows 0 and 1.
    q, k, v = _rand((1, 1, 4, 4), 15), _rand((1, 1, 4, 4), 16), _rand((1, 1, 4, 4), 17)
    O, L = attention_fwd_kv_ref(q, k, v, 1.0, True, 2, 4)
    assert np.all(O[0, 0, :2] == 0) and np.all(np.isneginf(L[0, 0, :2]))
    assert np.all(np.isfinite(L[0, 0, 2:]))


def test_causal_needs_nq_at_most_nk():
    with pytest.raises(ValueError):
        attention_fwd_kv_ref(np.zeros((1, 1, 5, 4)), np.zeros((1, 1, 4, 4)), np.zeros((1, 1, 4, 4)), 1.0, True)
