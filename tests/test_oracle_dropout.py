"""Pins of the dropout oracle (``oracle/dropout.py``) to facts outside it: the
generator's published known-answer vectors, the element map written out call by
call, the statistics of the random bytes, the reduction to the attention
without dropout at rate 0, the unbiasedness of the inverted scaling, and
central finite differences of its forward for its backward."""
import json
import os

import numpy as np
import pytest

from oracle import attention_bwd_ref, attention_fwd_ref
from oracle.dropout import (attention_bwd_dropout_ref, attention_fwd_dropout_ref,
                            drop_threshold, keep_mask, philox4x32_10, random_bytes)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def _hex(xs):
    return np.array([int(x, 16) for x in xs], dtype=np.uint32)


def test_philox_known_answers():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        got = philox4x32_10(_hex(c["counter"]), _hex(c["key"]))
        assert [f"{x:08x}" for x in got] == c["out"]
    # Vectorised over a batch of counters, every row as if alone.
    ctr = np.stack([_hex(c["counter"]) for c in cases])
    for i, c in enumerate(cases):
        assert np.array_equal(philox4x32_10(ctr[i:i + 1], _hex(c["key"]))[0], _hex(c["out"]))


@pytest.mark.parametrize("B,H,Nq,Nk,seed,offset", [(2, 3, 13, 10, 0x123456789ABCDEF, 7), (1, 1, 4, 4, 0, 0),
                                                   (1, 2, 1, 9, 2 ** 64 - 1, 2 ** 32 - 1)])
def test_element_map_call_by_call(B, H, Nq, Nk, seed, offset):
    by = random_bytes(B, H, Nq, Nk, seed, offset)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                for j in range(Nk):
                    w = philox4x32_10(np.array([j // 4, i // 4, b * H + h, offset], dtype=np.uint32), key)
                    assert by[b, h, i, j] == (int(w[i % 4]) >> (8 * (j % 4))) & 0xFF


def test_byte_statistics_and_keep_rate():
    by = random_bytes(1, 2, 256, 512, seed=99, offset=3).astype(np.int64)
    n = by.size
    counts = np.bincount(by.ravel(), minlength=256)
    chi2 = float(((counts - n / 256) ** 2 / (n / 256)).sum())
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)           # 255 degrees of freedom, ~6 sigma
    # Neighbouring elements are not correlated (same word, next byte; next row).
    x = (by - 127.5) / 73.9
    assert abs(float(np.mean(x[..., :-1] * x[..., 1:]))) < 6 / np.sqrt(n)
    assert abs(float(np.mean(x[:, :, :-1] * x[:, :, 1:]))) < 6 / np.sqrt(n)
    # Heads and offsets draw different bytes.
    assert np.mean(by[0, 0] == by[0, 1]) < 0.01
    assert np.mean(random_bytes(1, 1, 64, 64, 99, 3) == random_bytes(1, 1, 64, 64, 99, 4)) < 0.01
    for p in (0.1, 0.3, 0.5, 0.9):
        t, keep = drop_threshold(p)
        M, keep2 = keep_mask(1, 2, 256, 512, p, 99, 3)
        assert keep == keep2 == (256 - t) / 256
        assert abs(float(M.mean()) - keep) < 6 * np.sqrt(keep * (1 - keep) / M.size)


def test_threshold_rule():
    assert drop_threshold(0.0) == (0, 1.0)
    assert drop_threshold(0.1)[0] == 26 and drop_threshold(0.5)[0] == 128
    assert drop_threshold(255 / 256)[0] == 255
    for bad in (-0.1, 0.999, 1.0):
        with pytest.raises(ValueError):
            drop_threshold(bad)
    assert keep_mask(1, 1, 8, 8, 0.0, 5, 0)[0].min() == 1.0


def _inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, H, N, d)))


@pytest.mark.parametrize("causal", [False, True])
def test_rate_zero_is_plain_attention(causal):
    q, k, v, do = _inputs(2, 4, 2, 11, 8, 1)
    O, L = attention_fwd_dropout_ref(q, k, v, 0.3, causal, 0.0, 1234, 5)
    O0, L0 = attention_fwd_ref(q, k, v, 0.3, causal)
    np.testing.assert_allclose(O, O0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, L0, rtol=0, atol=1e-13)
    g = attention_bwd_dropout_ref(q, k, v, do, 0.3, causal, 0.0, 1234, 5)
    g0 = attention_bwd_ref(q, k, v, do, 0.3, causal)
    for a, b in zip(g, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_lse_does_not_see_the_mask():
    q, k, v, _ = _inputs(1, 2, 1, 9, 4, 2)
    _, L0 = attention_fwd_ref(q, k, v, 0.5, True)
    for p, seed in ((0.2, 1), (0.7, 2)):
        _, L = attention_fwd_dropout_ref(q, k, v, 0.5, True, p, seed, 0)
        np.testing.assert_allclose(L, L0, rtol=0, atol=1e-13)


def test_inverted_scaling_is_unbiased():
    # E over seeds of O equals the attention without dropout; checked against
    # the sample's own standard error.
    q, k, v, _ = _inputs(1, 1, 1, 6, 3, 3)
    O0, _ = attention_fwd_ref(q, k, v, 0.7, False)
    draws = np.stack([attention_fwd_dropout_ref(q, k, v, 0.7, False, 0.4, s, 0)[0] for s in range(1500)])
    mean, se = draws.mean(axis=0), draws.std(axis=0) / np.sqrt(len(draws))
    assert np.all(np.abs(mean - O0) <= 5 * se + 1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_against_finite_differences(causal):
    B, H, Hkv, N, d, s, p, seed, off = 1, 2, 1, 6, 3, 0.6, 0.35, 77, 1
    q, k, v, do = _inputs(B, H, Hkv, N, d, 4)
    M, _ = keep_mask(B, H, N, N, p, seed, off)
    assert 0 < M.mean() < 1                              # the mask drops something and keeps something

    def loss(q_, k_, v_):
        return float(np.sum(attention_fwd_dropout_ref(q_, k_, v_, s, causal, p, seed, off)[0] * do))

    dq, dk, dv = attention_bwd_dropout_ref(q, k, v, do, s, causal, p, seed, off)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        num = np.zeros_like(args[which])
        for idx in np.ndindex(*args[which].shape):
            plus = [a.copy() for a in args]; minus = [a.copy() for a in args]
            plus[which][idx] += h; minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7)


def test_single_head_draw_is_that_head_of_the_full_draw():
    full = random_bytes(2, 3, 9, 14, 0xABCDEF, 4)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(random_bytes(1, 1, 9, 14, 0xABCDEF, 4, bh=b * 3 + h)[0, 0], full[b, h])
    q, k, v, do = _inputs(2, 3, 3, 9, 4, 6)
    O, L = attention_fwd_dropout_ref(q, k, v, 0.4, True, 0.3, 0xABCDEF, 4)
    g = attention_bwd_dropout_ref(q, k, v, do, 0.4, True, 0.3, 0xABCDEF, 4)
    b, h = 1, 2
    sl = (slice(b, b + 1), slice(h, h + 1))
    O1, L1 = attention_fwd_dropout_ref(q[sl], k[sl], v[sl], 0.4, True, 0.3, 0xABCDEF, 4, bh=b * 3 + h)
    g1 = attention_bwd_dropout_ref(q[sl], k[sl], v[sl], do[sl], 0.4, True, 0.3, 0xABCDEF, 4, bh=b * 3 + h)
    np.testing.assert_array_equal(O1[0, 0], O[b, h])
    np.testing.assert_array_equal(L1[0, 0], L[b, h])
    for x1, x in zip(g1, g):
        np.testing.assert_allclose(x1[0, 0], x[b, h], rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        random_bytes(2, 1, 4, 4, 0, 0, bh=1)
