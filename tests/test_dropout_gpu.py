"""Parity of the dropout entry points (``fa_fwd_dropout`` and ``fa_bwd_dropout``,
through the C ABI) with the float64 dropout oracle of ``oracle/dropout.py``.

* The mask itself, bit for bit: with V = I (rows of the identity, d >= N), O's
  zero pattern is the keep mask on the visible scores; with dO = I, dV's zero
  pattern is its transpose.  This checks the generator, the 4 x 4 block map
  and the threshold in the forward and in the dK/dV kernel as integer work.
* A sweep of shapes over several tiles with ragged ends, both dtypes, both
  head sizes, GQA and MHA, causal and not, several rates, seeds and offsets,
  compared element by element on O, LSE, dQ, dK, dV with the bars of the
  square-attention tests (f32: 1e-5 * max(1, max |ref|); bf16: LSE 1e-3, O
  within max(1e-2, 1.05 u (attn(|V|) + |O|) + 1e-5), u = 2^-8, attn(|V|)
  being the oracle's dropout attention of |V|; dQ/dK/dV relative L2 2e-2).
* Twelve seeded random cases (shape, rate, seed, offset) compared the same way.
* Rate 0 runs the plain path; LSE does not depend on the mask.
* The benchmarked size (B=2, H=32, N=4096, d=128, causal, rate 0.1) run
  whole, two heads compared in full (O 1e-2, LSE 1e-3, gradients 2e-2).
"""
import numpy as np
import pytest

from oracle import attention_fwd_ref
from oracle.dropout import attention_bwd_dropout_ref, attention_fwd_dropout_ref, keep_mask
from tiled_attention_14_amd import fa, synth

from gpu_common import check, host64, say, to_device

pytestmark = pytest.mark.gpu


def _run(w, p, seed, offset, t=None):
    import torch
    inp = synth.make_inputs(w)
    t = to_device(inp) if t is None else t
    say(f"[dropout] {w.name} B={w.B} H={w.H} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} causal={w.causal} "
        f"p={p} seed={seed:#x} offset={offset}")
    o, lse = fa.forward_dropout(t["q"], t["k"], t["v"], p, seed, offset, w.scale, w.causal)
    dq, dk, dv = fa.backward_dropout(t["q"], t["k"], t["v"], o, t["do"], lse, p, seed, offset, w.scale, w.causal)
    torch.cuda.synchronize()
    return inp, {n: host64(x) for n, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}


def _refs(w, inp, p, seed, offset):
    q, k, v, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    O, L = attention_fwd_dropout_ref(q, k, v, w.scale, w.causal, p, seed, offset)
    dq, dk, dv = attention_bwd_dropout_ref(q, k, v, do, w.scale, w.causal, p, seed, offset)
    floor = None
    if w.dtype == "bf16":
        floor, _ = attention_fwd_dropout_ref(q, k, np.abs(v), w.scale, w.causal, p, seed, offset)
    return {"o": O, "lse": L, "dq": dq, "dk": dk, "dv": dv}, floor


@pytest.mark.parametrize("dt,d,N,causal", [("bf16", 128, 128, False), ("bf16", 64, 61, True),
                                           ("f32", 128, 100, True), ("f32", 64, 64, False)])
def test_mask_bit_exact(dt, d, N, causal):
    import torch
    B, H, p, seed, off = 2, 3, 0.3, 0xDEADBEEF12345, 11
    w = synth.Workload("mask_exact", B, H, H, N, d, dt, causal, seed=9000 + N + d)
    inp = synth.make_inputs(w)
    t = to_device(inp)
    eye = torch.zeros((B, H, N, d), dtype=t["v"].dtype, device="cuda")
    idx = torch.arange(N, device="cuda")
    eye[:, :, idx, idx] = 1
    t["v"] = eye.contiguous()
    t["do"] = eye.clone()
    _, got = _run(w, p, seed, off, t)
    M, _ = keep_mask(B, H, N, N, p, seed, off)
    vis = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    want = (M > 0) & vis
    o_nz = got["o"][..., :N] != 0
    dv_nz = np.swapaxes(got["dv"][..., :N], -1, -2) != 0   # dV[j, i] = Z[i, j]
    say(f"[dropout]   kept {want.mean():.3f}; O pattern mismatches {int((o_nz != want).sum())}, "
        f"dV pattern mismatches {int((dv_nz != want).sum())}")
    assert np.array_equal(o_nz, want)
    assert np.array_equal(dv_nz, want)
    assert not np.any(got["o"][..., N:])


@pytest.mark.parametrize("which", ["dk", "dq"])
@pytest.mark.parametrize("dt,d,N,causal", [("bf16", 128, 128, True), ("bf16", 64, 61, False),
                                           ("f32", 128, 100, False), ("f32", 64, 64, True)])
def test_mask_element_by_element_in_dk_and_dq(which, dt, d, N, causal):
    """The mask as the dS wave of the dK/dV kernel and the dQ kernel apply it.
    With Q = one-hot rows (Q[i] = e_i), dK[j, i] = scale * dS[i, j]; with K =
    one-hot rows, dQ[i, j] = scale * dS[i, j]: every element of the checked
    gradient is one element of dS = P (dP M / keep - D).  Each must match the
    oracle's (correct-mask) value within a rounding bound, and flipping the
    mask bit of an element would move its value by P dP / keep, which is
    required to exceed twice that bound for most visible elements, so a
    single misplaced mask bit fails the test."""
    import torch
    B, H, p, seed, off = 1, 2, 0.3, 0xBADC0FFEE, 5
    w = synth.Workload("mask_dkdq", B, H, H, N, d, dt, causal, seed=9300 + N + d)
    inp = synth.make_inputs(w)
    onehot = np.zeros((B, H, N, d), dtype=np.float32)
    onehot[:, :, np.arange(N), np.arange(N)] = 1.0
    vals = dict(inp.vals)
    vals["q" if which == "dk" else "k"] = onehot
    bits = None if inp.bits is None else {n: synth.bf16_round_bits(x) for n, x in vals.items()}
    inp = synth.Inputs(w, vals, bits)
    _, got = _run(w, p, seed, off, to_device(inp))
    ref, _ = _refs(w, inp, p, seed, off)
    g, r = got[which][..., :N], ref[which][..., :N]
    if which == "dk":  # dK[j, i] = scale dS[i, j]: put both in (i, j) order
        g, r = np.swapaxes(g, -1, -2), np.swapaxes(r, -1, -2)
    # Size of the change a flipped mask bit would cause: scale P dP / keep.
    q, k, v, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    S = w.scale * q @ np.swapaxes(k, -1, -2)
    vis = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    S = np.where(vis, S, -np.inf)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    keep = 1.0 - round(256 * p) / 256
    flip = np.abs(w.scale * P * (do @ np.swapaxes(v, -1, -2)) / keep)
    scale_ref = float(np.max(np.abs(r)))
    # Rounding bound per element: dS and the output rounded to bf16 (or fp32
    # noise), plus the absolute error of dP M / keep - D, which matters where
    # the two terms cancel: D = rowsum(dO * O) formed from the stored (bf16) O,
    # and dP accumulated in fp32 over d products.
    u_o = 2.0 ** -8 if dt == "bf16" else 2.0 ** -23
    dD = u_o * np.sum(np.abs(do * ref["o"]), axis=-1, keepdims=True)
    dDP = 2.0 ** -16 * (np.abs(do) @ np.swapaxes(np.abs(v), -1, -2)) / keep
    tol = w.scale * P * (dD + dDP) + ((1e-2 * np.abs(r) + 1e-5 * scale_ref) if dt == "bf16"
                                      else (1e-5 * np.abs(r) + 1e-7 * scale_ref))
    err = np.abs(g - r)
    sensitive = vis & (flip > 2 * tol)
    say(f"[dropout]   {which}: max err/tol {float(np.max(np.where(vis, err / tol, 0))):.3f}, "
        f"elements where a flipped bit would show: {sensitive.sum()} of {vis.sum() * B * H} visible")
    assert np.all(err <= tol), f"{which}: {int((err > tol).sum())} elements off the correct-mask value"
    assert sensitive.sum() >= 0.8 * vis.sum() * B * H


SWEEP = [
    # dtype, d, causal, B, H, Hkv, N, p, seed, offset
    ("bf16", 128, True, 1, 4, 2, 300, 0.1, 1, 0),
    ("bf16", 128, False, 2, 2, 1, 129, 0.5, 2 ** 40 + 3, 9),
    ("bf16", 64, True, 1, 8, 1, 777, 0.2, 77, 1),
    ("bf16", 64, False, 1, 4, 4, 1000, 0.3, 5, 2 ** 32 - 1),
    ("bf16", 128, True, 1, 2, 2, 1, 0.5, 6, 0),     # 1/keep = 2: O = 2 V exactly, so dS = 0 stays ~0
    ("f32", 128, True, 1, 4, 2, 300, 0.25, 7, 3),
    ("f32", 64, False, 2, 3, 3, 200, 0.6, 8, 4),
    ("f32", 64, True, 1, 2, 1, 65, 0.9, 9, 5),
]


@pytest.mark.parametrize("dt,d,causal,B,H,Hkv,N,p,seed,offset", SWEEP, ids=lambda x: str(x))
def test_dropout_sweep(dt, d, causal, B, H, Hkv, N, p, seed, offset):
    w = synth.Workload("dropout_sweep", B, H, Hkv, N, d, dt, causal, seed=9100 + N + d + H + causal)
    inp, got = _run(w, p, seed, offset)
    ref, floor = _refs(w, inp, p, seed, offset)
    check(w, got, ref, "dropout", f32_scaled=True, o_floor=floor)


def test_rate_zero_is_the_plain_path_and_lse_ignores_the_mask():
    import torch
    w = synth.Workload("dropout_zero", 1, 4, 2, 257, 128, "bf16", True, seed=9200)
    inp = synth.make_inputs(w)
    t = to_device(inp)
    o0, l0 = fa.forward(t["q"], t["k"], t["v"], w.scale, True)
    o1, l1 = fa.forward_dropout(t["q"], t["k"], t["v"], 0.0, 123, 0, w.scale, True)
    o2, l2 = fa.forward_dropout(t["q"], t["k"], t["v"], 0.5, 123, 0, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert float((l0 - l2).abs().max()) <= 1e-6
    assert not torch.equal(o0, o2)
    _, L = attention_fwd_ref(inp.f64("q"), inp.f64("k"), inp.f64("v"), w.scale, True)
    assert float(np.max(np.abs(host64(l2) - L))) <= 1e-3


@pytest.mark.parametrize("b,h", [(0, 5), (1, 31)])
def test_dropout_at_the_benchmarked_size(b, h):
    # The benchmark's dropout leg: the 7B-shaped causal layer (B=2, H=32,
    # N=4096, d=128, bf16), rate 0.1, seed 0x5EED, offset 0, run whole; two
    # heads compared in full with the bars of the named bf16 workloads.
    w = synth.WORKLOADS[synth.HEADLINE]
    assert (w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.causal) == (2, 32, 32, 4096, 128, "bf16", True)
    p, seed, off = 0.1, 0x5EED, 0
    inp, got = _run(w, p, seed, off)
    sl = (slice(b, b + 1), slice(h, h + 1))
    q, k, v, do = (inp.f64(n)[sl] for n in ("q", "k", "v", "do"))
    O, L = attention_fwd_dropout_ref(q, k, v, w.scale, True, p, seed, off, bh=b * w.H + h)
    dq, dk, dv = attention_bwd_dropout_ref(q, k, v, do, w.scale, True, p, seed, off, bh=b * w.H + h)
    one = synth.Workload(f"{w.name}_head_{b}_{h}", 1, 1, 1, w.N, w.d, "bf16", True)
    check(one, {n: x[sl] for n, x in got.items()}, {"o": O, "lse": L, "dq": dq, "dk": dk, "dv": dv}, "dropout-full")


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 3]))
        out.append((str(rng.choice(["bf16", "f32"])), int(rng.choice([64, 128])), bool(rng.integers(2)),
                    int(rng.integers(1, 3)), hkv * int(rng.choice([1, 2, 4])), hkv, int(rng.integers(1, 400)),
                    float(rng.integers(1, 250)) / 256, int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 32))))
    return out


@pytest.mark.parametrize("dt,d,causal,B,H,Hkv,N,p,seed,offset", _random_cases(12, 9300), ids=lambda x: str(x))
def test_dropout_random_shapes(dt, d, causal, B, H, Hkv, N, p, seed, offset):
    # Seeded random shapes, rates, seeds and offsets, compared like the sweep.
    w = synth.Workload("dropout_random", B, H, Hkv, N, d, dt, causal, seed=9400 + N + d + H)
    inp, got = _run(w, p, seed, offset)
    ref, floor = _refs(w, inp, p, seed, offset)
    check(w, got, ref, "dropout-random", f32_scaled=True, o_floor=floor)
