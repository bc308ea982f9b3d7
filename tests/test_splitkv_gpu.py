"""Parity of the key/value-cache forward (``fa_fwd_splitkv``) and of the merge
(``fa_merge``) with the float64 oracle of ``oracle/kvcache.py``.

Shapes cover decoding (Nq = 1) with and without GQA packing, chunks of several
query rows against longer caches (bottom-right causal mask), Nq > Nk without
the mask, several row blocks, ragged key counts, key ranges that hold a
single key or none visible to a row, and range counts above the number of
tiles (capped by the library).  The two decode workloads run at full size and
are compared on every row.

Tolerances: float32, max |gpu - ref| <= 1e-5 * max(1, max |ref|) for O and
LSE; bfloat16, LSE max abs <= 1e-3 and O per element within
max(1e-2, 1.05 u (attn(|V|) + |O|) + 1e-5), u = 2^-8, the bound of the
square-attention tests for P and O rounded to bf16 (the decode variant, at
most 32 rows per KV head, rounds P to bf16; the general kernel to fp16).
"""
import numpy as np
import pytest

from oracle.kvcache import attention_fwd_kv_ref, merge_ref
from tiled_attention_14_amd import fa, synth

from gpu_common import say

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def _dev(inp, name):
    import torch
    if inp.bits is not None:
        return torch.from_numpy(inp.bits[name].view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(inp.vals[name]).to("cuda")


def _run(w, nsplit):
    import torch
    inp = synth.make_kv_inputs(w)
    q, k, v = (_dev(inp, n) for n in ("q", "k", "v"))
    say(f"[splitkv] {w.name} B={w.B} H={w.H} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} "
        f"causal={w.causal} nsplit={nsplit}")
    o, lse = fa.forward_kv(q, k, v, w.scale, w.causal, nsplit)
    torch.cuda.synchronize()
    return inp, o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(w, inp, o, lse):
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    O, L = attention_fwd_kv_ref(q, k, v, w.scale, w.causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo, el = float(np.max(np.abs(o - O))), float(np.max(np.abs(lse - L)))
    say(f"[splitkv]   O maxabs {eo:.3e}  LSE maxabs {el:.3e}")
    if w.dtype == "f32":
        assert eo <= 1e-5 * max(1.0, float(np.max(np.abs(O))))
        assert el <= 1e-5 * max(1.0, float(np.max(np.abs(L))))
    else:
        floor, _ = attention_fwd_kv_ref(q, k, np.abs(v), w.scale, w.causal)
        bound = np.maximum(1e-2, 1.05 * U * (floor + np.abs(O)) + 1e-5)
        assert np.all(np.abs(o - O) <= bound), f"O above the bf16 bound by {float(np.max(np.abs(o - O) - bound)):.3e}"
        assert el <= 1e-3


CASES = [
    # dtype, d, causal, B, H, Hkv, Nq, Nk, nsplit
    ("bf16", 128, True, 2, 8, 1, 1, 1, 0),        # a single key
    ("bf16", 128, True, 1, 8, 2, 1, 300, 0),      # decode, 4 heads per KV head
    ("bf16", 128, True, 3, 4, 4, 1, 1000, 3),     # decode, MHA, 3 ranges
    ("bf16", 64, True, 1, 16, 2, 5, 777, 7),      # 5 tokens x 8 heads = 40 rows per KV head
    ("bf16", 64, False, 2, 4, 2, 37, 200, 2),
    ("bf16", 128, False, 1, 2, 1, 150, 40, 1),    # more queries than keys, no mask
    ("bf16", 128, True, 1, 4, 2, 129, 129, 0),    # square mask
    ("bf16", 128, True, 1, 2, 2, 200, 1000, 4),   # two row blocks; causal cuts the ranges
    ("bf16", 64, True, 1, 64, 8, 1, 64, 1),       # exactly one tile
    ("bf16", 128, True, 1, 4, 1, 3, 300, 100),    # more ranges requested than tiles
    ("f32", 64, True, 1, 4, 2, 3, 500, 0),
    ("f32", 128, False, 2, 2, 1, 70, 130, 3),
    ("f32", 128, True, 1, 8, 8, 1, 65, 2),        # the second range holds one key
    ("f32", 64, True, 2, 3, 3, 200, 200, 3),      # rows 0-127 see no key of the range [128, 200)
]


@pytest.mark.parametrize("dt,d,causal,B,H,Hkv,Nq,Nk,nsplit", CASES, ids=lambda x: str(x))
def test_splitkv_small(dt, d, causal, B, H, Hkv, Nq, Nk, nsplit):
    w = synth.KvWorkload("kv_sweep", B, H, Hkv, Nq, Nk, d, dt, causal, seed=7000 + Nq + Nk + d + H + nsplit)
    inp, o, lse = _run(w, nsplit)
    _check(w, inp, o, lse)


def test_splitkv_range_count_does_not_change_the_result_beyond_rounding():
    w = synth.KvWorkload("kv_ranges", 1, 8, 2, 2, 2000, 128, "f32", True, seed=7100)
    _, o1, l1 = _run(w, 1)
    _, o8, l8 = _run(w, 8)
    assert float(np.max(np.abs(o1 - o8))) <= 2e-6 and float(np.max(np.abs(l1 - l8))) <= 2e-6


@pytest.mark.parametrize("name", sorted(synth.KV_WORKLOADS))
def test_decode_workloads_full(name):
    w = synth.KV_WORKLOADS[name]
    inp, o, lse = _run(w, 0)
    _check(w, inp, o, lse)


def test_decode_long_cache_peaked_rows():
    # The long-sequence distribution (Q and K with std 2: logits with std 4,
    # peaked rows) against a 65536-token cache, held to the flat O bar of the
    # named bf16 workloads (1e-2 max abs) besides the bf16 rounding bound.
    w = synth.KvWorkload("decode_long_std2", 1, 8, 8, 1, 65536, 128, "bf16", True, seed=7300, qk_std=2.0)
    inp, o, lse = _run(w, 0)
    _check(w, inp, o, lse)
    O, _ = attention_fwd_kv_ref(inp.f64("q"), inp.f64("k"), inp.f64("v"), w.scale, True)
    assert float(np.max(np.abs(o - O))) <= 1e-2


@pytest.mark.parametrize("dt,d", [("f32", 64), ("bf16", 128)])
def test_merge_of_oracle_ranges(dt, d):
    import torch
    rng = np.random.default_rng(7200 + d)
    B, H, Hkv, Nq, Nk = 2, 4, 2, 9, 300
    q = rng.standard_normal((B, H, Nq, d)); k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    cuts = [0, 64, 65, 200, 300]
    parts = [attention_fwd_kv_ref(q, k, v, 0.1, True, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    op = np.stack([p[0] for p in parts]).astype(np.float32)
    lp = np.stack([p[1] for p in parts]).astype(np.float32)
    rows = B * H * Nq
    say(f"[merge] {dt} d={d} ranges={len(parts)} rows={rows}")
    op_d = torch.from_numpy(np.ascontiguousarray(op.reshape(len(parts), rows, d))).to("cuda")
    lp_d = torch.from_numpy(np.ascontiguousarray(lp.reshape(len(parts), rows))).to("cuda")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    o = torch.empty((rows, d), dtype=tdt, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    st = fa.fa_merge(op_d, lp_d, o, lse, len(parts), rows, d, fa.FA_BF16 if dt == "bf16" else fa.FA_F32)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    O, L = merge_ref(op.astype(np.float64), lp.astype(np.float64))
    Of, Lf = attention_fwd_kv_ref(q, k, v, 0.1, True)
    np.testing.assert_allclose(O, Of.reshape(O.shape), atol=1e-5)   # float32 partials, exact merge
    got = o.float().cpu().numpy().astype(np.float64)
    tol_o = 1e-5 if dt == "f32" else None
    if tol_o is not None:
        assert float(np.max(np.abs(got - O.reshape(rows, d)))) <= tol_o
    else:
        assert np.all(np.abs(got - O.reshape(rows, d)) <= U * np.abs(O.reshape(rows, d)) + 1e-6)
    assert float(np.max(np.abs(lse.cpu().numpy() - L.reshape(rows)))) <= 1e-5
