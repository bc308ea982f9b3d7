"""Parity of the fp8 forward (``fa_fwd_fp8``) with the float64 oracle applied to
the values the codes stand for (code * tensor scale).

Tolerances follow from the arithmetic: the products of e4m3 codes are exact in
float32, so S and the log-sum-exp carry only float32 rounding (LSE max abs
<= 1e-3).  P is rounded to e4m3 for the P V product (relative error at most
u8 = 2^-4 per probability) and O is rounded to bf16 (u = 2^-8), so per element
|O - O_ref| <= 1.05 (u8 attn(|V|) + u |O|) + 1e-5, with attn(|V|) the oracle's
attention of |V|.
"""
import numpy as np
import pytest

from oracle import attention_fwd_ref
from tiled_attention_14_amd import fa, synth

from gpu_common import say

pytestmark = pytest.mark.gpu

U8, U = 2.0 ** -4, 2.0 ** -8


def _run(B, H, Hkv, N, causal, seed, qk_std=1.0):
    import torch
    inp = synth.make_fp8_inputs(B, H, Hkv, N, 128, seed, qk_std=qk_std)
    t = {n: torch.from_numpy(inp.codes[n]).to("cuda") for n in ("q", "k", "v")}
    o = torch.empty((B, H, N, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1.0) / np.sqrt(np.float32(128)))
    say(f"[fp8] B={B} H={H} Hkv={Hkv} N={N} causal={causal} seed={seed}")
    st = fa.fa_fwd_fp8(t["q"], t["k"], t["v"], o, lse, B, H, Hkv, N, 128, scale,
                       inp.scales["q"], inp.scales["k"], inp.scales["v"], causal)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    return inp, scale, o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(inp, scale, causal, o, lse, rows=None):
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    O, L = attention_fwd_ref(q, k, v, scale, causal, rows=rows)
    floor, _ = attention_fwd_ref(q, k, np.abs(v), scale, causal, rows=rows)
    if rows is not None:
        bi = np.arange(o.shape[0])[:, None, None]
        hi = np.arange(o.shape[1])[None, :, None]
        o, lse = o[bi, hi, rows], lse[bi, hi, rows]
    bound = 1.05 * (U8 * floor + U * np.abs(O)) + 1e-5
    err = np.abs(o - O)
    say(f"[fp8]   O maxabs {err.max():.3e} (bound max {bound.max():.3e}), rel L2 "
        f"{np.linalg.norm(o - O) / np.linalg.norm(O):.3e}, LSE maxabs {np.abs(lse - L).max():.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.all(err <= bound), f"O above the fp8 bound by {float((err - bound).max()):.3e}"
    assert float(np.abs(lse - L).max()) <= 1e-3


CASES = [(1, 1, 1, 1), (1, 2, 1, 64), (2, 4, 2, 129), (1, 4, 4, 300), (1, 2, 2, 777)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N", CASES, ids=lambda x: str(x))
def test_fp8_small(B, H, Hkv, N, causal):
    inp, scale, o, lse = _run(B, H, Hkv, N, causal, seed=8000 + N + H + causal)
    _check(inp, scale, causal, o, lse)


def test_fp8_llama2_7b_shape_every_row():
    B, H, N = 2, 32, 4096
    inp, scale, o, lse = _run(B, H, H, N, True, seed=8100)
    _check(inp, scale, True, o, lse)


def test_fp8_llama2_70b_gqa_shape_sampled_rows():
    B, H, Hkv, N = 1, 64, 8, 8192
    inp, scale, o, lse = _run(B, H, Hkv, N, True, seed=8200)
    rows = synth.sample_rows(N, 256, 8201, B * H).reshape(B, H, -1)
    _check(inp, scale, True, o, lse, rows=rows)


def test_fp8_long_sequence_sampled_rows():
    # The long-sequence distribution (Q and K with std 2: peaked rows) over
    # 65536 keys, where the running max moves most.
    B, H, N = 1, 8, 65536
    inp, scale, o, lse = _run(B, H, H, N, True, seed=8300, qk_std=2.0)
    rows = synth.sample_rows(N, 256, 8301, B * H).reshape(B, H, -1)
    _check(inp, scale, True, o, lse, rows=rows)
