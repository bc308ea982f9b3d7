"""Properties of the HIP path on the GPU beyond element-wise parity with the
oracle: the stated input domain of the bf16 forward, buffer bounds, bitwise
determinism, the GQA head mapping and invariance under a shift of the keys.

* V at the edge of the bf16 forward's domain (|v| <= 65280, where the fp16
  conversion of V is still exact) against the oracle, through fa_fwd, fa_bwd
  and the general key/value-cache kernel;
* canaries: every output and the workspace sit inside larger buffers filled
  with a marker pattern; nothing outside the documented extent may change;
* determinism: the backward has no atomics, so two runs on the same inputs
  give identical bits in all five outputs;
* GQA equals multi-head attention with K/V repeated per query head
  (repeat_interleave; "FlashAttention V2深度解析", 对比 table, GQA/MQA rows):
  O, LSE and dQ bit for bit, dK/dV as the sum over each group;
* shifting every key row by one vector c leaves P unchanged, so O, dQ, dK, dV
  are unchanged and LSE moves by scale * q_i . c (the shift-invariance of
  softmax that the max subtraction of the incremental softmax relies on,
  "FlashAttention 在昇腾NPU上到底快在哪", section 三).
"""
import numpy as np
import pytest

from oracle import attention_fwd_ref, attention_ref
from oracle.kvcache import attention_fwd_kv_ref
from tiled_attention_14_amd import fa, synth

from gpu_common import check, host64, o_bound, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

VMAX = 65280.0  # largest bfloat16 below fp16's overflow threshold


def _bf16_inputs(inp, v_vals):
    """Inputs with V replaced by v_vals (already bf16-exact float32 values)."""
    bits = dict(inp.bits)
    vals = dict(inp.vals)
    bits["v"] = synth.bf16_round_bits(v_vals)
    vals["v"] = synth.bf16_bits_to_f32(bits["v"])
    assert np.array_equal(vals["v"], v_vals)
    return synth.Inputs(inp.w, vals, bits)


def _large_v(inp, rng):
    v = inp.vals["v"] * np.float32(16384.0)  # a power of two: still bf16-exact
    v = np.clip(v, -VMAX, VMAX)
    flat = v.reshape(-1)
    idx = rng.choice(flat.size, 8, replace=False)
    flat[idx[:4]] = VMAX
    flat[idx[4:]] = -VMAX
    return v


@pytest.mark.parametrize("causal,d,heads", [(True, 128, (4, 2)), (False, 64, (2, 2))])
def test_v_at_the_fp16_limit(causal, d, heads):
    H, Hkv = heads
    w = synth.Workload("v_limit", 1, H, Hkv, 333, d, "bf16", causal, seed=911 + d)
    rng = np.random.default_rng(912)
    inp = synth.make_inputs(w)
    inp = _bf16_inputs(inp, _large_v(inp, rng))
    assert float(np.max(np.abs(inp.vals["v"]))) == VMAX
    g = run_gpu(w, to_device(inp))
    gpu = {n: host64(t) for n, t in g.items()}
    q, k, v, do = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do")
    O, LSE, dQ, dK, dV = attention_ref(q, k, v, do, w.scale, causal)
    floor, _ = attention_fwd_ref(q, k, np.abs(v), w.scale, causal)
    check(w, gpu, {"o": O, "lse": LSE, "dq": dQ, "dk": dK, "dv": dV}, "|v|<=65280", o_floor=floor)


def test_v_at_the_fp16_limit_cache_kernel():
    """The key/value-cache kernel for more than 32 query rows per KV head also
    runs P V in fp16."""
    import torch
    w = synth.KvWorkload("v_limit_kv", 1, 4, 2, 200, 700, 128, "bf16", True, seed=913)
    inp = synth.make_kv_inputs(w)
    rng = np.random.default_rng(914)
    inp = _bf16_inputs(inp, _large_v(inp, rng))
    t = {n: torch.from_numpy(inp.bits[n].view(np.int16)).view(torch.bfloat16).to("cuda") for n in ("q", "k", "v")}
    o, lse = fa.forward_kv(t["q"], t["k"], t["v"], w.scale, True, 3)
    torch.cuda.synchronize()
    o, lse = host64(o), host64(lse)
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    O, L = attention_fwd_kv_ref(q, k, v, w.scale, True)
    floor, _ = attention_fwd_kv_ref(q, k, np.abs(v), w.scale, True)
    assert np.all(np.isfinite(o))
    err = np.abs(o - O)
    say(f"[v-limit kv] O maxabs {err.max():.3e} (max |O| {np.abs(O).max():.1f}), LSE maxabs {np.abs(lse - L).max():.2e}")
    assert np.all(err <= o_bound(floor, O))
    assert np.max(np.abs(lse - L)) <= 1e-3


# ---------------------------------------------------------------- canaries
CANARY_BF16 = 0x7FA5           # a NaN pattern no kernel writes
CANARY_F32 = 0x7FC0DEAD
PAD = 4096                      # elements of canary before and after each buffer


def _padded(shape, dtype):
    import torch
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        buf = torch.full((n + 2 * PAD,), CANARY_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        buf = torch.full((n + 2 * PAD,), CANARY_F32, dtype=torch.int32, device="cuda").view(torch.float32)
    return buf, buf[PAD:PAD + n].view(shape)


def _canary_intact(buf, name):
    import torch
    raw = buf.view(torch.int16 if buf.dtype == torch.bfloat16 else torch.int32)
    want = CANARY_BF16 if buf.dtype == torch.bfloat16 else CANARY_F32
    head, tail = raw[:PAD], raw[-PAD:]
    assert bool(torch.all(head == want)) and bool(torch.all(tail == want)), f"{name}: canary overwritten"


@pytest.mark.parametrize("dt,d,causal,N,heads", [
    ("bf16", 128, True, 777, (2, 4, 2)),    # sliced GQA group: float32 partials in the workspace
    ("bf16", 64, False, 1000, (1, 8, 1)),
    ("bf16", 64, True, 333, (1, 4, 2)),     # four-wave workgroups at d = 64, ragged causal tail
    ("bf16", 128, False, 129, (1, 3, 3)),
    ("f32", 128, True, 300, (1, 4, 2)),
    ("f32", 64, False, 97, (2, 2, 1)),
])
def test_canaries_around_outputs_and_workspace(dt, d, causal, N, heads):
    import torch
    B, H, Hkv = heads
    w = synth.Workload("canary", B, H, Hkv, N, d, dt, causal, seed=6000 + N)
    t = to_device(synth.make_inputs(w))
    tdt = t["q"].dtype
    ft = fa.FA_BF16 if dt == "bf16" else fa.FA_F32
    bo, o = _padded((B, H, N, d), tdt)
    bl, lse = _padded((B, H, N), torch.float32)
    bq, dq = _padded((B, H, N, d), tdt)
    bk, dk = _padded((B, Hkv, N, d), tdt)
    bv, dv = _padded((B, Hkv, N, d), tdt)
    n = fa.fa_bwd_workspace_size(B, H, Hkv, N, d, ft)
    wbuf = torch.full((n + 2048 + 256,), 0x5A, dtype=torch.uint8, device="cuda")
    addr = (wbuf.data_ptr() + 1024 + 255) // 256 * 256  # 256-byte aligned, >= 1 KiB of canary on each side
    lo = addr - wbuf.data_ptr()
    sh = (B, H, Hkv, N, d)
    assert fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, *sh, w.scale, causal, ft) == fa.FA_OK
    assert fa.fa_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, *sh, w.scale, causal, ft,
                     addr, n) == fa.FA_OK
    torch.cuda.synchronize()
    say(f"[canary] {dt} d={d} causal={causal} N={N} heads={heads}: workspace {n} B")
    for b, name in ((bo, "o"), (bl, "lse"), (bq, "dq"), (bk, "dk"), (bv, "dv")):
        _canary_intact(b, name)
    assert bool(torch.all(wbuf[:lo] == 0x5A)) and bool(torch.all(wbuf[lo + n:] == 0x5A)), "workspace canary"
    # and what was written is the right result
    ref = {"o": host64(o), "lse": host64(lse), "dq": host64(dq), "dk": host64(dk), "dv": host64(dv)}
    plain = {n_: host64(x) for n_, x in run_gpu(w, t).items()}
    for n_ in ref:
        assert np.array_equal(ref[n_], plain[n_]), n_


# ---------------------------------------------------------------- determinism
@pytest.mark.parametrize("dt,d,causal,N,heads", [
    ("bf16", 128, True, 2048, (1, 8, 2)),
    ("bf16", 128, True, 1000, (1, 8, 2)),   # ragged, sliced GQA group
    ("bf16", 64, False, 1500, (2, 4, 4)),
    ("f32", 128, True, 700, (1, 4, 1)),
])
def test_run_twice_bitwise(dt, d, causal, N, heads):
    import torch
    B, H, Hkv = heads
    w = synth.Workload("determinism", B, H, Hkv, N, d, dt, causal, seed=7000 + N)
    t = to_device(synth.make_inputs(w))
    a = run_gpu(w, t)
    b = run_gpu(w, t)
    say(f"[determinism] {dt} d={d} causal={causal} N={N} heads={heads}")
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), f"{n} differs between two runs"


# ---------------------------------------------------------------- GQA == repeated K/V
@pytest.mark.parametrize("dt,d,causal,N,heads", [
    ("bf16", 128, True, 1000, (8, 2)),
    ("bf16", 64, False, 600, (8, 1)),
    ("bf16", 128, True, 2048, (16, 2)),     # wide group: the dK/dV work is sliced
    ("f32", 64, True, 300, (4, 2)),
])
def test_gqa_equals_repeated_kv(dt, d, causal, N, heads):
    import torch
    H, Hkv = heads
    g = H // Hkv
    w = synth.Workload("gqa", 1, H, Hkv, N, d, dt, causal, seed=8000 + N)
    t = to_device(synth.make_inputs(w))
    a = run_gpu(w, t)
    rep = dict(t)
    rep["k"] = t["k"].repeat_interleave(g, dim=1).contiguous()
    rep["v"] = t["v"].repeat_interleave(g, dim=1).contiguous()
    b = run_gpu(w.with_(Hkv=H), rep)
    say(f"[gqa=mha] {dt} d={d} causal={causal} N={N} H={H} Hkv={Hkv}")
    for n in ("o", "lse", "dq"):
        assert torch.equal(a[n], b[n]), f"{n}: GQA differs from repeated K/V"
    for n in ("dk", "dv"):
        ga = host64(a[n])
        gb = host64(b[n]).reshape(1, Hkv, g, N, d).sum(axis=2)
        rel = np.linalg.norm(ga - gb) / np.linalg.norm(gb)
        say(f"[gqa=mha]   {n}: rel L2 {rel:.2e}")
        assert rel <= (1e-6 if dt == "f32" else 1e-2)


# ---------------------------------------------------------------- key shift
@pytest.mark.parametrize("dt,d,causal", [("bf16", 128, True), ("bf16", 64, False), ("f32", 128, False)])
def test_key_shift_invariance(dt, d, causal):
    """K and c on a grid of 1/16 with |K + c| < 16, so K + c is exact in bf16
    and the GPU sees the shifted keys without rounding."""
    import torch
    w = synth.Workload("kshift", 1, 4, 2, 500, d, dt, causal, seed=9000 + d)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(9001)
    kq = np.clip(np.round(inp.vals["k"] * 16.0) / 16.0, -12.0, 12.0).astype(np.float32)
    c = (rng.integers(-32, 33, size=d) / 16.0).astype(np.float32)
    ks = (kq + c).astype(np.float32)
    assert np.max(np.abs(ks)) < 16.0
    t = to_device(inp)
    mk = (lambda x: torch.from_numpy(synth.bf16_round_bits(x).view(np.int16)).view(torch.bfloat16).to("cuda")) \
        if dt == "bf16" else (lambda x: torch.from_numpy(x).to("cuda"))
    t0 = dict(t); t0["k"] = mk(kq)
    t1 = dict(t); t1["k"] = mk(ks)
    a = run_gpu(w, t0)
    b = run_gpu(w, t1)
    q = host64(t["q"])
    shift = w.scale * np.einsum("bhnd,d->bhn", q, c.astype(np.float64))
    dl = np.abs(host64(b["lse"]) - host64(a["lse"]) - shift).max()
    do_ = np.abs(host64(b["o"]) - host64(a["o"])).max()
    tol_o, tol_l = (1e-5, 1e-5) if dt == "f32" else (1e-2, 1e-3)
    say(f"[k-shift] {dt} d={d} causal={causal}: O maxabs {do_:.2e}, LSE - shift maxabs {dl:.2e}")
    assert do_ <= tol_o and dl <= tol_l
    for n in ("dq", "dk", "dv"):
        x, y = host64(a[n]), host64(b[n])
        rel = np.linalg.norm(x - y) / np.linalg.norm(x)
        say(f"[k-shift]   {n}: rel L2 {rel:.2e}")
        assert rel <= (1e-5 if dt == "f32" else 2e-2)
