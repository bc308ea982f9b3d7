"""fa_bwd_noalloc (the backward pass with its workspace in the library's fixed
device scratch, for callers that cannot allocate) against fa_bwd with a
caller workspace: the same kernels on the same inputs, so the results must be
identical bit for bit.  Two calls in a row, the second with smaller sizes, so
that the second runs on scratch the first left behind; one GQA shape whose
group is sliced (float32 partial dK/dV in the scratch)."""
import pytest

from tiled_attention_14_amd import fa, synth

from gpu_common import run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def _noalloc_bwd(w, t, o, lse):
    import torch
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ft = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    st = fa.fa_bwd_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, w.B, w.H, w.Hkv, w.N, w.d,
                           w.scale, w.causal, ft)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("first,second", [
    (synth.Workload("noalloc_a", 2, 32, 32, 4096, 128, "bf16", True, seed=31),
     synth.Workload("noalloc_b", 1, 4, 2, 777, 128, "bf16", True, seed=32)),
    (synth.Workload("noalloc_c", 1, 16, 2, 2048, 64, "bf16", False, seed=33),   # sliced GQA: partials
     synth.Workload("noalloc_d", 1, 2, 1, 300, 64, "f32", True, seed=34)),
])
def test_noalloc_matches_fa_bwd_twice(first, second):
    import torch
    for w in (first, second):
        say(f"[noalloc] {w.name} B={w.B} H={w.H} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
        t = to_device(synth.make_inputs(w))
        ref = run_gpu(w, t)
        dq, dk, dv = _noalloc_bwd(w, t, ref["o"], ref["lse"])
        for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert torch.equal(x, ref[name]), f"{w.name}: {name} differs from fa_bwd"


def test_noalloc_too_large_enqueues_nothing():
    import torch
    w = synth.Workload("noalloc_big", 1, 4, 4, 1024, 128, "bf16", True, seed=35)
    t = to_device(synth.make_inputs(w))
    o = torch.zeros_like(t["q"])
    lse = torch.zeros((1, 4, 1024), dtype=torch.float32, device="cuda")
    dq = torch.full_like(t["q"], 3.0)
    # B = 64 * 32 heads of 4096 rows: shapes the pointers do not cover, rejected before any launch
    st = fa.fa_bwd_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dq, dq, 64, 32, 32, 4096, 128,
                           w.scale, True, fa.FA_BF16)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_TOO_LARGE
    assert bool(torch.all(dq == 3.0))
