#!/usr/bin/env python3
"""Benchmark of exact attention forward + backward on one MI355X (gfx950).

One step is one pass of the whole path on one batch of synthetic input that is
already resident in HBM: ``fa_fwd`` followed by the backward phases of
``fa_bwd`` (``fa_bwd_dq``, which also forms the row terms D and lse * log2 e,
then ``fa_bwd_dkdv``), all on one stream.  W untimed warm-up steps; then K
steps with HIP events between the kernels, which bring the shader clock to
its loaded level (that takes some tens of milliseconds of work after an idle
gap); then exactly K steps bracketed by ``torch.cuda.synchronize()``, whose
wall time gives ``value``; then K more steps with events for the per-kernel
breakdown.  The secondary legs (other workloads, preprocess, decode, fp8,
dropout) each run back to back for a quarter second before their timed calls,
for the same reason.  Prints ONE JSON line on stdout.

Throughput uses the algorithmic flop count (what the method must compute; the
masked half under the causal mask is work it avoids):
    F_fwd = 4 B H N^2 d (x 1/2 if causal),  F_bwd = 2.5 F_fwd,  F_tot = 3.5 F_fwd.

HIP events recorded between the kernels on the launch stream give each
kernel's average duration; the dominant kernel's achieved rate is reported
against the MI355X dense bf16 MFMA peak (2.5 PFLOP/s published).  The CPU
oracle is timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 (matrix and vector)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SOURCES = {"fa_fwd": ["tiled_attention_14_amd/csrc/fa_fwd.hip", "tiled_attention_14_amd/csrc/fa_device.h"],
                  "fa_bwd_dkdv": ["tiled_attention_14_amd/csrc/fa_bwd.hip", "tiled_attention_14_amd/csrc/fa_device.h"],
                  "fa_bwd_dq": ["tiled_attention_14_amd/csrc/fa_bwd.hip", "tiled_attention_14_amd/csrc/fa_device.h"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def settle(fn, seconds=0.25):
    """Runs fn back to back for about `seconds` of wall time (synchronising
    every few calls) so that a leg is timed at the loaded shader clock: after
    the host-side input generation between legs the clock starts low and takes
    some tens of milliseconds of sustained work to come up."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def flops(w):
    f_fwd = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return f_fwd, 2.5 * f_fwd, 3.5 * f_fwd


def hbm_bytes(w):
    """Algorithmic HBM bytes of one fwd + bwd pass: every input read once and
    every output written once (forward: Q, K, V in, O and LSE out; backward:
    Q, K, V, O, dO, LSE in, dQ, dK, dV out)."""
    e = 2 if w.dtype == "bf16" else 4
    q = w.B * w.H * w.N * w.d * e
    kv = w.B * w.Hkv * w.N * w.d * e
    rows = w.B * w.H * w.N * 4
    return (2 * q + 2 * kv + rows) + (4 * q + 4 * kv + rows)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for_current_kernel(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary of the
    headline workload, or None when it is missing or the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_llama2_7b_causal_n4096_d128.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, inp, budget_s=12.0):
    """Times the float64 oracle (unchanged) on whole (batch, head) slices of the
    workload, as many rounds of `cores` heads as fit in about `budget_s`."""
    import numpy as np
    from oracle import attention_bwd_ref, attention_fwd_ref
    cores = len(os.sched_getaffinity(0))
    g = w.H // w.Hkv
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_total, f_total = 0, 0.0, 0.0
    q, k, v, do = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do")
    while done < len(heads):
        batch = heads[done:done + cores]
        qs = np.stack([q[b, h] for b, h in batch])[None]
        ks = np.stack([k[b, h // g] for b, h in batch])[None]
        vs = np.stack([v[b, h // g] for b, h in batch])[None]
        ds = np.stack([do[b, h] for b, h in batch])[None]
        t0 = time.perf_counter()
        attention_fwd_ref(qs, ks, vs, w.scale, w.causal)
        attention_bwd_ref(qs, ks, vs, ds, w.scale, w.causal)
        t_total += time.perf_counter() - t0
        f_total += 3.5 * 4.0 * len(batch) * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
        done += len(batch)
        if t_total >= budget_s:
            break
    return {"value": f_total / t_total / 1e12, "unit": "TFLOP/s", "cores": min(cores, done),
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} (batch, head) slices, full fwd+bwd in float64 "
                      f"({t_total:.1f} s on the host CPU)"}


def decode_leg(dev, calls=50, warmup=10):
    """Times fa_fwd_splitkv (key-range kernel + merge) on the decode workloads
    with HIP events on the launch stream.  Decoding is bound by reading the
    cache: the rate is algorithmic bytes (q, k, v read; o, lse written) per
    call against the HBM peak; the float32 partials are overhead, not credited."""
    import numpy as np
    import torch
    from tiled_attention_14_amd import fa, synth
    res = []
    for name in sorted(synth.KV_WORKLOADS):
        w = synth.KV_WORKLOADS[name]
        inp = synth.make_kv_inputs(w)
        t = {n: torch.from_numpy(inp.bits[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v")}
        del inp
        o = torch.empty_like(t["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        n = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, fa.FA_BF16, 0)
        buf = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        addr = (buf.data_ptr() + 255) // 256 * 256
        stream = torch.cuda.current_stream()

        def call():
            st = fa.fa_fwd_splitkv(t["q"], t["k"], t["v"], o, lse, w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.scale,
                                   w.causal, fa.FA_BF16, 0, addr, n, stream)
            if st != fa.FA_OK:
                raise RuntimeError("fa_fwd_splitkv failed")

        for _ in range(warmup):
            call()
        settle(call)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(calls):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        nbytes = 2 * (2 * w.B * w.H * w.Nq * w.d + 2 * w.B * w.Hkv * w.Nk * w.d) + 4 * w.B * w.H * w.Nq
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"[bench] decode {name}: {us:.1f} us per call, {gbs:.0f} GB/s")
        res.append({"workload": name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                    "causal": w.causal, "us_per_call": round(us, 2), "bytes": nbytes, "bound": "hbm",
                    "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)})
        del t, o, lse, buf
    return res


def fp8_leg(dev, calls=50, warmup=10):
    """Times fa_fwd_fp8 on the headline shape (e4m3 Q, K, V with per-tensor
    scales, bf16 O) with HIP events on the launch stream; the rate is the
    forward's algorithmic flops against the dense fp8 matrix-core peak."""
    import numpy as np
    import torch
    from tiled_attention_14_amd import fa, synth
    w = synth.WORKLOADS[synth.HEADLINE]
    inp = synth.make_fp8_inputs(w.B, w.H, w.Hkv, w.N, w.d, seed=w.seed)
    t = {n: torch.from_numpy(inp.codes[n]).to(dev) for n in ("q", "k", "v")}
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        st = fa.fa_fwd_fp8(t["q"], t["k"], t["v"], o, lse, w.B, w.H, w.Hkv, w.N, w.d, w.scale,
                           inp.scales["q"], inp.scales["k"], inp.scales["v"], w.causal, stream)
        if st != fa.FA_OK:
            raise RuntimeError("fa_fwd_fp8 failed")

    for _ in range(warmup):
        call()
    settle(call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(calls):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    f_fwd = flops(w)[0]
    tf = f_fwd / (ms * 1e-3) / 1e12
    log(f"[bench] fp8 forward {w.name}: {ms:.4f} ms, {tf:.1f} TFLOP/s")
    return {"workload": w.name, "dtype": "e4m3 in, bf16 out", "ms": round(ms, 4), "tflops": round(tf, 2),
            "bound": "mfma", "peak": PEAK_FP8_TFLOPS, "frac": round(tf / PEAK_FP8_TFLOPS, 4)}


def dropout_leg(dev, calls=20, warmup=5, p_drop=0.1):
    """Times fa_fwd_dropout + fa_bwd_dropout (rate p_drop, one seed and offset)
    on the headline shape with HIP events on the launch stream; the rate is the
    step's algorithmic matrix flops (those of attention without dropout)
    against the dense bf16 peak, beside the plain step's."""
    import torch
    from tiled_attention_14_amd import fa, synth
    w = synth.WORKLOADS[synth.HEADLINE]
    inp = synth.make_inputs(w)
    t = {n: torch.from_numpy(inp.bits[n].view("int16")).view(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do")}
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ws_buf, addr, nbytes = fa.workspace(w.B, w.H, w.Hkv, w.N, w.d, fa.FA_BF16, dev)  # ws_buf owns the memory
    stream = torch.cuda.current_stream()
    args = (w.B, w.H, w.Hkv, w.N, w.d, w.scale, w.causal, p_drop, 0x5EED, 0)

    def fwd():
        if fa.fa_fwd_dropout(t["q"], t["k"], t["v"], o, lse, *args, fa.FA_BF16, stream) != fa.FA_OK:
            raise RuntimeError("fa_fwd_dropout failed")

    def bwd():
        if fa.fa_bwd_dropout(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, *args, fa.FA_BF16, addr, nbytes,
                             stream) != fa.FA_OK:
            raise RuntimeError("fa_bwd_dropout failed")

    def timed(fn):
        for _ in range(warmup):
            fn()
        settle(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls

    ms_f, ms_b = timed(fwd), timed(bwd)
    f_all = flops(w)[2]
    tf = f_all / ((ms_f + ms_b) * 1e-3) / 1e12
    log(f"[bench] dropout p={p_drop} {w.name}: fwd {ms_f:.4f} ms, bwd {ms_b:.4f} ms, {tf:.1f} TFLOP/s")
    return {"workload": w.name, "p_drop": p_drop, "fwd_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
            "tflops": round(tf, 2), "bound": "mfma", "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def flops_of(w):
    return flops(w)


def host_info():
    """CPU model, BLAS library numpy uses, and the host threads the oracle may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name')} {b.get('version')}".strip()
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "threads": len(os.sched_getaffinity(0))}


def sample_sclk():
    """Current shader clock in MHz as rocm-smi reports it, or None."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    try:
        r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
    except Exception:
        return None
    for card in d.values():
        if isinstance(card, dict):
            for key, val in card.items():
                if "sclk" in key.lower():
                    txt = str(val).lower().replace("(", " ").replace(")", " ").replace("mhz", " ")
                    for tok in txt.split():
                        try:
                            return float(tok)
                        except ValueError:
                            continue
    return None


class Layer:
    """Device buffers of one workload and its step: fa_fwd, fa_bwd_dq, fa_bwd_dkdv."""

    def __init__(self, w, dev):
        import numpy as np
        import torch
        from tiled_attention_14_amd import fa, synth
        self.w, self.fa = w, fa
        inp = synth.make_inputs(w)
        self.inp = inp

        def up(name):
            if inp.bits is not None:
                return torch.from_numpy(inp.bits[name].view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(inp.vals[name]).to(dev)

        self.q, self.k, self.v, self.do = up("q"), up("k"), up("v"), up("do")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.dt = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
        self.ws_buf, self.ws, self.ws_n = fa.workspace(w.B, w.H, w.Hkv, w.N, w.d, self.dt, dev)
        self.stream = torch.cuda.current_stream()
        self.sargs = (w.B, w.H, w.Hkv, w.N, w.d)

    def step(self, ev=None):
        fa, w, s = self.fa, self.w, self.stream
        if ev is not None: ev[0].record(s)
        st = fa.fa_fwd(self.q, self.k, self.v, self.o, self.lse, *self.sargs, w.scale, w.causal, self.dt, s)
        if ev is not None: ev[1].record(s)
        st |= fa.fa_bwd_dq(self.q, self.k, self.v, self.o, self.do, self.lse, self.dq, *self.sargs, w.scale,
                           w.causal, self.dt, self.ws, self.ws_n, s)
        if ev is not None: ev[2].record(s)
        st |= fa.fa_bwd_dkdv(self.q, self.k, self.v, self.do, self.dk, self.dv, *self.sargs, w.scale, w.causal,
                             self.dt, self.ws, self.ws_n, s)
        if ev is not None: ev[3].record(s)
        if st != fa.FA_OK:
            raise RuntimeError("attention call failed")

    def kernel_times(self, steps):
        """Average per-kernel milliseconds over `steps` steps (HIP events on the launch stream)."""
        import numpy as np
        import torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        names = ["fa_fwd", "fa_bwd_dq", "fa_bwd_dkdv"]
        return {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}


def other_workloads(dev, names, steps=3, warmup=2):
    """fwd / bwd / fwd+bwd TFLOP/s of the other named workloads (HIP events)."""
    import torch
    from tiled_attention_14_amd import synth
    res = []
    for name in names:
        w = synth.WORKLOADS[name]
        L = Layer(w, dev)
        del L.inp
        for _ in range(warmup):
            L.step()
        settle(L.step)
        per = L.kernel_times(steps if w.N >= 32768 else 4 * steps)
        f_fwd, f_bwd, f_tot = flops(w)
        t_fwd, t_bwd = per["fa_fwd"], per["fa_bwd_dq"] + per["fa_bwd_dkdv"]
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        r = {"workload": name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d, "dtype": w.dtype,
             "causal": w.causal, "fwd_ms": round(t_fwd, 4), "bwd_ms": round(t_bwd, 4),
             "fwd_tflops": round(f_fwd / (t_fwd * 1e-3) / 1e12, 2),
             "bwd_tflops": round(f_bwd / (t_bwd * 1e-3) / 1e12, 2),
             "tflops": round(f_tot / ((t_fwd + t_bwd) * 1e-3) / 1e12, 2),
             "kernel_ms": {n: round(t, 4) for n, t in per.items()}}
        r["frac"] = round(r["tflops"] / peak, 4)
        # Intensity of the whole pass: far above the ridge point (peak flop/s
        # over 8 TB/s, about 313 flop/B for bf16), so even the shortest named
        # sequence is bound by the matrix cores and the softmax, not by HBM.
        r["hbm_bytes"] = hbm_bytes(w)
        r["flop_per_byte"] = round(f_tot / r["hbm_bytes"], 1)
        r["achieved_gbs"] = round(r["hbm_bytes"] / ((t_fwd + t_bwd) * 1e-3) / 1e9, 1)
        log(f"[bench] {name}: fwd {t_fwd:.4f} ms ({r['fwd_tflops']} TFLOP/s), bwd {t_bwd:.4f} ms "
            f"({r['bwd_tflops']} TFLOP/s)")
        res.append(r)
        del L
        torch.cuda.empty_cache()
    return res


def preprocess_leg(L, calls=50, warmup=5):
    """fa_bwd_preprocess alone on the headline shape (bound by HBM): it reads O,
    dO and LSE and writes -D and lse * log2 e.  fa_bwd forms the same values
    inside the dQ kernel; the standalone phase is measured for its bandwidth."""
    import torch
    fa, w = L.fa, L.w

    def call():
        if fa.fa_bwd_preprocess(L.o, L.do, L.lse, *L.sargs, L.dt, L.ws, L.ws_n, L.stream) != fa.FA_OK:
            raise RuntimeError("fa_bwd_preprocess failed")

    for _ in range(warmup):
        call()
    settle(call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(L.stream)
    for _ in range(calls):
        call()
    e1.record(L.stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    el = 2 if w.dtype == "bf16" else 4
    nbytes = 2 * w.B * w.H * w.N * w.d * el + 3 * 4 * w.B * w.H * w.N
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] preprocess {w.name}: {us:.1f} us, {gbs:.0f} GB/s")
    return {"workload": w.name, "us": round(us, 2), "bytes": nbytes, "bound": "hbm", "achieved_gbs": round(gbs, 1),
            "peak_gbs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}


def clock_leg(L, seconds=2.0):
    """Shader clock sampled by rocm-smi while the headline step runs back to back."""
    import threading
    import torch
    box = {}
    t = threading.Thread(target=lambda: box.setdefault("mhz", sample_sclk()))
    L.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t.start()
    n = 0
    while t.is_alive() or time.perf_counter() - t0 < 0.3:
        for _ in range(20):
            L.step()
        torch.cuda.synchronize()
        n += 20
        if time.perf_counter() - t0 > seconds + 20:
            break
    t.join(timeout=30)
    log(f"[bench] shader clock under load: {box.get('mhz')} MHz ({n} steps while sampling)")
    return box.get("mhz")


def main():
    from tiled_attention_14_amd import synth
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=synth.HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the extra legs (other workloads, decode, fp8, dropout, preprocess, clock)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the attention path here is single-GPU "
              f"(--gpus {args.gpus}, WORLD_SIZE={world} requested); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    w = synth.WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    L = Layer(w, dev)
    for _ in range(args.warmup):
        L.step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warm-up steps done")

    # K steps with events between the kernels: they bring the shader clock to
    # its loaded level before the timed region (their times are logged, not used).
    settle = L.kernel_times(args.steps)
    log("[bench] settling pass, kernel averages (ms): " + ", ".join(f"{n}={t:.4f}" for n, t in settle.items()))

    # Timed region: exactly K steps, no events (wall clock between synchronizations).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] {args.steps} timed steps: {wall * 1e3 / args.steps:.3f} ms/step")

    # Per-kernel durations: K more steps with events between the kernels,
    # recorded on the stream the kernels are launched on.
    per = L.kernel_times(args.steps)
    log("[bench] kernel averages (ms): " + ", ".join(f"{n}={t:.4f}" for n, t in per.items()))

    f_fwd, f_bwd, f_tot = flops(w)
    ms = wall * 1e3 / args.steps
    value = f_tot / (ms * 1e-3) / 1e12
    t_fwd = per["fa_fwd"]
    t_bwd = per["fa_bwd_dq"] + per["fa_bwd_dkdv"]
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # Algorithmic flops per kernel, in units of one N x N x d product (F_fwd / 2):
    # the forward does 2 (S, P V); the backward's 5 (S, dP, dV, dK, dQ) split into
    # 4 in the dK/dV kernel and 1 in the dQ kernel, whose recomputation of S and
    # dP is not credited.  Executed products: fwd 2, dK/dV 4, dQ 3.
    unit = f_fwd / 2
    algo = {"fa_fwd": 2 * unit, "fa_bwd_dkdv": 4 * unit, "fa_bwd_dq": 1 * unit}
    executed = {"fa_fwd": 2 * unit, "fa_bwd_dkdv": 4 * unit, "fa_bwd_dq": 3 * unit}
    dom = max(algo, key=lambda n: per[n])
    achieved = algo[dom] / (per[dom] * 1e-3) / 1e12
    traffic = traffic_for_current_kernel(dom) if w.name == synth.HEADLINE else None

    out = {
        "metric": "attention fwd+bwd TFLOP/s (bf16, causal) and % of MFMA bf16 peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q, K, V, dO; bf16-rounded)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "fwd_tflops": round(f_fwd / (t_fwd * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (t_bwd * 1e-3) / 1e12, 2),
        "fwd_ms": round(t_fwd, 4),
        "bwd_ms": round(t_bwd, 4),
        "kernel_ms": {n: round(t, 4) for n, t in per.items()},
        "kernel_mfma_tflops_executed": {n: round(f / (per[n] * 1e-3) / 1e12, 2) for n, f in executed.items()},
        "timing": "W warm-up steps; K steps with events (settling, not used); K wall-timed steps (value); "
                  "K steps with events (kernel_ms)",
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic},
    }
    if not args.no_decode:
        out["sclk_mhz_under_load"] = clock_leg(L)
        out["bwd_preprocess"] = preprocess_leg(L)
        others = [n for n in ("mha_bf16_n2048_d64", "llama2_70b_gqa_causal_n8192_d128", "long_seq_causal_n65536_d128")
                  if n != w.name]
        inp = L.inp
        del L
        torch.cuda.empty_cache()
        out["other_workloads"] = other_workloads(dev, others)
        out["decode"] = decode_leg(dev)
        out["fp8_forward"] = fp8_leg(dev)
        out["dropout"] = dropout_leg(dev)
    else:
        inp = L.inp
        for key in ("sclk_mhz_under_load", "bwd_preprocess", "other_workloads", "decode", "fp8_forward", "dropout"):
            out[key] = None
    out["host"] = host_info()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, inp)
        out["cpu_baseline"]["cpu_model"] = out["host"]["cpu_model"]
        out["cpu_baseline"]["blas"] = out["host"]["blas"]
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
