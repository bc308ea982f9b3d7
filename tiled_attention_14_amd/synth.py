"""Seeded synthetic inputs and the named attention workloads.

This module is shared by the parity tests, the smoke check and the benchmark.
It holds *no* attention arithmetic: it only draws random tensors, rounds them
to bfloat16 when a workload asks for bf16 inputs, and describes the shapes.
Both the HIP path and the CPU oracle receive exactly the values produced here.

Recipe (stated once, used everywhere):
  * ``numpy.random.Generator(PCG64(seed))``; tensors drawn in the order
    Q, K, V, dO, each as C-order float32 ``standard_normal`` times a std.
  * bf16 workloads round every float32 draw to bfloat16 with
    round-to-nearest-even on the host; the GPU receives the bf16 bit patterns
    and the oracle receives the same values upcast to float64.
  * Shapes are ``[B, H, N, d]`` for Q and dO, ``[B, Hkv, N, d]`` for K and V.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    qk_std: float = 1.0
    vdo_std: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32 (the value the library receives)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five named workloads of the exact-attention study.  Seeds are 14000 + k.
WORKLOADS = {
    "single_head_f32_n256_d64": Workload(
        "single_head_f32_n256_d64", 1, 1, 1, 256, 64, "f32", False, seed=14000),
    "mha_bf16_n2048_d64": Workload(
        "mha_bf16_n2048_d64", 4, 16, 16, 2048, 64, "bf16", False, seed=14001),
    "llama2_7b_causal_n4096_d128": Workload(
        "llama2_7b_causal_n4096_d128", 2, 32, 32, 4096, 128, "bf16", True, seed=14002),
    "llama2_70b_gqa_causal_n8192_d128": Workload(
        "llama2_70b_gqa_causal_n8192_d128", 1, 64, 8, 8192, 128, "bf16", True, seed=14003),
    "long_seq_causal_n65536_d128": Workload(
        "long_seq_causal_n65536_d128", 1, 8, 8, 65536, 128, "bf16", True,
        qk_std=2.0, seed=14004),
}

HEADLINE = "llama2_7b_causal_n4096_d128"


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normals, so the NaN/Inf special cases of the
    conversion never arise; they are rejected to keep that assumption honest.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round_bits expects finite values")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


@dataclasses.dataclass
class Inputs:
    """One seeded draw.  ``vals`` are float32 arrays holding exactly the values
    the library sees (bf16-rounded for bf16 workloads); ``bits`` holds the
    uint16 bf16 patterns for bf16 workloads and is ``None`` for f32."""
    w: Workload
    vals: dict
    bits: dict | None

    def f64(self, name: str) -> np.ndarray:
        return self.vals[name].astype(np.float64)


def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    qshape = (w.B, w.H, w.N, w.d)
    kshape = (w.B, w.Hkv, w.N, w.d)
    raw = {
        "q": rng.standard_normal(qshape, dtype=np.float32) * np.float32(w.qk_std),
        "k": rng.standard_normal(kshape, dtype=np.float32) * np.float32(w.qk_std),
        "v": rng.standard_normal(kshape, dtype=np.float32) * np.float32(w.vdo_std),
        "do": rng.standard_normal(qshape, dtype=np.float32) * np.float32(w.vdo_std),
    }
    if w.dtype == "f32":
        return Inputs(w, raw, None)
    if w.dtype != "bf16":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    bits = {n: bf16_round_bits(a) for n, a in raw.items()}
    vals = {n: bf16_bits_to_f32(b) for n, b in bits.items()}
    return Inputs(w, vals, bits)


def sample_rows(n_total: int, n_sample: int, seed: int, count: int) -> np.ndarray:
    """``count`` independent sorted samples (uniform, without replacement) of
    ``min(n_sample, n_total)`` row indices from ``range(n_total)``; one per head."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = min(n_sample, n_total)
    return np.stack([np.sort(rng.choice(n_total, size=k, replace=False)) for _ in range(count)])


@dataclasses.dataclass(frozen=True)
class KvWorkload:
    """Nq query rows against a cache of Nk keys (decoding when Nq == 1)."""
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    seed: int = 0
    qk_std: float = 1.0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0) / np.sqrt(np.float32(self.d)))


# Decoding one token per sequence against a cache, at the attention shapes of
# the two models above: 70B-shaped GQA (64 query heads over 8 KV heads) with a
# 8192-token cache, and 7B-shaped MHA with a 4096-token cache.
KV_WORKLOADS = {
    "decode_llama2_70b_gqa_b16_nk8192_d128": KvWorkload("decode_llama2_70b_gqa_b16_nk8192_d128",
                                                        16, 64, 8, 1, 8192, 128, "bf16", True, seed=14100),
    "decode_llama2_7b_b16_nk4096_d128": KvWorkload("decode_llama2_7b_b16_nk4096_d128",
                                                   16, 32, 32, 1, 4096, 128, "bf16", True, seed=14101),
}


def make_kv_inputs(w: KvWorkload, seed: int | None = None) -> Inputs:
    """Seeded q [B,H,Nq,d], k and v [B,Hkv,Nk,d], drawn in that order like
    make_inputs: q and k iid N(0, qk_std^2), v iid N(0, 1); bf16 workloads are
    rounded to bf16 (RNE)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    raw = {
        "q": rng.standard_normal((w.B, w.H, w.Nq, w.d), dtype=np.float32) * np.float32(w.qk_std),
        "k": rng.standard_normal((w.B, w.Hkv, w.Nk, w.d), dtype=np.float32) * np.float32(w.qk_std),
        "v": rng.standard_normal((w.B, w.Hkv, w.Nk, w.d), dtype=np.float32),
    }
    if w.dtype == "f32":
        return Inputs(w, raw, None)
    if w.dtype != "bf16":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    bits = {n: bf16_round_bits(a) for n, a in raw.items()}
    vals = {n: bf16_bits_to_f32(b) for n, b in bits.items()}
    return Inputs(w, vals, bits)


# ---------------------------------------------------------------- fp8 (OCP e4m3) inputs
# 8-bit floats in the OCP "E4M3" format: sign, 4 exponent bits (bias 7), 3
# mantissa bits; exponent field 0 holds subnormals (m / 8 * 2^-6); the code
# S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448;
# there is no infinity.
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> nearest e4m3 code (ties to even), saturating at +-448.  Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode expects finite values")
    table = e4m3_decode(np.arange(128, dtype=np.uint8))   # non-negative codes 0..127
    finite = np.arange(127)                               # 127 is NaN
    vals = table[finite]
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left").clip(0, 126)
    lo = (hi - 1).clip(0, 126)
    dlo, dhi = np.abs(a - vals[lo]), np.abs(vals[hi] - a)
    # nearest; on a tie the even code (its mantissa's last bit 0)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(x < 0, 0x80, 0)).astype(np.uint8)


@dataclasses.dataclass
class Fp8Inputs:
    """fp8 attention inputs: e4m3 codes and per-tensor scales; ``f64(name)`` is
    the value the library computes with (decoded code times scale)."""
    codes: dict
    scales: dict

    def f64(self, name: str) -> np.ndarray:
        return e4m3_decode(self.codes[name]) * self.scales[name]


def make_fp8_inputs(B, H, Hkv, N, d, seed, qk_std=1.0) -> Fp8Inputs:
    """Seeded Q, K, V (iid normal, drawn in that order) quantized per tensor to
    e4m3 with the scale that maps the tensor's largest magnitude to 448."""
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = {"q": rng.standard_normal((B, H, N, d), dtype=np.float32) * np.float32(qk_std),
           "k": rng.standard_normal((B, Hkv, N, d), dtype=np.float32) * np.float32(qk_std),
           "v": rng.standard_normal((B, Hkv, N, d), dtype=np.float32)}
    codes, scales = {}, {}
    for n, a in raw.items():
        s = float(np.float32(np.max(np.abs(a)) / E4M3_MAX))
        codes[n] = e4m3_encode(a / s)
        scales[n] = s
    return Fp8Inputs(codes, scales)
