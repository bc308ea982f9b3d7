"""Thin Python binding of the C ABI in ``include/fa.h``.

``fa_fwd``, ``fa_fwd_fp8``, ``fa_bwd``, ``fa_bwd_noalloc``, ``fa_bwd_preprocess``, ``fa_bwd_dkdv``, ``fa_fwd_splitkv``,
``fa_fwd_splitkv_workspace_size``, ``fa_merge``,
``fa_bwd_dq``, ``fa_bwd_workspace_size`` and ``fa_status_string`` have
the C names and argument order; pointer arguments accept an integer device
address or any object with ``data_ptr()`` (a torch tensor), and ``stream`` an
integer ``hipStream_t``, a torch stream, or ``None`` for torch's current stream.
They return the C status code unchanged.  ``forward``/``backward`` are small
conveniences that allocate outputs with torch and raise on a non-zero status.
Every step of the computation runs in the HIP library; nothing here computes.
"""
from __future__ import annotations

import ctypes
import math
import os

FA_BF16, FA_F32 = 0, 1
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_TOO_LARGE = range(6)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(fa_status_string(status))
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tiled_attention_14_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, P]
        L.fa_fwd.restype = I
        L.fa_bwd_workspace_size.argtypes = [I, I, I, I, I, I]
        L.fa_bwd_workspace_size.restype = S
        L.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, S, P]
        L.fa_bwd.restype = I
        L.fa_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
        L.fa_bwd_noalloc.restype = I
        L.fa_bwd_preprocess.argtypes = [P, P, P, I, I, I, I, I, I, P, S, P]
        L.fa_bwd_preprocess.restype = I
        L.fa_bwd_dkdv.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, S, P]
        L.fa_bwd_dkdv.restype = I
        L.fa_bwd_dq.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, S, P]
        L.fa_bwd_dq.restype = I
        L.fa_fwd_splitkv_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
        L.fa_fwd_splitkv_workspace_size.restype = S
        L.fa_fwd_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P, S, P]
        L.fa_fwd_splitkv.restype = I
        L.fa_merge.argtypes = [P, P, P, P, I, ctypes.c_long, I, I, P]
        L.fa_merge.restype = I
        L.fa_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, F, F, F, F, I, P]
        L.fa_fwd_fp8.restype = I
        U64, U32 = ctypes.c_ulonglong, ctypes.c_uint
        L.fa_fwd_dropout.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, F, U64, U32, I, P]
        L.fa_fwd_dropout.restype = I
        L.fa_bwd_dropout.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, F, U64, U32, I, P, S, P]
        L.fa_bwd_dropout.restype = I
        L.fa_status_string.argtypes = [I]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_build_hash.argtypes = []
        L.fa_build_hash.restype = ctypes.c_char_p
        from tiled_attention_14_amd.build import source_hash
        built, tree = L.fa_build_hash().decode(), source_hash()
        if built != tree:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (hash {built}) than this tree holds "
                               f"({tree}): rebuild it with `python -m tiled_attention_14_amd.build`")
        _lib = L
    return _lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int | None:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(s, int):
        return s or None
    return int(s.cuda_stream) or None


# ------------------------------------------------------------------ C names
def fa_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, dtype, stream=None) -> int:
    return lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                        float(scale), int(bool(causal)), int(dtype), _stream(stream))


def fa_bwd_workspace_size(B, H, Hkv, N, d, dtype) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, Hkv, N, d, int(dtype)))


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, dtype,
           workspace, workspace_bytes, stream=None) -> int:
    return lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                        _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                        int(bool(causal)), int(dtype), _ptr(workspace), int(workspace_bytes),
                        _stream(stream))


def fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, dtype, stream=None) -> int:
    return lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                int(bool(causal)), int(dtype), _stream(stream))


def fa_fwd_dropout(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, p_drop, seed, offset, dtype,
                   stream=None) -> int:
    return lib().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale),
                                int(bool(causal)), float(p_drop), int(seed), int(offset), int(dtype),
                                _stream(stream))


def fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, p_drop, seed, offset,
                   dtype, workspace, workspace_bytes, stream=None) -> int:
    return lib().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                int(bool(causal)), float(p_drop), int(seed), int(offset), int(dtype),
                                _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_bwd_preprocess(o, dO, lse, B, H, Hkv, N, d, dtype, workspace, workspace_bytes, stream=None) -> int:
    return lib().fa_bwd_preprocess(_ptr(o), _ptr(dO), _ptr(lse), B, H, Hkv, N, d, int(dtype),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_bwd_dkdv(q, k, v, dO, dk, dv, B, H, Hkv, N, d, scale, causal, dtype,
                workspace, workspace_bytes, stream=None) -> int:
    return lib().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dk), _ptr(dv),
                             B, H, Hkv, N, d, float(scale), int(bool(causal)), int(dtype),
                             _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_bwd_dq(q, k, v, o, dO, lse, dq, B, H, Hkv, N, d, scale, causal, dtype,
              workspace, workspace_bytes, stream=None) -> int:
    return lib().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq),
                           B, H, Hkv, N, d, float(scale), int(bool(causal)), int(dtype),
                           _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_fwd_fp8(q, k, v, o, lse, B, H, Hkv, N, d, scale, q_scale, k_scale, v_scale, causal, stream=None) -> int:
    return lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale),
                            float(q_scale), float(k_scale), float(v_scale), int(bool(causal)), _stream(stream))


def fa_fwd_splitkv_workspace_size(B, H, Hkv, Nq, Nk, d, dtype, nsplit=0) -> int:
    return lib().fa_fwd_splitkv_workspace_size(B, H, Hkv, Nq, Nk, d, int(dtype), int(nsplit))


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, nsplit,
                   workspace, workspace_bytes, stream=None) -> int:
    return lib().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                                float(scale), int(bool(causal)), int(dtype), int(nsplit),
                                _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_merge(o_parts, lse_parts, o, lse, nsplit, rows, d, dtype, stream=None) -> int:
    return lib().fa_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse), int(nsplit), int(rows), d,
                          int(dtype), _stream(stream))


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


# ------------------------------------------------------------------ conveniences
def _dims(q, k):
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k/v [B, Hkv, N, d]")
    if q.dtype == torch.bfloat16:
        dt = FA_BF16
    elif q.dtype == torch.float32:
        dt = FA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    return B, H, k.shape[1], N, d, dt


def _check_tensors(*ts):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")


def workspace(B, H, Hkv, N, d, dtype, device):
    """A caller-owned workspace tensor and its 256-byte-aligned address and size."""
    import torch
    n = fa_bwd_workspace_size(B, H, Hkv, N, d, dtype)
    if n == 0:
        raise FAError(FA_ERR_INVALID_ARG)
    buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
    addr = (buf.data_ptr() + 255) // 256 * 256
    return buf, addr, n


def forward(q, k, v, scale=None, causal=False, stream=None):
    """(o, lse) for q [B,H,N,d], k/v [B,Hkv,N,d] (bf16 or f32 device tensors)."""
    import torch
    _check_tensors(q, k, v)
    B, H, Hkv, N, d, dt = _dims(q, k)
    s = float(scale) if scale is not None else 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_fwd(q, k, v, o, lse, B, H, Hkv, N, d, s, causal, dt, stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def backward(q, k, v, o, do, lse, scale=None, causal=False, stream=None, ws=None):
    """(dq, dk, dv) of sum(do * o); ``ws`` may pass a workspace from :func:`workspace`."""
    import torch
    _check_tensors(q, k, v, o, do, lse)
    B, H, Hkv, N, d, dt = _dims(q, k)
    s = float(scale) if scale is not None else 1.0 / math.sqrt(d)
    dq = torch.empty_like(q); dk = torch.empty_like(k); dv = torch.empty_like(v)
    if ws is None:
        ws = workspace(B, H, Hkv, N, d, dt, q.device)
    _, addr, n = ws
    st = fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, Hkv, N, d, s, causal, dt, addr, n, stream)
    if st != FA_OK:
        raise FAError(st)
    return dq, dk, dv


def forward_dropout(q, k, v, p_drop, seed, offset=0, scale=None, causal=False, stream=None):
    """(o, lse) with dropout of rate ``p_drop`` on the probabilities (mask drawn
    from ``seed`` and ``offset``; see fa_fwd_dropout in include/fa.h)."""
    import torch
    _check_tensors(q, k, v)
    B, H, Hkv, N, d, dt = _dims(q, k)
    s = float(scale) if scale is not None else 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_fwd_dropout(q, k, v, o, lse, B, H, Hkv, N, d, s, causal, p_drop, seed, offset, dt, stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def backward_dropout(q, k, v, o, do, lse, p_drop, seed, offset=0, scale=None, causal=False, stream=None,
                     ws=None):
    """(dq, dk, dv) of sum(do * o) for the o of :func:`forward_dropout` with the
    same rate, seed and offset (the mask is regenerated, not stored)."""
    import torch
    _check_tensors(q, k, v, o, do, lse)
    B, H, Hkv, N, d, dt = _dims(q, k)
    s = float(scale) if scale is not None else 1.0 / math.sqrt(d)
    dq = torch.empty_like(q); dk = torch.empty_like(k); dv = torch.empty_like(v)
    if ws is None:
        ws = workspace(B, H, Hkv, N, d, dt, q.device)
    _, addr, n = ws
    st = fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, B, H, Hkv, N, d, s, causal, p_drop, seed, offset, dt,
                        addr, n, stream)
    if st != FA_OK:
        raise FAError(st)
    return dq, dk, dv


def forward_kv(q, k, v, scale=None, causal=False, nsplit=0, stream=None):
    """(o, lse) for q [B,H,Nq,d] against k/v [B,Hkv,Nk,d] through ``fa_fwd_splitkv``
    (bottom-right causal alignment; ``nsplit`` key ranges, 0 = library's choice)."""
    import torch
    _check_tensors(q, k, v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    dt = FA_BF16 if q.dtype == torch.bfloat16 else FA_F32
    s = float(scale) if scale is not None else 1.0 / math.sqrt(d)
    n = fa_fwd_splitkv_workspace_size(B, H, Hkv, Nq, Nk, d, dt, nsplit)
    if n == 0:
        raise FAError(FA_ERR_INVALID_ARG)
    buf = torch.empty(n + 256, dtype=torch.uint8, device=q.device)
    addr = (buf.data_ptr() + 255) // 256 * 256
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = fa_fwd_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, s, causal, dt, nsplit, addr, n, stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse
