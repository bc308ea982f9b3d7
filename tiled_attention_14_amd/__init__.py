"""Exact softmax attention (tiled online-softmax forward, FlashAttention-2
backward) for AMD Instinct MI355X (gfx950), behind the C ABI of ``include/fa.h``.

The HIP library is loaded on first use by :mod:`tiled_attention_14_amd.fa`;
importing the package itself loads nothing.
"""
__all__ = ["fa", "synth"]
