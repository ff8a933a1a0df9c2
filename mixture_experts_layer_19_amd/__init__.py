"""MI355X-native forward pass of one Hunyuan-style mixture-of-experts layer.

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP for
gfx950, built from ``csrc/``); :mod:`.binding` is a thin ctypes layer over it.
The library is loaded on first use and loading fails loudly if it has not
been built: there is no fallback path.
"""
__all__ = ["binding", "inputs"]
