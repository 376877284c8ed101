"""Persistent, tile-scheduled, pipelined GEMM for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmigemm.so`` (hand-written HIP for
gfx950, declared in ``include/migemm.h``); ``migemm`` is its thin ctypes
binding and ``synth`` draws seeded synthetic inputs.  Nothing is loaded at
import time: the binding loads the library on first use and raises if it has
not been built.
"""
