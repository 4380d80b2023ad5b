"""Gated block-sparse decode attention on AMD Instinct MI355X (gfx950).

The computation lives in libseer.so (HIP kernels behind a C-ABI, see
include/seer.h); ``seer`` is its thin Python binding and ``pipeline`` wires the
calls of one decode step together.
"""
