"""Split-KV (FlashDecoding) decode attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libfd.so`` built from ``csrc/``
(hand-written HIP kernels plus a thin host layer).  ``binding`` marshals torch
tensors into that ABI and loads the library on first use; it raises if the
library is missing rather than falling back to any other implementation.
"""
