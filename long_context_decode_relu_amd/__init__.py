"""Decode-time Sevren Sparse Attention on MI355X (gfx950).

The compute runs in the HIP library ``libssa.so`` built from ``csrc/``; the
module :mod:`long_context_decode_relu_amd.ssa` is its thin ctypes binding and
:mod:`long_context_decode_relu_amd.synth` draws seeded synthetic inputs.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""

__all__ = ["ssa", "synth"]
