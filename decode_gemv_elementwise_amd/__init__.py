"""Fused-epilogue decode GEMV for MI355X (gfx950).

y = epilogue(W x) for one output column, with the epilogue applied straight
out of the accumulator in the same HIP kernel.  The compute lives in the
C-ABI library ``libgemv_fused.so`` (hand-written HIP for gfx950); the
``binding`` module marshals torch tensors into it.  ``synth`` holds the
seeded synthetic inputs and the weight packers.
"""
__all__ = ["binding", "synth"]
