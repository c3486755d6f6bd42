"""MI355X (gfx950) library for one tensor-parallel shard of a parallel
transformer block with causal sliding-window attention, forward and backward,
and the fused LAMB optimizer step.

The computation lives in libptb.so (hand-written HIP kernels behind the C ABI
of include/ptb.h); ``binding`` is a thin ctypes layer over it and
``device`` holds device-buffer helpers built on that binding.
"""
from . import binding  # noqa: F401
