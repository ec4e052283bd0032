"""MI355X-native paged BF16 block operator (Precision-Preserving Subtensor
Inference): a fixed device arena, weight pages streamed from pinned host
memory, and hand-written gfx950 kernels behind a C ABI (``include/psi.h``).

Importing the package does not load the HIP library; ``psi`` does, and it
raises if the library has not been built.
"""
__all__ = ["psi", "synth"]
