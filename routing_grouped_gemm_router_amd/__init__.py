"""MI355X-native MoE-layer hot path: router, permutation, SwiGLU grouped GEMM
and combine, forward and backward, as hand-written HIP kernels for gfx950
behind a C-ABI library (``include/moe.h``).

``abi`` loads the library and marshals arguments; ``layer`` composes one
forward and backward pass from its calls; ``inputs`` draws seeded synthetic
workloads.  Nothing here computes on the CPU: if the HIP library is missing,
loading it raises.
"""

__all__ = ["abi", "layer", "inputs"]
