"""MI355X (gfx950) library for weight-absorbed MLA / TPLA decode over a latent KV cache.

The compute lives in a C-ABI shared library built from ``csrc/`` (HIP kernels
for gfx950); ``binding`` marshals torch device tensors into its entry points.
Nothing here computes on the CPU.  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""

__all__ = ["binding", "inputs", "build"]
