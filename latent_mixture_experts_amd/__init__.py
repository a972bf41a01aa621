"""latent_mixture_experts_amd -- the latent MoE layer on one MI355X (gfx950).

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP kernels
for gfx950), declared in ``include/moe.h``. This package holds:

* :mod:`.binding` -- argument marshalling from torch tensors to the C-ABI;
* :mod:`.build`   -- the hipcc build of ``libmoe.so``;
* :mod:`.synth`   -- seeded synthetic inputs (no arithmetic of the layer).

Importing the package loads nothing; the library is loaded on first use and
a missing or unloadable library raises immediately (there is no fallback).
"""

__all__ = ["binding", "build", "synth"]
