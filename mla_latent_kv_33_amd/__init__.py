"""MLA decode over a paged latent KV cache on MI355X (gfx950).

The compute lives in libmla.so (hand-written HIP kernels behind the C ABI of
include/mla.h).  `binding` wraps those calls for torch tensors, `layer`
holds a layer's device buffers, `workloads` draws seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use.
"""
__all__ = ["binding", "layer", "workloads", "build"]
