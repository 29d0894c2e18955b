"""Forward pass of a top-k routed Mixture-of-Experts FFN layer on MI355X
(gfx950): HIP kernels behind a C ABI (include/moe.h), with a thin torch
binding for device memory and streams.

Importing the package loads nothing; the library is loaded on first use and
raises if it has not been built.
"""

__all__ = ["binding", "build"]
