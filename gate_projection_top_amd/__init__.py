"""Fused MoE router for AMD MI355X (gfx950).

The compute path is ``librouter.so`` (hand-written HIP kernels behind a C ABI,
declared in include/router.h); ``gate_projection_top_amd.router`` is its thin
Python binding.  ``workloads`` builds seeded synthetic inputs.

Submodules are imported explicitly so that importing the package does not load
the HIP library.
"""
__all__ = ["router", "workloads"]
