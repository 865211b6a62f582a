"""MiniMax Sparse Attention (MSA) hot path for one MI355X (gfx950).

The work happens in ``libmsa.so`` (hand-written HIP kernels behind the C ABI in
``include/msa.h``); ``_lib`` is its ctypes binding, ``pipeline`` runs one
layer-step through it, and ``inputs`` draws the seeded synthetic workloads.
Submodules load lazily so that importing the package never touches a GPU.
"""
__all__ = ["_lib", "pipeline", "inputs"]
