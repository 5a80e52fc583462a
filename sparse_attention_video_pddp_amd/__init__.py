"""MC-Sparse token-sparse attention for video diffusion transformers, native
on AMD Instinct MI355X (gfx950).

* ``mcs``   - ctypes binding of libmcs.so (include/mcs.h): mcs_group,
              mcs_anchor, mcs_sparse_attn, mcs_dense_attn.
* ``synth`` - seeded synthetic video-token workloads.
* ``build`` - hipcc build of libmcs.so.
"""
from . import mcs, synth  # noqa: F401

__all__ = ["mcs", "synth"]
