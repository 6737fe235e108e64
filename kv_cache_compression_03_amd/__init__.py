"""CSA2 compressed-sparse-attention layer for MI355X (gfx950).

The layer runs in the HIP library ``libcsa2.so`` (sources in ``csrc/``, C ABI in
``include/csa2.h``).  ``binding`` exposes the six calls to Python over ctypes;
``schedule`` runs a Full/Reindex/Reuse layer schedule on top of them.
"""
__all__ = ["binding", "schedule", "build"]
