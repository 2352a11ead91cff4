"""Weight-absorbed MLA decode for MI355X (gfx950).

The compute path is the C-ABI library ``libmla.so`` (hand-written HIP
kernels); ``mla_latent_kv_05_amd.mla`` is a thin ctypes binding with the same
entry-point names.  Importing this package loads nothing: the library is loaded
on first use and raises if it has not been built.
"""
__all__ = ["inputs", "accounting", "mla"]
