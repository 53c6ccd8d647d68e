"""MI355X-native absorbed MLA decode over a paged latent KV cache.

The compute path is the C-ABI library ``libmla_kv.so`` (hand-written HIP for
gfx950); ``mla_latent_kv_09_amd.mla`` is its thin Python binding.  Importing
this package loads nothing; the binding loads the library on first use and
raises if it is missing.
"""

__all__ = ["workloads", "mla"]
