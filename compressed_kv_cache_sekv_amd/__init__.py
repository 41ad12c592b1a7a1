"""SeKV decode path for MI355X (gfx950): Python binding of the C-ABI library.

Importing the package loads nothing; `compressed_kv_cache_sekv_amd.lib` loads
the HIP library (libsekv.so) and raises if it has not been built.
"""
