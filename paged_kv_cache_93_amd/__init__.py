"""MI355X-native paged attention decode (HIP kernels behind the C ABI of libpagedattn).

Importing the package loads nothing native; ``paged_kv_cache_93_amd.lib``
loads the shared library on first use and fails loudly when it is missing.
"""
