"""MI355X-native Core Context Aware (CCA) attention.

The compute path is the HIP library ``libcca.so`` built from ``csrc/``; this
package only marshals arguments to its C entry points (see ``include/cca.h``).
Importing the package does not load the library; the first use of a binding
does, and fails loudly if the library has not been built.
"""

__all__ = [
    "pool_kv", "prefill", "attention", "KVCache", "cache_append", "decode_step",
    "kv_cache_bytes", "load_library", "CCAError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
