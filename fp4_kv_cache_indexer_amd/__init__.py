"""CSA2 decode hot path (FP4 main-KV cache + sparse indexer) for MI355X.

The compute lives in the HIP library ``libcsa2.so`` (built from ``csrc/``);
``fp4_kv_cache_indexer_amd.csa2`` is its thin ctypes binding, imported on
demand so that importing the package (e.g. for the synthetic inputs) needs
no GPU and no built library.
"""

__all__ = ["csa2", "synth", "config"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
