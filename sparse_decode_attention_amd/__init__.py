"""SparK on MI355X: query-aware, recoverable KV-cache channel pruning.

The compute path is the HIP library ``libspark.so`` (built from ``csrc/``)
behind the C ABI declared in ``include/spark.h``; ``ops`` is a thin ctypes
binding over torch device tensors. Importing this package does not load the
library; the first call into ``ops`` does, and fails loudly if it is missing.
"""
__all__ = ["configs", "gen", "ops"]
