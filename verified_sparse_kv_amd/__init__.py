"""VerKV hot path on AMD Instinct MI355X: PoissonComp and KVFetch as HIP
kernels behind a C ABI (include/verkv.h).

``verified_sparse_kv_amd.verkv`` loads ``libverkv.so`` (built in-tree by
``verified_sparse_kv_amd.build``) and raises when it is missing; importing
this package alone loads nothing.
"""

__all__ = ["verkv", "build"]
