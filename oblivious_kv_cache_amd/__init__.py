"""TurboQuant packed-key attention for MI355X (gfx950).

The compute path is the C-ABI library ``lib/libtq.so`` (HIP kernels), reached
through :mod:`oblivious_kv_cache_amd.binding`; importing that module fails
loudly if the library has not been built.  :mod:`oblivious_kv_cache_amd.workloads`
holds the seeded synthetic input recipes.
"""

__all__ = ["binding", "workloads", "build"]
