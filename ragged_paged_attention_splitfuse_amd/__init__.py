"""Ragged paged attention for Dynamic SplitFuse passes on MI355X (gfx950).

The compute path is the C-ABI library ``libfg.so`` (hand-written HIP kernels
plus a host planner) declared in ``include/fg.h``; ``binding`` is a thin
ctypes layer with the same entry-point names.  ``workloads`` draws seeded
synthetic passes and ``splitfuse`` composes passes from a request trace at a
fixed token budget.

The binding is imported lazily so that the input generator and the host
scheduler can be used without loading the library; every compute entry point
raises if the library is missing -- there is no fallback path.
"""

__all__ = ["binding", "workloads", "splitfuse"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
