"""MI355X (gfx950) H2O heavy-hitter KV-cache eviction decode step.

The compute path is libh2o.so (HIP kernels behind the C ABI of include/h2o.h);
``H2OCache`` is its Python binding.  ``synth`` draws the seeded inputs and
``workloads`` lists the five synthetic workloads.
"""
from __future__ import annotations

__all__ = ["H2OCache", "H2OConfig", "H2OError", "make_config", "config_from_workload",
           "load_library", "synth", "workloads"]


def __getattr__(name):
    if name in ("H2OCache", "H2OConfig", "H2OError", "make_config", "config_from_workload",
                "load_library", "pages_needed"):
        from . import _lib
        return getattr(_lib, name)
    if name in ("synth", "workloads"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
