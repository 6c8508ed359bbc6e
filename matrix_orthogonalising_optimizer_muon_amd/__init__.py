"""MI355X-native per-matrix Muon update (HIP kernels for gfx950 behind a C-ABI library).

``binding`` (loaded on first use) marshals arguments into ``libmuon_amd.so``; every step
of the update runs in the library's HIP kernels. ``workloads`` holds the seeded synthetic
inputs.
"""

import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in ("binding", "workloads"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
