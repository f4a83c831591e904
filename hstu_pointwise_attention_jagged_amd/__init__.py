"""MI355X-native (gfx950) HSTU layer forward: hand-written HIP kernels behind a C ABI.

The computation lives in ``libhstu.so`` (sources in ``csrc/``, declarations in
``include/hstu.h``).  ``ops`` is a thin ctypes binding with the same entry-point names;
``workloads`` draws seeded synthetic inputs; ``device`` moves them onto the GPU.
"""

from . import workloads  # noqa: F401

__all__ = ["workloads", "ops", "device"]


def __getattr__(name):
    # torch-dependent modules load on first use, so the input generators stay importable
    # without touching the GPU stack
    if name in ("ops", "device"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
