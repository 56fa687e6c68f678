"""FLASH layer forward (gated attention unit with mixed-chunk attention) for AMD MI355X.

The compute path is the HIP library libflashgau.so (C ABI in include/flashgau.h); the binding
in ``flashgau`` only marshals arguments. ``inputs`` draws seeded synthetic workloads.
"""

__all__ = ["flashgau", "inputs"]


def __getattr__(name):
    # Submodules load on first use so that importing the input generator does not need the library.
    if name in ("flashgau", "inputs", "build"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
