"""Batched prompt-lookup (n-gram) drafting on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libpld.so`` (HIP kernels for gfx950,
declared in ``include/pld.h``); ``prompt_lookup_gram_amd.binding`` is a thin
ctypes layer over it with the same entry-point names. ``workloads`` holds the
seeded synthetic inputs. PyTorch is used only for device memory and streams.
"""

import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
