"""MI355X (gfx950) implementation of the Gecko per-layer forward: sliding chunk
attention plus adaptive working memory, behind a C-ABI library (libgecko.so).

The compute entry points live in :mod:`chunked_attention_memory_amd.gecko`
(a ctypes binding; importing it loads the HIP library and fails loudly if it
is not built). :mod:`configs` and :mod:`inputs` are host-only helpers.
"""

from . import configs, inputs  # noqa: F401

__all__ = ["configs", "inputs", "gecko"]


def __getattr__(name):
    if name == "gecko":
        import importlib

        return importlib.import_module(__name__ + ".gecko")
    raise AttributeError(name)
