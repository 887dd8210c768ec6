"""MI355X-native Nectar attention hot path.

The compute path is the C-ABI library ``libnectar.so`` (hand-written HIP for
gfx950, declared in ``include/nectar.h``); ``nectar.py`` is its thin ctypes
binding for torch tensors.  ``configs`` and ``synth`` describe and generate the
synthetic workloads.
"""
from . import configs, synth  # noqa: F401  (pure Python, no GPU needed)

__all__ = ["configs", "synth"]
