"""Windowed grouped-query softmax attention for MI355X (gfx950).

The compute lives in the HIP library ``libwa.so`` (C ABI declared in ``include/wa.h``);
this package holds its thin binding (``api``), the seeded input generators
(``workloads``) and the build step (``build``).
"""

__all__ = ["api", "workloads", "build"]


def __getattr__(name):
    if name in ("decode", "prompt", "merge", "decode_workspace_bytes", "window"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
