"""Scored decode attention for MI355X (gfx950).

One decode step attends each query over its sequence's KV cache, returns the
attention output, and reduces the post-softmax weights into one attention mass
per (sequence, 16-token block), summed over heads and scored layers. The mass
feeds a per-block side-car (Attended, EMA, Cumulative, trajectory ring) and a
heavy-hitter block selection (top blocks plus a recent window).

The compute lives in ``libkvs.so`` (HIP kernels behind a C ABI declared in
``include/kvs.h``); ``heavy_hitter_eviction_amd.api`` is the thin ctypes binding
over it. Importing this package does not load the library; importing ``api``
does, and raises if the library has not been built.
"""

from . import workloads  # noqa: F401

__all__ = ["workloads"]
