"""libssd: Mamba-2 SSD varlen chunked scan (forward prefill) for AMD MI355X.

The compute path is the HIP library ``libssd.so`` (built for gfx950) behind
the C ABI declared in ``include/ssd.h``; ``binding`` marshals torch tensors
into that ABI.  Importing this package does not load the library; the first
call does, and raises if it is missing (there is no CPU fallback).
"""

__all__ = ["workloads"]
