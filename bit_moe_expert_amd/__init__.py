"""libmoe4: the quantized (W4A16) mixture-of-experts layer as hand-written HIP for gfx950.

The compute lives in ``libmoe4.so`` (C ABI in ``include/moe4.h``); ``binding`` is a
thin torch marshalling layer over it and ``workloads`` draws seeded synthetic inputs.
Importing this package loads nothing; ``binding`` loads the library on first use and
raises if it has not been built.
"""
__all__ = ["binding", "workloads", "build"]
