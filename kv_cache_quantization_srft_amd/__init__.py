"""kv_cache_quantization_srft_amd: SRFT / SRHT rotate-then-quantize of KV-cache
vectors on AMD Instinct MI355X (gfx950).

The GPU path lives in libsrftq.so (HIP kernels behind the C ABI in
include/srftq.h); ``srftq`` is its Python binding (the library is loaded on
first use), ``kvcache`` a per-layer K/V cache grown by quantize-on-append,
``workloads`` the seeded synthetic inputs, ``build`` the hipcc build.
"""
from . import kvcache, srftq, workloads  # noqa: F401

__all__ = ["kvcache", "srftq", "workloads"]
