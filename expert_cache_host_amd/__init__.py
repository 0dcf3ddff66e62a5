"""MI355X-native routed-MoE layer served from a per-layer GPU cache of hot experts.

The work happens in libmoecache.so (HIP kernels for gfx950 plus a C++ host
runtime) behind the C ABI of include/moe_cache.h; `binding` marshals arguments
to it with ctypes.  Build the library with `python -m expert_cache_host_amd.build`.
"""
from .binding import (MISS_HOST, MISS_STREAM, MoECache, MoeError, Planner,  # noqa: F401
                      host_expert_forward, host_topk, lib_path, load_library, slot_bytes)
