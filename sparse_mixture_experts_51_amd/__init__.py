"""MI355X-native DeepSeekMoE layer forward.

    libmoe.so          gfx950 HIP kernels behind the C ABI in include/moe.h
    moe                thin ctypes binding with the C entry points' names
    workloads          seeded synthetic inputs for the named workloads
    build              in-tree hipcc build of libmoe.so
"""
__all__ = ["moe", "workloads", "build"]
