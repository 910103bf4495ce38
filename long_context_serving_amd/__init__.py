"""MI355X-native segmented paged KV attention (head-classified global/local heads).

The compute path is libsegkv.so (HIP kernels for gfx950 behind the C ABI in
include/segkv.h); ``segkv`` is its thin ctypes binding and ``workloads`` the
seeded synthetic input generator.  Importing the package does not load the
library; constructing ``segkv.SegKV`` does, and fails if it is not built.
"""

__all__ = ["segkv", "workloads", "build"]
