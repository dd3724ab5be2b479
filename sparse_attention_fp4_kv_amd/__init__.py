"""libcsa2: sparse FP4-KV decode path for MI355X (gfx950).

The compute lives in the HIP library libcsa2.so (C ABI in include/csa2.h);
``csa2`` is its thin ctypes binding, ``workloads`` holds the seeded synthetic
inputs, ``build_lib`` compiles the library.
"""
