"""kvc: budgeted KV-cache compaction on AMD MI355X (gfx950).

The product is libkvc.so (HIP kernels behind the C ABI of include/kvc.h);
``budgeted_retention_amd.kvc`` is its Python binding and
``budgeted_retention_amd.synth`` the seeded workload generators. Importing
this package loads nothing; the library is loaded on first use and its
absence is an error.
"""
