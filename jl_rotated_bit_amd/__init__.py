"""QJL KV-cache compression for AMD Instinct MI355X (gfx950).

* ``jl_rotated_bit_amd.qjl``       - binding of libqjl.so (C ABI in include/qjl.h)
* ``jl_rotated_bit_amd.build``     - builds libqjl.so with hipcc
* ``jl_rotated_bit_amd.workloads`` - seeded synthetic inputs of the five workloads
"""
