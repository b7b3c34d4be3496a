"""MI355X-native persistent decode megakernel for a parallel-block MoE transformer.

Importing the package loads nothing native.  ``persistent_moe_amd.mk`` is the
ctypes binding of the C-ABI library ``libmk.so`` (see ``include/mk.h``);
``persistent_moe_amd.workloads`` holds the workload shapes and the seeded input
generator; ``persistent_moe_amd.runner`` allocates inputs on the GPU and drives
decode steps through the binding.
"""
