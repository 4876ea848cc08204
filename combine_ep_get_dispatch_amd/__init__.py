"""MoE token dispatch and combine for MI355X (gfx950).

The work is done by hand-written HIP kernels behind a C ABI
(``include/ep.h``, built into ``libep_mi355x.so``); ``binding`` marshals torch
tensors into those calls.  ``workloads`` draws seeded synthetic inputs.
"""
