"""MI355X-native exact MoE-layer forward over a global expert cache.

The compute path is the HIP library ``libftmoe.so`` (C ABI, ``include/ft_moe.h``);
``sparse_moe_expert_softmax_amd.ftmoe`` is its thin ctypes binding.  ``configs``
and ``synth`` describe and generate the synthetic workloads.
"""
