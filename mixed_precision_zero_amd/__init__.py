"""MI355X-native ZeRO-1 shard optimizer step.

The work is done by ``libz1.so`` (HIP for gfx950, C ABI in ``include/z1.h``);
``binding`` marshals torch tensors into it, ``shard`` wires one rank's
buffers together, ``workloads`` defines the synthetic parameter lists.
"""
__all__ = ["binding", "shard", "workloads", "build"]
