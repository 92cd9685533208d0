"""Memory accounting of mixed-precision AdamW and ZeRO-1 (TEST INFRASTRUCTURE ONLY).

Plain arithmetic of the per-parameter byte budget the pages state:

* "Distributed Training" (atlas wiki), How it works, section 0 "The baseline":
  mixed-precision Adam keeps 2 bytes of bf16/fp16 weight, 2 bytes of gradient
  and 12 bytes of fp32 optimizer state (master copy, first and second moment)
  per parameter, 16 bytes in all; the optimizer state is three quarters of it.
* "ZeRO-1 风格的 Distributed Optimizer" (nanotron tutorial), sections 6.1 and
  6.3: ZeRO-1 splits only the fp32 optimizer state over the data-parallel
  ranks; bf16 weights stay whole on every rank.
"""

WEIGHT_BYTES = 2          # bf16 / fp16 working weight
GRAD_BYTES = 2            # bf16 / fp16 gradient
MASTER_BYTES = 4          # fp32 master weight
MOMENT_BYTES = 4 + 4      # fp32 first and second moments

OPT_STATE_BYTES = MASTER_BYTES + MOMENT_BYTES              # 12
TOTAL_BYTES = WEIGHT_BYTES + GRAD_BYTES + OPT_STATE_BYTES  # 16


def total_bytes(psi: float) -> float:
    """16 * psi: everything mixed-precision Adam keeps on one replica."""
    return TOTAL_BYTES * psi


def optimizer_state_bytes(psi: float) -> float:
    """12 * psi: fp32 master + m + v."""
    return OPT_STATE_BYTES * psi


def zero1_optimizer_state_per_rank(psi: float, dp_size: int) -> float:
    """ZeRO-1 partitions only the optimizer state: 12 * psi / dp_size."""
    return OPT_STATE_BYTES * psi / dp_size


def zero1_total_per_rank(psi: float, dp_size: int) -> float:
    """Weights and gradients stay whole: (2 + 2) * psi + 12 * psi / dp_size."""
    return (WEIGHT_BYTES + GRAD_BYTES) * psi + zero1_optimizer_state_per_rank(psi, dp_size)


def shard_state_bytes(shard_elems: int) -> int:
    """fp32 master + m + v actually held for a shard of `shard_elems` elements."""
    return OPT_STATE_BYTES * int(shard_elems)
