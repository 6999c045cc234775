"""MI355X-native ZeRO / FSDP shard-local update.

The compute path is the C-ABI library libzero_shard.so (hand-written HIP
kernels for gfx950, declared in include/zero_shard.h); this package only
exposes it to Python.
"""
from .binding import (ACC_EMIT_BF16, ACC_NO_STORE, ACC_OVERWRITE, DTYPE_BF16, DTYPE_F32,
                      GRAD_COMPACT, GRAD_FLAT, OUT_AG_SLOT, OUT_SHARD, AdamW, Layout, ZeroError,
                      load, zero_bucket_pack, zero_gather_params, zero_grad_accumulate,
                      zero_reshard, zero_shard_step, zero_shard_step_accumulate,
                      zero_shard_step_buckets, zero_step_scalars)

__all__ = ["ACC_EMIT_BF16", "ACC_NO_STORE", "ACC_OVERWRITE", "DTYPE_BF16", "DTYPE_F32",
           "GRAD_COMPACT", "GRAD_FLAT",
           "OUT_AG_SLOT", "OUT_SHARD", "AdamW", "Layout", "ZeroError", "load",
           "zero_bucket_pack", "zero_gather_params", "zero_grad_accumulate", "zero_reshard",
           "zero_shard_step", "zero_shard_step_accumulate", "zero_shard_step_buckets",
           "zero_step_scalars"]
