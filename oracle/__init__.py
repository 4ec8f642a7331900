"""CPU oracle of the FSDP2 per-rank sharded step (test infrastructure only).

Only tests/, the smoke check and the bench's CPU-baseline leg use this package.
The product library never imports, links or runs it.
"""
from .fsdp import (  # noqa: F401
    AdamWScalars, E4M3_MAX, Entry, Plan, accumulate_grad, adamw, amax, e4m3_sat, e4m3_to_f32,
    pack_fp8, unpack_fp8, adamw_scalars, bf16_rne, bf16_to_f32,
    chunk_rows, pack, pack_reduce_scatter, pack_reduce_scatter_acc, pack_reduce_scatter_f32, plan, reduce, reduce_f32,
    reshard, reshard_runs, rows_of_rank, state_bytes, unpack,
)
