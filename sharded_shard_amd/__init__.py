"""MI355X-native FSDP2 per-rank sharded step: HIP kernels behind a C ABI.

``sharded_shard_amd.capi`` is the ctypes binding of ``include/fsdp_shard.h``;
``sharded_shard_amd.group`` holds a parameter group's persistent device tensors
and drives the four calls.  Build with ``python -m sharded_shard_amd.build``.
"""
