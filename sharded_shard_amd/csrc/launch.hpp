// Kernel launchers of the sharded-step library.  Each enqueues one kernel
// (amax: a clear and a kernel) over a plan's device tile table on `st` and
// returns hipGetLastError(); n is the number of tiles, and n == 0 launches
// nothing.  Callers (the C ABI) have checked every argument before.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "plan.hpp"

namespace fsdp {

// copy-in: fp32 master shards -> bf16 segment ag_in
hipError_t launch_pack(const PackTile *tiles, int64_t n, const DevEntry *ents, uint16_t *ag_in,
                       hipStream_t st);
// copy-out: [N, S] bf16 ag_out -> full parameters; chunk_aligned: every row
// piece starts 16-byte aligned
hipError_t launch_unpack(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *ag_out, bool chunk_aligned, hipStream_t st);
// reduce: [N, S] bf16 contributions -> fp32 mean into the grad shards
hipError_t launch_reduce(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *rs_in, int64_t S, int32_t N, bool chunk_aligned,
                         hipStream_t st);
// AdamW on the bound shards; scal: beta1, 1-beta1, beta2, 1-beta2, eps,
// 1-lr*wd, lr/(1-beta1^t), sqrt(1-beta2^t); one_launch: the tiles cover every
// group of a step (a group set), so no later kernel reads what it leaves in
// the caches
hipError_t launch_adamw(const EwTile *tiles, int64_t n, const DevEntry *ents,
                        const float scal[8], bool one_launch, hipStream_t st);
// AdamW, then the bf16 copy-in of the new master, over the copy-in tiles
hipError_t launch_adamw_pack(const PackTile *tiles, int64_t n, const DevEntry *ents,
                             uint16_t *ag_in, const float scal[8], hipStream_t st);
// fused reduce -> AdamW -> copy-in over the copy-in tiles
hipError_t launch_step(const PackTile *tiles, int64_t n, const DevEntry *ents,
                       const uint16_t *rs_in, uint16_t *ag_in, int64_t S, int32_t N,
                       const float scal[8], bool write_grad, bool chunk_aligned,
                       hipStream_t st);
// reduce-scatter copy-in: full bf16 gradients -> [N, S] bf16 or widened fp32
hipError_t launch_rspack(const PackTile *tiles, int64_t n, const DevEntry *ents, void *out,
                         bool f32, bool chunk_aligned, hipStream_t st);
// reduce of fp32 contributions
hipError_t launch_reduce_f32(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                             const float *rs_in, int64_t S, int32_t N, bool chunk_aligned,
                             hipStream_t st);
// fp32 accumulators += (or, with reset, =) bf16 full gradients
hipError_t launch_accumulate(const EwTile *tiles, int64_t n, const DevEntry *ents, bool reset,
                             hipStream_t st);
// FP8 copy-in (scales: one fp32 per parameter) and copy-out
hipError_t launch_pack_fp8(const PackTile *tiles, int64_t n, const DevEntry *ents, uint8_t *ag_in,
                           const float *scales, hipStream_t st);
hipError_t launch_unpack_fp8(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                             const uint8_t *ag_out, bool chunk_aligned, hipStream_t st);
// per-parameter amax of the master shards into amax[0 .. n_params)
hipError_t launch_amax(const EwTile *tiles, int64_t n, const DevEntry *ents, float *amax,
                       int32_t n_params, hipStream_t st);
// reduce-scatter copy-in from the fp32 accumulators
hipError_t launch_rspack_acc(const PackTile *tiles, int64_t n, const DevEntry *ents, float *out,
                             bool chunk_aligned, hipStream_t st);
// resharding: runs of 2-byte units between absolute addresses
hipError_t launch_copy_runs(const CopyTile *tiles, int64_t n, hipStream_t st);

}  // namespace fsdp
