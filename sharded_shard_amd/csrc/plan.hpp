// Internal structures of the shard-layout planner and the device work tables.
//
// Shard(0) layout ("Sharded Training: FSDP2, DTensor, Tensor and Pipeline
// Parallelism", fully_shard paragraph): rank r keeps chunk r of
// torch.chunk(param, N, dim=0), each rank's piece padded to c = ceil(rows/N)
// rows; one group's pieces sit back to back in registration order and form
// one communication segment of S elements per rank.
//
// The planner cuts every kernel's iteration space into tiles of at most
// kTile* elements, so that workgroups get balanced work no matter how ragged
// the parameter sizes are (1 element to tens of millions) and no kernel ever
// searches for its parameter: a workgroup reads one 16- or 32-byte tile
// record and one entry record.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/fsdp_shard.h"

namespace fsdp {

// Tile lengths in elements, multiples of every sub-range length.  Tiles of a
// run follow its start, except the reduce-scatter copy-in's, which follow
// its destination's cache lines (plan.cpp); kernels take each sub-range's
// alignment from its addresses.
#ifndef FSDP_TILE_PACK
#define FSDP_TILE_PACK 16384
#endif
#ifndef FSDP_TILE_UNPACK
#define FSDP_TILE_UNPACK 32768
#endif
#ifndef FSDP_TILE_REDUCE
#define FSDP_TILE_REDUCE 4096
#endif
#ifndef FSDP_TILE_ADAMW
#define FSDP_TILE_ADAMW 8192
#endif
constexpr int64_t kTilePack = FSDP_TILE_PACK;
constexpr int64_t kTileUnpack = FSDP_TILE_UNPACK;
constexpr int64_t kTileReduce = FSDP_TILE_REDUCE;
constexpr int64_t kTileAdamw = FSDP_TILE_ADAMW;

// Device-side per-parameter record (64 bytes): the bound tensors.
struct DevEntry {
    float *master;
    float *grad;
    float *exp_avg;
    float *exp_avg_sq;
    uint16_t *full;
    uint8_t *full_fp8;     // unsharded FP8 E4M3 parameter (FP8 copy-out)
    uint16_t *full_grad;   // unsharded bf16 gradient (reduce-scatter copy-in)
    float *grad_acc;       // unsharded fp32 gradient accumulator
};
static_assert(sizeof(DevEntry) == 64, "DevEntry layout");

// copy-in: ag_in[dst .. dst+len) <- bf16(master[src .. src+valid)), then zeros.
struct PackTile {
    int64_t dst;
    int64_t src;
    int32_t entry;
    int32_t len;
    int32_t valid;
    int32_t rsv;
};
static_assert(sizeof(PackTile) == 32, "PackTile layout");

// copy-out: full[dst .. dst+len) <- ag_out[src .. src+len) (src counts rows*S).
struct UnpackTile {
    int64_t src;
    int64_t dst;
    int32_t entry;
    int32_t len;
    int64_t rsv;
};
static_assert(sizeof(UnpackTile) == 32, "UnpackTile layout");

// reduce: grad[dst .. dst+len) <- mean over rows j of rs_in[j*S + src ...].
struct ReduceTile {
    int64_t src;
    int64_t dst;
    int32_t entry;
    int32_t len;
    int64_t rsv;
};
static_assert(sizeof(ReduceTile) == 32, "ReduceTile layout");

// Generic copy of 2-byte units between absolute device addresses (resharding).
struct CopyTile {
    const uint16_t *src;
    uint16_t *dst;
    int64_t len;
    int64_t rsv;
};
static_assert(sizeof(CopyTile) == 32, "CopyTile layout");

// AdamW: elements [off .. off+len) of one parameter's shards.
struct EwTile {
    int64_t off;
    int32_t entry;
    int32_t len;
};
static_assert(sizeof(EwTile) == 16, "EwTile layout");

struct Layout {
    int32_t world = 0, rank = 0, align = 1;
    std::vector<fsdp_shard_entry_t> entries;
    int64_t S = 0, V = 0, F = 0;
    int32_t n_empty = 0;
    // S and every shard_offset are multiples of 8 elements: with a 16-byte
    // aligned [N, S] buffer every piece of every row starts 16-byte aligned
    bool offsets8 = true;
    std::vector<PackTile> pack;
    std::vector<PackTile> rspack;     // reduce-scatter copy-in: dst counts rows*S
    std::vector<UnpackTile> unpack;
    std::vector<ReduceTile> reduce;
    std::vector<EwTile> adamw;
    std::vector<EwTile> full;         // every element of the unsharded parameters
};

// ceil(rows / world) and rank j's [row_begin, row_begin + local_rows).
int64_t chunk_rows(int64_t rows, int32_t world);
void rows_of_rank(int64_t rows, int32_t world, int32_t j, int64_t *begin,
                  int64_t *local);

// Builds entries and tiles.  Returns FSDP_OK or an error with `err` set.
fsdp_status build_layout(const int64_t *rows, const int64_t *cols, int32_t n,
                         int32_t world, int32_t rank, int32_t align, Layout *out,
                         std::string *err);

}  // namespace fsdp
