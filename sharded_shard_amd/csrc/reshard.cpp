// Reshard planner and executor: load Shard(0) shards saved by world_src ranks
// into rank rank_dst of world_dst ranks.
//
// "Sharded Training: FSDP2, DTensor, Tensor and Pipeline Parallelism",
// distributed checkpoint paragraph: a checkpoint keeps every rank's chunks
// with their offsets in the global tensor, and a loading rank reads only the
// chunks that overlap its target placement, so changing the world size is
// planning, not conversion.  The planner intersects the source and target
// row ranges of every parameter (both torch.chunk layouts); the executor
// copies the overlaps with one launch over a tile table built at bind time.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/fsdp_shard.h"
#include "launch.hpp"
#include "plan.hpp"

namespace fsdp {
fsdp_status set_error(fsdp_status s, const std::string &msg);
fsdp_status set_hip_error(hipError_t e, const char *what);
hipError_t injected_fault();
}  // namespace fsdp

struct fsdp_reshard_plan {
    int32_t n_params = 0, world_src = 0, world_dst = 0, rank_dst = 0;
    std::vector<int64_t> rows, cols;
    std::vector<fsdp_reshard_run_t> runs;
    int64_t dst_numel = 0;
    std::vector<fsdp::CopyTile> tiles;
    fsdp::CopyTile *d_tiles = nullptr;
    size_t d_cap = 0;
    int device = -1;
    bool bound = false;
};

namespace {

using fsdp::set_error;

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

}  // namespace

extern "C" {

fsdp_status fsdp_reshard_plan_create(const int64_t *rows, const int64_t *cols, int32_t n_params,
                                     int32_t world_src, int32_t world_dst, int32_t rank_dst,
                                     fsdp_reshard_plan **out) {
    if (out == nullptr) return set_error(FSDP_E_INVAL, "fsdp_reshard_plan_create: null out");
    *out = nullptr;
    if (n_params < 0 || (n_params > 0 && (rows == nullptr || cols == nullptr)))
        return set_error(FSDP_E_INVAL, "fsdp_reshard_plan_create: null arrays or negative n_params");
    if (world_src < 1 || world_dst < 1 || rank_dst < 0 || rank_dst >= world_dst)
        return set_error(FSDP_E_INVAL,
                         "fsdp_reshard_plan_create: need world sizes >= 1 and rank_dst in [0, world_dst)");
    try {
        fsdp_reshard_plan *p = new fsdp_reshard_plan();
        p->n_params = n_params;
        p->world_src = world_src;
        p->world_dst = world_dst;
        p->rank_dst = rank_dst;
        for (int32_t i = 0; i < n_params; ++i) {
            if (rows[i] < 0 || cols[i] < 1 || (rows[i] > 0 && cols[i] > (INT64_MAX / 8) / rows[i])) {
                delete p;
                return set_error(FSDP_E_INVAL, "fsdp_reshard_plan_create: parameter " +
                                                   std::to_string(i) + ": bad rows or cols");
            }
            p->rows.push_back(rows[i]);
            p->cols.push_back(cols[i]);
            int64_t b2 = 0, l2 = 0;
            fsdp::rows_of_rank(rows[i], world_dst, rank_dst, &b2, &l2);
            p->dst_numel += l2 * cols[i];
            for (int32_t s = 0; s < world_src; ++s) {
                int64_t b1 = 0, l1 = 0;
                fsdp::rows_of_rank(rows[i], world_src, s, &b1, &l1);
                const int64_t lo = std::max(b1, b2), hi = std::min(b1 + l1, b2 + l2);
                if (hi <= lo) continue;
                fsdp_reshard_run_t r{};
                r.param = i;
                r.src_rank = s;
                r.src_offset = (lo - b1) * cols[i];
                r.dst_offset = (lo - b2) * cols[i];
                r.numel = (hi - lo) * cols[i];
                p->runs.push_back(r);
            }
        }
        *out = p;
        return FSDP_OK;
    } catch (...) {
        return set_error(FSDP_E_NOMEM, "fsdp_reshard_plan_create: host allocation failed");
    }
}

fsdp_status fsdp_reshard_plan_runs(const fsdp_reshard_plan *p, int64_t *n_runs, int64_t *dst_numel) {
    if (p == nullptr || n_runs == nullptr || dst_numel == nullptr)
        return set_error(FSDP_E_INVAL, "fsdp_reshard_plan_runs: null argument");
    *n_runs = static_cast<int64_t>(p->runs.size());
    *dst_numel = p->dst_numel;
    return FSDP_OK;
}

fsdp_status fsdp_reshard_plan_run(const fsdp_reshard_plan *p, int64_t i, fsdp_reshard_run_t *out) {
    if (p == nullptr || out == nullptr) return set_error(FSDP_E_INVAL, "fsdp_reshard_plan_run: null argument");
    if (i < 0 || i >= static_cast<int64_t>(p->runs.size()))
        return set_error(FSDP_E_INVAL, "fsdp_reshard_plan_run: index out of range");
    *out = p->runs[static_cast<size_t>(i)];
    return FSDP_OK;
}

fsdp_status fsdp_reshard_bind(fsdp_reshard_plan *p, const void *const *src, void *const *dst,
                              int32_t elem_bytes, void *stream) {
    if (p == nullptr || (p->n_params > 0 && (src == nullptr || dst == nullptr)))
        return set_error(FSDP_E_INVAL, "fsdp_reshard_bind: null plan or array");
    if (elem_bytes != 2 && elem_bytes != 4)
        return set_error(FSDP_E_UNSUPPORTED, "fsdp_reshard_bind: elem_bytes must be 2 or 4");
    std::vector<fsdp::CopyTile> tiles;
    const int64_t units = elem_bytes / 2;   // copies move 2-byte units
    for (const fsdp_reshard_run_t &r : p->runs) {
        const void *s = src[static_cast<size_t>(r.param) * p->world_src + r.src_rank];
        void *d = dst[r.param];
        if (s == nullptr || d == nullptr)
            return set_error(FSDP_E_INVAL, "fsdp_reshard_bind: null shard pointer of parameter " +
                                               std::to_string(r.param));
        if (misaligned(s, elem_bytes) || misaligned(d, elem_bytes))
            return set_error(FSDP_E_ALIGN, "fsdp_reshard_bind: shard pointer of parameter " +
                                               std::to_string(r.param) + " misaligned");
        const int64_t len = r.numel * units;
        for (int64_t t = 0; t < len; t += fsdp::kTileUnpack) {
            fsdp::CopyTile ct{};
            ct.src = static_cast<const uint16_t *>(s) + r.src_offset * units + t;
            ct.dst = static_cast<uint16_t *>(d) + r.dst_offset * units + t;
            ct.len = std::min<int64_t>(fsdp::kTileUnpack, len - t);
            tiles.push_back(ct);
        }
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(FSDP_E_HIP, std::string("fsdp_reshard_bind: ") + hipGetErrorString(e));
    hipStream_t st = static_cast<hipStream_t>(stream);
    e = hipStreamSynchronize(st);   // queued executions may still read the old table
    if (e != hipSuccess) return set_error(FSDP_E_HIP, std::string("fsdp_reshard_bind: ") + hipGetErrorString(e));
    const size_t bytes = tiles.size() * sizeof(fsdp::CopyTile);
    // From here the device table is being replaced: until the upload below
    // succeeds the plan is unbound, so a failed bind cannot leave a stale or
    // freed table behind for fsdp_reshard_execute.
    p->bound = false;
    p->tiles.clear();
    if (p->d_tiles != nullptr && (bytes > p->d_cap || dev != p->device)) {
        (void)hipFree(p->d_tiles);
        p->d_tiles = nullptr;
        p->d_cap = 0;
    }
    if (p->d_tiles == nullptr && bytes > 0) {
        void *mem = nullptr;
        if (hipMalloc(&mem, bytes) != hipSuccess)
            return set_error(FSDP_E_NOMEM, "fsdp_reshard_bind: hipMalloc of the tile table failed");
        p->d_tiles = static_cast<fsdp::CopyTile *>(mem);
        p->d_cap = bytes;
    }
    p->device = dev;
    if (bytes > 0) {
        e = hipMemcpyAsync(p->d_tiles, tiles.data(), bytes, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return set_error(FSDP_E_HIP, std::string("fsdp_reshard_bind: ") + hipGetErrorString(e));
    }
    p->tiles = std::move(tiles);
    p->bound = true;
    return FSDP_OK;
}

fsdp_status fsdp_reshard_execute(const fsdp_reshard_plan *p, void *stream) {
    if (p == nullptr) return set_error(FSDP_E_INVAL, "fsdp_reshard_execute: null plan");
    if (!p->bound) return set_error(FSDP_E_STATE, "fsdp_reshard_execute: plan not bound");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(FSDP_E_HIP, std::string("fsdp_reshard_execute: ") + hipGetErrorString(e));
    if (dev != p->device) return set_error(FSDP_E_STATE, "fsdp_reshard_execute: wrong device");
    e = fsdp::injected_fault();
    if (e == hipSuccess)
        e = fsdp::launch_copy_runs(p->d_tiles, static_cast<int64_t>(p->tiles.size()),
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fsdp::set_hip_error(e, "fsdp_reshard_execute");
    return FSDP_OK;
}

void fsdp_reshard_plan_destroy(fsdp_reshard_plan *p) {
    if (p == nullptr) return;
    if (p->d_tiles != nullptr) {
        (void)hipDeviceSynchronize();
        (void)hipFree(p->d_tiles);
    }
    delete p;
}

}  // extern "C"
