// Stand-ins for the library's kernel launchers, for the host sanitizer build.
// Each one walks the tile table the host code uploaded and reads the first
// and last element of every range a kernel would read or write (through the
// bound entry pointers and the caller's buffers), so AddressSanitizer reports
// any tile that reaches outside its allocation; every written range is also
// recorded for the harness, which checks that the writes cover each output
// exactly once.  No kernel arithmetic is reproduced here.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <vector>

#include "../../sharded_shard_amd/csrc/launch.hpp"
#include "../../sharded_shard_amd/csrc/plan.hpp"
#include "harness.hpp"

namespace harness {
std::vector<Span> spans;
long launches = 0;
}  // namespace harness

namespace {

template <typename T>
void touch(const T *base, int64_t off, int64_t len) {
    if (len <= 0) return;
    volatile T a = base[off];
    volatile T b = base[off + len - 1];
    (void)a;
    (void)b;
}

template <typename T>
void wrote(const T *base, int64_t off, int64_t len, int kind) {
    touch(base, off, len);
    if (len > 0) harness::spans.push_back({static_cast<const void *>(base), off, len, kind});
}

}  // namespace

namespace fsdp {

hipError_t launch_pack(const PackTile *tiles, int64_t n, const DevEntry *ents, uint16_t *ag_in,
                       hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const PackTile &t = tiles[i];
        touch(ents[t.entry].master, t.src, t.valid);
        wrote(ag_in, t.dst, t.len, harness::kSegment);
    }
    return hipSuccess;
}

hipError_t launch_unpack(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *ag_out, bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const UnpackTile &t = tiles[i];
        touch(ag_out, t.src, t.len);
        wrote(ents[t.entry].full, t.dst, t.len, harness::kFull);
    }
    return hipSuccess;
}

namespace {
template <typename R>
void rows(const R *rs_in, int64_t S, int32_t N, int64_t off, int64_t len) {
    for (int32_t j = 0; j < N; ++j) touch(rs_in, static_cast<int64_t>(j) * S + off, len);
}
}  // namespace

hipError_t launch_reduce(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *rs_in, int64_t S, int32_t N, bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const ReduceTile &t = tiles[i];
        rows(rs_in, S, N, t.src, t.len);
        wrote(ents[t.entry].grad, t.dst, t.len, harness::kShard);
    }
    return hipSuccess;
}

hipError_t launch_adamw_pack(const PackTile *tiles, int64_t n, const DevEntry *ents,
                             uint16_t *ag_in, const float *, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const PackTile &t = tiles[i];
        const DevEntry &e = ents[t.entry];
        touch(e.grad, t.src, t.valid);
        touch(e.exp_avg, t.src, t.valid);
        touch(e.exp_avg_sq, t.src, t.valid);
        wrote(e.master, t.src, t.valid, harness::kShard);
        wrote(ag_in, t.dst, t.len, harness::kSegment);
    }
    return hipSuccess;
}

hipError_t launch_adamw(const EwTile *tiles, int64_t n, const DevEntry *ents, const float *,
                        bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const EwTile &t = tiles[i];
        const DevEntry &e = ents[t.entry];
        touch(e.grad, t.off, t.len);
        touch(e.exp_avg, t.off, t.len);
        touch(e.exp_avg_sq, t.off, t.len);
        wrote(e.master, t.off, t.len, harness::kShard);
    }
    return hipSuccess;
}

hipError_t launch_step(const PackTile *tiles, int64_t n, const DevEntry *ents,
                       const uint16_t *rs_in, uint16_t *ag_in, int64_t S, int32_t N,
                       const float *, bool write_grad, bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const PackTile &t = tiles[i];
        const DevEntry &e = ents[t.entry];
        rows(rs_in, S, N, t.dst, t.valid);
        touch(e.exp_avg, t.src, t.valid);
        touch(e.exp_avg_sq, t.src, t.valid);
        if (write_grad) touch(e.grad, t.src, t.valid);
        wrote(e.master, t.src, t.valid, harness::kShard);
        wrote(ag_in, t.dst, t.len, harness::kSegment);
    }
    return hipSuccess;
}

hipError_t launch_rspack(const PackTile *tiles, int64_t n, const DevEntry *ents, void *out,
                         bool f32, bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const PackTile &t = tiles[i];
        touch(ents[t.entry].full_grad, t.src, t.valid);
        if (f32) wrote(static_cast<const float *>(out), t.dst, t.len, harness::kRows);
        else wrote(static_cast<const uint16_t *>(out), t.dst, t.len, harness::kRows);
    }
    return hipSuccess;
}

hipError_t launch_reduce_f32(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                             const float *rs_in, int64_t S, int32_t N, bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const ReduceTile &t = tiles[i];
        rows(rs_in, S, N, t.src, t.len);
        wrote(ents[t.entry].grad, t.dst, t.len, harness::kShard);
    }
    return hipSuccess;
}

hipError_t launch_accumulate(const EwTile *tiles, int64_t n, const DevEntry *ents, bool,
                             hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const EwTile &t = tiles[i];
        touch(ents[t.entry].full_grad, t.off, t.len);
        wrote(ents[t.entry].grad_acc, t.off, t.len, harness::kFull);
    }
    return hipSuccess;
}

hipError_t launch_pack_fp8(const PackTile *tiles, int64_t n, const DevEntry *ents, uint8_t *ag_in,
                           const float *scales, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const PackTile &t = tiles[i];
        touch(scales, t.entry, 1);
        touch(ents[t.entry].master, t.src, t.valid);
        wrote(ag_in, t.dst, t.len, harness::kSegment);
    }
    return hipSuccess;
}

hipError_t launch_unpack_fp8(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                             const uint8_t *ag_out, bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const UnpackTile &t = tiles[i];
        touch(ag_out, t.src, t.len);
        wrote(ents[t.entry].full_fp8, t.dst, t.len, harness::kFull);
    }
    return hipSuccess;
}

hipError_t launch_amax(const EwTile *tiles, int64_t n, const DevEntry *ents, float *amax,
                       int32_t n_params, hipStream_t) {
    ++harness::launches;
    wrote(amax, 0, n_params, harness::kSmall);
    for (int64_t i = 0; i < n; ++i) {
        touch(amax, tiles[i].entry, 1);
        touch(ents[tiles[i].entry].master, tiles[i].off, tiles[i].len);
    }
    return hipSuccess;
}

hipError_t launch_rspack_acc(const PackTile *tiles, int64_t n, const DevEntry *ents, float *out,
                             bool, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        const PackTile &t = tiles[i];
        touch(ents[t.entry].grad_acc, t.src, t.valid);
        wrote(out, t.dst, t.len, harness::kRows);
    }
    return hipSuccess;
}

hipError_t launch_copy_runs(const CopyTile *tiles, int64_t n, hipStream_t) {
    ++harness::launches;
    for (int64_t i = 0; i < n; ++i) {
        touch(tiles[i].src, 0, tiles[i].len);
        wrote(tiles[i].dst, 0, tiles[i].len, harness::kReshard);
    }
    return hipSuccess;
}

}  // namespace fsdp
