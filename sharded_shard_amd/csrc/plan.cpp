// Shard-layout planner: host only, no HIP calls.
//
// Layout rules ("Sharded Training: FSDP2, DTensor, Tensor and Pipeline
// Parallelism", fully_shard paragraph and lab commentary):
//  * rank j owns rows [min(j*c, rows), min((j+1)*c, rows)) with
//    c = ceil(rows / N), the chunks of torch.chunk(param, N, dim=0); ranks
//    past the last chunk own nothing (a (1, 32) head leaves rank 1 empty);
//  * every rank's piece is padded to c*cols elements ("padded internally");
//  * one group's pieces are concatenated in registration order into one
//    segment; a piece starts at a multiple of align_elems (1 or 8).
#include "plan.hpp"

#include <algorithm>
#include <limits>

namespace fsdp {

int64_t chunk_rows(int64_t rows, int32_t world) {
    if (rows <= 0) return 0;
    return (rows + world - 1) / world;
}

void rows_of_rank(int64_t rows, int32_t world, int32_t j, int64_t *begin,
                  int64_t *local) {
    const int64_t c = chunk_rows(rows, world);
    const int64_t b = std::min<int64_t>(static_cast<int64_t>(j) * c, rows);
    const int64_t e = std::min<int64_t>(static_cast<int64_t>(j + 1) * c, rows);
    *begin = b;
    *local = e - b;
}

namespace {

constexpr int64_t kMaxElems = std::numeric_limits<int64_t>::max() / 8;

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a != 0 && b > kMaxElems / a) return false;
    *out = a * b;
    return true;
}

// Destination elements per alignment unit of the tiles that write [N, S]
// rows: 128 bytes of bf16, 256 of fp32, whole cache lines either way.
constexpr int64_t kLineElems = 64;

// Calls f(t, len) for the tiles of a run of n elements whose destination
// starts at element d0 of a 256-byte aligned buffer: at most `tile` elements
// each, the first shortened so that every later tile, and every block's
// sub-range in it (sub-ranges divide the tile), starts on a kLineElems
// boundary of the destination.  Outside a run's first tile, blocks then
// never share a destination line (measured on the ragged MoE rows: the
// reduce-scatter copy-ins 4-6% faster than with tiles cut from the run's
// start).
template <typename F>
void for_line_tiles(int64_t n, int64_t tile, int64_t d0, F &&f) {
    const int64_t ph = d0 % kLineElems;
    for (int64_t t = 0; t < n;) {
        const int64_t len = std::min((t == 0 && ph != 0) ? tile - ph : tile, n - t);
        f(t, len);
        t += len;
    }
}

}  // namespace

fsdp_status build_layout(const int64_t *rows, const int64_t *cols, int32_t n,
                         int32_t world, int32_t rank, int32_t align, Layout *out,
                         std::string *err) {
    if (n < 0 || (n > 0 && (rows == nullptr || cols == nullptr))) {
        *err = "rows/cols: null array or negative n_params";
        return FSDP_E_INVAL;
    }
    if (world < 1) {
        *err = "world must be >= 1";
        return FSDP_E_INVAL;
    }
    if (rank < 0 || rank >= world) {
        *err = "rank must be in [0, world)";
        return FSDP_E_INVAL;
    }
    if (align != 1 && align != 8) {
        *err = "align_elems must be 1 or 8";
        return FSDP_E_UNSUPPORTED;
    }
    Layout L;
    L.world = world;
    L.rank = rank;
    L.align = align;
    L.entries.resize(static_cast<size_t>(n));
    int64_t off = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t r = rows[i], c = cols[i];
        if (r < 0 || c < 1) {
            *err = "parameter " + std::to_string(i) + ": rows must be >= 0 and cols >= 1";
            return FSDP_E_INVAL;
        }
        int64_t full = 0;
        if (!mul_ok(r, c, &full)) {
            *err = "parameter " + std::to_string(i) + ": rows * cols overflows";
            return FSDP_E_INVAL;
        }
        fsdp_shard_entry_t &e = L.entries[i];
        e.rows = r;
        e.cols = c;
        e.chunk_rows = chunk_rows(r, world);
        rows_of_rank(r, world, rank, &e.row_begin, &e.local_rows);
        e.shard_offset = off;
        e.shard_numel = e.chunk_rows * c;
        e.valid_numel = e.local_rows * c;
        e.pad_numel = e.shard_numel - e.valid_numel;
        e.seg_numel = (e.shard_numel + align - 1) / align * align;
        if (e.seg_numel > kMaxElems - off) {
            *err = "segment length overflows";
            return FSDP_E_INVAL;
        }
        off += e.seg_numel;
        L.V += e.valid_numel;
        L.F += full;
        if (e.local_rows == 0) ++L.n_empty;
    }
    L.S = off;
    L.offsets8 = (L.S % 8) == 0;
    for (const fsdp_shard_entry_t &e : L.entries)
        if (e.shard_offset % 8 != 0) L.offsets8 = false;

    // Tiles.  Every run below is split into pieces of at most kTile* elements.
    for (int32_t i = 0; i < n; ++i) {
        const fsdp_shard_entry_t &e = L.entries[i];
        // copy-in covers the whole segment slot: valid values, then zeros.
        for (int64_t t = 0; t < e.seg_numel; t += kTilePack) {
            PackTile pt{};
            pt.dst = e.shard_offset + t;
            pt.src = t;
            pt.entry = i;
            pt.len = static_cast<int32_t>(std::min(kTilePack, e.seg_numel - t));
            pt.valid = static_cast<int32_t>(
                std::max<int64_t>(0, std::min<int64_t>(pt.len, e.valid_numel - t)));
            L.pack.push_back(pt);
        }
        // reduce-scatter copy-in: rank j's segment slot of this parameter in
        // row j, chunk j's rows first, then zeros (the mirror of copy-out).
        for (int32_t j = 0; j < world; ++j) {
            int64_t b = 0, lr = 0;
            rows_of_rank(e.rows, world, j, &b, &lr);
            const int64_t valid = lr * e.cols;
            const int64_t d0 = static_cast<int64_t>(j) * L.S + e.shard_offset;
            for_line_tiles(e.seg_numel, kTileUnpack, d0, [&](int64_t t, int64_t len) {
                PackTile rt{};
                rt.dst = d0 + t;
                rt.src = b * e.cols + t;
                rt.entry = i;
                rt.len = static_cast<int32_t>(len);
                rt.valid = static_cast<int32_t>(
                    std::max<int64_t>(0, std::min<int64_t>(len, valid - t)));
                L.rspack.push_back(rt);
            });
        }
        // copy-out: one run per source rank j, rows of chunk j.
        for (int32_t j = 0; j < world; ++j) {
            int64_t b = 0, lr = 0;
            rows_of_rank(e.rows, world, j, &b, &lr);
            const int64_t len = lr * e.cols;
            const int64_t src = static_cast<int64_t>(j) * L.S + e.shard_offset;
            for (int64_t t = 0; t < len; t += kTileUnpack) {
                UnpackTile ut{};
                ut.src = src + t;
                ut.dst = b * e.cols + t;
                ut.entry = i;
                ut.len = static_cast<int32_t>(std::min(kTileUnpack, len - t));
                L.unpack.push_back(ut);
            }
        }
        // reduce and AdamW: this rank's valid elements only.
        for (int64_t t = 0; t < e.valid_numel; t += kTileReduce) {
            ReduceTile rt{};
            rt.src = e.shard_offset + t;
            rt.dst = t;
            rt.entry = i;
            rt.len = static_cast<int32_t>(std::min(kTileReduce, e.valid_numel - t));
            L.reduce.push_back(rt);
        }
        for (int64_t t = 0; t < e.valid_numel; t += kTileAdamw) {
            EwTile at{};
            at.off = t;
            at.entry = i;
            at.len = static_cast<int32_t>(std::min(kTileAdamw, e.valid_numel - t));
            L.adamw.push_back(at);
        }
        // gradient accumulation: every element of the unsharded parameter
        const int64_t numel = e.rows * e.cols;
        for (int64_t t = 0; t < numel; t += kTileAdamw) {
            EwTile ft{};
            ft.off = t;
            ft.entry = i;
            ft.len = static_cast<int32_t>(std::min(kTileAdamw, numel - t));
            L.full.push_back(ft);
        }
    }
    *out = std::move(L);
    return FSDP_OK;
}

}  // namespace fsdp
