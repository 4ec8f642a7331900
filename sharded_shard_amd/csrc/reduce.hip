// Local reductions of the reduce-scatter: N bf16 or fp32 gradient
// contributions summed in fp32 in rank order, then one correctly rounded
// division by N; and gradient accumulation without sync (fp32 += bf16).
#include "launch.hpp"
#include "rows.hpp"

// the bf16 reduction's wide variant: non-temporal loads
#ifndef FSDP_REDUCE_POL
#define FSDP_REDUCE_POL 1
#endif
// the bf16 reduction below the wide threshold, aligned or misaligned rows:
// a quad per lane, non-temporal loads and stores (on the ragged MoE rows
// 5.0 TB/s, against 4.1 for 63 groups of 8 per wave)
#ifndef FSDP_REDUCE_QUAD_POL
#define FSDP_REDUCE_QUAD_POL 3
#endif
// the fp32 reduction: a vector per lane, so every wave instruction is
// contiguous (lanes storing two 16-byte halves of a 32-byte span, an earlier
// layout, made non-temporal stores cost 1.1-1.7x the algorithmic bytes), and
// non-temporal loads and stores (on the ragged MoE rows 6.2 TB/s, against
// 5.5 for that layout with plain ones)
#ifndef FSDP_REDUCE_F32_POL
#define FSDP_REDUCE_F32_POL 3
#endif
// rows in flight per lane of the fp32 reduction on misaligned rows (2:
// 6.34-6.42 TB/s on the ragged MoE rows against 5.77-6.13 with 1; the bf16
// reduction there keeps 1, 2 measured 2% slower) and on aligned rows (1:
// 2 and 4 measured 1% and 0.5% slower at 8 ranks, 4% and 8% at 64)
#ifndef FSDP_REDUCE_F32_MIS_ROW_BATCH
#define FSDP_REDUCE_F32_MIS_ROW_BATCH 2
#endif
#ifndef FSDP_REDUCE_F32_ROW_BATCH
#define FSDP_REDUCE_F32_ROW_BATCH 1
#endif
// the fp32 reduction on aligned rows below this many ranks: one vector per
// lane over half its rows budget (1024 elements per block at 8 ranks, 3.5-5%
// faster than two vectors per lane over 2048); from it on, and on misaligned
// rows, two vectors per lane (at 64 ranks 1.3% faster than one, on the ragged
// MoE rows 8%)
#ifndef FSDP_REDUCE_F32_PAIR_MIN_N
#define FSDP_REDUCE_F32_PAIR_MIN_N 16
#endif
// gradient accumulation: non-temporal loads and stores
#ifndef FSDP_ACC_POL
#define FSDP_ACC_POL 3
#endif
// Groups per lane of the bf16 reduction's wide variant, used on aligned rows
// from FSDP_REDUCE_WIDE_MIN_N ranks (fp32 contributions measured slower read
// this way: 5.65 vs 5.87 TB/s at N = 64, so their reduction has none).
#ifndef FSDP_REDUCE_WIDE
#define FSDP_REDUCE_WIDE 4
#endif
#ifndef FSDP_REDUCE_WIDE_MIN_N
#define FSDP_REDUCE_WIDE_MIN_N 16
#endif

namespace fsdp {

namespace {

// ---------------------------------------------------------------------------
// reduce: [N, S] bf16 contributions -> fp32 mean, this rank's pieces
// ---------------------------------------------------------------------------

// Valid elements [0, len) of one run.  One or two rows in flight per lane
// (C == 1): a quad per lane and pass, two passes 64 quads apart, so every
// wave instruction is contiguous and loads and stores take
// FSDP_REDUCE_QUAD_POL; misaligned rows are funnel-shifted by their own
// phase (sum_rows_quad_mis).  The wide variant (C > 1, 16-byte aligned rows
// only) takes C groups of 8 per lane, row by row (sum_rows_wide).
template <int POL, int C, bool kChunkAligned>
__device__ __forceinline__ void reduce_run(float *__restrict__ dst, const uint16_t *__restrict__ src0,
                                           int64_t len, int64_t S, int32_t N, float fN) {
    static_assert(kChunkAligned || C == 1, "the wide variant needs aligned rows");
    const int tid = threadIdx.x;
    const uint32_t kS = static_cast<uint32_t>((S * 2) & 15);
    int64_t head = ((16u - (lo32(dst) & 15u)) & 15u) >> 2;
    if (head > len) head = len;
    const uint16_t *s0 = src0 + head;
    const uint32_t k0 = lo32(s0) & 15u;
    if (kChunkAligned && (k0 | kS) != 0) {
        // the launch assumed aligned rows; this run is not: element by element
        for (int64_t e = tid; e < len; e += static_cast<int64_t>(blockDim.x))
            dst[e] = sum_rows_scalar(src0, S, N, e) / fN;
        return;
    }
    if (tid < head) dst[tid] = sum_rows_scalar(src0, S, N, tid) / fN;
    const uint32_t dbytes = static_cast<uint32_t>(2 * (len - head));
    f32x4 *dv = reinterpret_cast<f32x4 *>(dst + head);
    if constexpr (C == 1) {
        constexpr int QL = FSDP_REDUCE_QUAD_POL & 1, QS = (FSDP_REDUCE_QUAD_POL >> 1) & 1;
        const int64_t nq = (len - head) >> 2;
        const int64_t lane = tid & 63;
        const int64_t qstep = static_cast<int64_t>(blockDim.x >> 6) * 128;
        for (int64_t qb = (tid >> 6) * 128; qb < nq; qb += qstep) {
            const uint32_t off = static_cast<uint32_t>(qb + lane) << 3;
            float acc[2][4];
            if constexpr (kChunkAligned)
                sum_rows_quad<QL, FSDP_REDUCE_ROW_BATCH, 2>(s0, off, dbytes, S, N, acc);
            else
                sum_rows_quad_mis<QL, FSDP_REDUCE_MIS_ROW_BATCH>(s0, off, dbytes, S, N, k0 & 7u,
                                                                 kS & 7u, acc);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t q = qb + lane + 64 * h;
                if (q < nq)
                    stp<QS>(dv + q, f32x4{acc[h][0] / fN, acc[h][1] / fN, acc[h][2] / fN,
                                          acc[h][3] / fN});
            }
        }
        const int64_t done = head + (nq << 2);
        if (tid < len - done) dst[done + tid] = sum_rows_scalar(src0, S, N, done + tid) / fN;
        return;
    } else {
        constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
        const int64_t ngrp = (len - head) >> 3;
        for (GroupWalk<C> w; w.more(ngrp); w.next()) {
            float acc[C][8];
            sum_rows_wide<LN, C>(s0, static_cast<uint32_t>(w.g) << 4, dbytes, S, N, acc);
#pragma unroll
            for (int q = 0; q < C; ++q) {
                if (!w.own(ngrp, q)) continue;
                const int64_t g = w.at(q);
                const float *a = acc[q];
                stp<SN>(dv + 2 * g, f32x4{a[0] / fN, a[1] / fN, a[2] / fN, a[3] / fN});
                stp<SN>(dv + 2 * g + 1, f32x4{a[4] / fN, a[5] / fN, a[6] / fN, a[7] / fN});
            }
        }
        const int64_t done = head + (ngrp << 3);
        if (tid < len - done) dst[done + tid] = sum_rows_scalar(src0, S, N, done + tid) / fN;
    }
}

template <int POL, int C, bool kChunkAligned>
__global__ __launch_bounds__(kBlock) void reduce_kernel(
    const ReduceTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ rs_in,
    int64_t S, int32_t N, float fN) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const ReduceTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        reduce_run<POL, C, kChunkAligned>(ents[tl.entry].grad + tl.dst + b, rs_in + tl.src + b,
                                          len, S, N, fN);
    }
}

// ---------------------------------------------------------------------------
// gradient accumulation without sync: fp32 acc <- acc + fp32(bf16 grad)
// ---------------------------------------------------------------------------

template <int POL, bool kReset>
__device__ __forceinline__ void accumulate_run(float *__restrict__ acc, const uint16_t *__restrict__ g,
                                               int64_t len) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = ((16u - (lo32(acc) & 15u)) & 15u) >> 2;
    if (head > len) head = len;
    const bool vec = (lo32(g + head) & 7u) == 0;   // 4 bf16 per 16 fp32 bytes
    if (!vec) head = len;
    for (int64_t i = tid; i < head; i += kBlock) acc[i] = kReset ? widen(g[i]) : acc[i] + widen(g[i]);
    if (!vec) return;
    const int64_t nvec = (len - head) >> 2;
    f32x4 *av = reinterpret_cast<f32x4 *>(acc + head);
    const u32x2 *gv = reinterpret_cast<const u32x2 *>(g + head);
    // one vector per lane in a sub-range of FSDP_ADAMW_SUB elements; longer
    // ones take two a block apart per iteration, both loaded before either is
    // stored (one per iteration measured 3-5% slower)
    int64_t v = tid;
    for (; v + kBlock < nvec; v += 2 * kBlock) {
        const int64_t v1 = v + kBlock;
        const u32x2 w0 = ldp<LN>(gv + v), w1 = ldp<LN>(gv + v1);
        const f32x4 x0{bf16_lo(w0.x), bf16_hi(w0.x), bf16_lo(w0.y), bf16_hi(w0.y)};
        const f32x4 x1{bf16_lo(w1.x), bf16_hi(w1.x), bf16_lo(w1.y), bf16_hi(w1.y)};
        if (kReset) {
            stp<SN>(av + v, x0);
            stp<SN>(av + v1, x1);
        } else {
            const f32x4 a0 = ldp<LN>(av + v), a1 = ldp<LN>(av + v1);
            stp<SN>(av + v, f32x4{a0.x + x0.x, a0.y + x0.y, a0.z + x0.z, a0.w + x0.w});
            stp<SN>(av + v1, f32x4{a1.x + x1.x, a1.y + x1.y, a1.z + x1.z, a1.w + x1.w});
        }
    }
    for (; v < nvec; v += kBlock) {
        const u32x2 w = ldp<LN>(gv + v);
        const f32x4 x{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
        if (kReset) {
            stp<SN>(av + v, x);
        } else {
            const f32x4 a = ldp<LN>(av + v);
            stp<SN>(av + v, f32x4{a.x + x.x, a.y + x.y, a.z + x.z, a.w + x.w});
        }
    }
    const int64_t e = head + (nvec << 2) + tid;
    if (e < len) acc[e] = kReset ? widen(g[e]) : acc[e] + widen(g[e]);
}

template <int POL, bool kReset>
__global__ __launch_bounds__(kBlock) void accumulate_kernel(const EwTile *__restrict__ tiles,
                                                            int64_t n_tiles, int32_t split,
                                                            int64_t sub,
                                                            const DevEntry *__restrict__ ents) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const EwTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        const DevEntry en = ents[tl.entry];
        accumulate_run<POL, kReset>(en.grad_acc + tl.off + b, en.full_grad + tl.off + b, len);
    }
}

// ---------------------------------------------------------------------------
// reduce of fp32 contributions: [N, S] fp32 -> fp32 mean, this rank's pieces
// ---------------------------------------------------------------------------

__device__ __forceinline__ float sum_rows_scalar_f32(const float *src0, int64_t S, int32_t N,
                                                     int64_t e) {
    float acc = src0[e];
    for (int32_t j = 1; j < N; ++j) acc = acc + src0[static_cast<int64_t>(j) * S + e];
    return acc;
}

// Valid elements [0, len) of one run: four elements (one vector) per lane
// and pass, H passes 64 vectors apart, so every wave instruction is
// contiguous and loads and stores take POL.  On misaligned rows (row j
// starts q_j = (q0 + j qS) & 3 dwords past a 16-byte boundary) lane l loads
// the aligned chunk holding its first element, takes the next chunk from
// lane l + 1 (DPP; lane 63 loads its own) and shifts by q_j dwords,
// FSDP_REDUCE_F32_MIS_ROW_BATCH rows at a time: every chunk of a row is
// read once.
template <int POL, bool kChunkAligned, int H>
__device__ __forceinline__ void reduce_f32_run(float *__restrict__ dst,
                                               const float *__restrict__ src0, int64_t len,
                                               int64_t S, int32_t N, float fN) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = ((16u - (lo32(dst) & 15u)) & 15u) >> 2;
    if (head > len) head = len;
    const float *s0 = src0 + head;
    const uint32_t q0 = (lo32(s0) >> 2) & 3u;
    const uint32_t qS = static_cast<uint32_t>(S & 3);
    if (kChunkAligned && (q0 | qS) != 0) {
        // the launch assumed aligned rows; this run is not: element by element
        for (int64_t e = tid; e < len; e += static_cast<int64_t>(blockDim.x))
            dst[e] = sum_rows_scalar_f32(src0, S, N, e) / fN;
        return;
    }
    if (tid < head) dst[tid] = sum_rows_scalar_f32(src0, S, N, tid) / fN;
    const uint32_t dbytes = static_cast<uint32_t>(4 * (len - head));
    f32x4 *dv = reinterpret_cast<f32x4 *>(dst + head);
    const char *r = reinterpret_cast<const char *>(s0);
    const int64_t Sb = S * 4;
    const int64_t nq = (len - head) >> 2;
    const int64_t lane = tid & 63;
    const bool last = lane == 63;
    const int64_t qstep = static_cast<int64_t>(blockDim.x >> 6) * 64 * H;
    for (int64_t qb = (tid >> 6) * 64 * H; qb < nq; qb += qstep) {
        const uint32_t off = static_cast<uint32_t>(qb + lane) << 4;
        f32x4 acc[H];
        if constexpr (kChunkAligned) {
            // whole batches, then the rest one row at a time (as sum_rows_quad)
            constexpr int RB = FSDP_REDUCE_F32_ROW_BATCH;
            const uint32_t nb = (dbytes + 15u) & ~15u;
            int32_t j = 0;
            for (; j + RB <= N; j += RB) {
                f32x4 x[RB][H];
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int h = 0; h < H; ++h)
                        x[i][h] = __builtin_bit_cast(
                            f32x4, bload16<LN>(r + (j + i) * Sb, off + 1024u * h, nb));
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int h = 0; h < H; ++h) {
                        const f32x4 y = x[i][h];
                        acc[h] = j + i == 0 ? y
                                            : f32x4{acc[h].x + y.x, acc[h].y + y.y,
                                                    acc[h].z + y.z, acc[h].w + y.w};
                    }
            }
            for (; j < N; ++j) {
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    const f32x4 y = __builtin_bit_cast(
                        f32x4, bload16<LN>(r + j * Sb, off + 1024u * h, nb));
                    acc[h] = j == 0 ? y
                                    : f32x4{acc[h].x + y.x, acc[h].y + y.y, acc[h].z + y.z,
                                            acc[h].w + y.w};
                }
            }
        } else {
            constexpr int RB = FSDP_REDUCE_F32_MIS_ROW_BATCH;
            for (int32_t j = 0; j < N; j += RB) {
                u32x4 a[RB][H], e[RB][H];
                uint32_t qq[RB];
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    // rows past N get an empty range: zeros, never added
                    qq[i] = (q0 + static_cast<uint32_t>(j + i) * qS) & 3u;
                    const char *al = r + (j + i) * Sb - 4 * qq[i];
                    const uint32_t n = j + i < N ? (4 * qq[i] + dbytes + 15u) & ~15u : 0u;
#pragma unroll
                    for (int h = 0; h < H; ++h) {
                        const uint32_t o = off + 1024u * h;
                        a[i][h] = bload16<LN>(al, o, n);
                        e[i][h] = bload16<kBoundaryNT>(al, last ? o + 16u : n, n);
                    }
                }
#pragma unroll
                for (int i = 0; i < RB; ++i) {
#pragma unroll
                    for (int h = 0; h < H; ++h) {
                        const u32x4 b = next_or_own(a[i][h], e[i][h]);
                        const f32x4 y = __builtin_bit_cast(f32x4, funnel(a[i][h], b, 4 * qq[i]));
                        if (j + i >= N) continue;
                        acc[h] = j + i == 0 ? y
                                            : f32x4{acc[h].x + y.x, acc[h].y + y.y,
                                                    acc[h].z + y.z, acc[h].w + y.w};
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int64_t q = qb + lane + 64 * h;
            if (q < nq)
                stp<SN>(dv + q, f32x4{acc[h].x / fN, acc[h].y / fN, acc[h].z / fN, acc[h].w / fN});
        }
    }
    const int64_t done = head + (nq << 2);
    if (tid < len - done) dst[done + tid] = sum_rows_scalar_f32(src0, S, N, done + tid) / fN;
}

template <int POL, bool kChunkAligned, int H>
__global__ __launch_bounds__(kBlock) void reduce_f32_kernel(
    const ReduceTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const float *__restrict__ rs_in, int64_t S, int32_t N,
    float fN) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const ReduceTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        reduce_f32_run<POL, kChunkAligned, H>(ents[tl.entry].grad + tl.dst + b, rs_in + tl.src + b,
                                          len, S, N, fN);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------

hipError_t launch_reduce(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *rs_in, int64_t S, int32_t N, bool chunk_aligned,
                         hipStream_t st) {
    if (n == 0) return hipSuccess;
    const float fN = static_cast<float>(N);
    if (chunk_aligned && N >= FSDP_REDUCE_WIDE_MIN_N) {
        // one wave per block, each block one sub-range of 64 * 8 * FSDP_REDUCE_WIDE elements
        constexpr int64_t wsub = 64 * 8 * FSDP_REDUCE_WIDE;
        static_assert(kTileReduce % wsub == 0, "wide sub-range must divide the tile");
        const int32_t wsp = static_cast<int32_t>(kTileReduce / wsub);
        reduce_kernel<FSDP_REDUCE_POL, FSDP_REDUCE_WIDE, true>
            <<<grid_for(n, wsp), 64, 0, st>>>(tiles, n, wsp, wsub, ents, rs_in, S, N, fN);
        return hipGetLastError();
    }
    // half the rows budget: one pass of two quads per lane at 8 ranks (2048
    // elements per block; the full budget measured 4% slower there and 7% on
    // the ragged MoE rows, a quarter 1-2%)
    const int32_t sp = split_rows(kTileReduce, 2 * N, 0);
    const unsigned grid = grid_for(n, sp);
    if (chunk_aligned)
        reduce_kernel<FSDP_REDUCE_POL, 1, true>
            <<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileReduce / sp, ents, rs_in, S, N, fN);
    else
        reduce_kernel<FSDP_REDUCE_POL, 1, false>
            <<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileReduce / sp, ents, rs_in, S, N, fN);
    return hipGetLastError();
}

hipError_t launch_accumulate(const EwTile *tiles, int64_t n, const DevEntry *ents, bool reset,
                             hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileAdamw, FSDP_ADAMW_SUB);
    const unsigned grid = grid_for(n, sp);
    if (reset)
        accumulate_kernel<FSDP_ACC_POL, true><<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileAdamw / sp, ents);
    else
        accumulate_kernel<FSDP_ACC_POL, false><<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileAdamw / sp, ents);
    return hipGetLastError();
}

hipError_t launch_reduce_f32(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                             const float *rs_in, int64_t S, int32_t N, bool chunk_aligned,
                             hipStream_t st) {
    if (n == 0) return hipSuccess;
    const float fN = static_cast<float>(N);
    // fp32 rows carry twice the bytes of bf16 rows per element; one vector
    // per lane takes half that budget again
    const bool one = chunk_aligned && N < FSDP_REDUCE_F32_PAIR_MIN_N;
    const int32_t sp = split_rows(kTileReduce, (one ? 4 : 2) * N, 0);
    const unsigned grid = grid_for(n, sp);
    if (one)
        reduce_f32_kernel<FSDP_REDUCE_F32_POL, true, 1>
            <<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileReduce / sp, ents, rs_in, S, N, fN);
    else if (chunk_aligned)
        reduce_f32_kernel<FSDP_REDUCE_F32_POL, true, 2>
            <<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileReduce / sp, ents, rs_in, S, N, fN);
    else
        reduce_f32_kernel<FSDP_REDUCE_F32_POL, false, 2>
            <<<grid, kBlock, 0, st>>>(tiles, n, sp, kTileReduce / sp, ents, rs_in, S, N, fN);
    return hipGetLastError();
}

}  // namespace fsdp
