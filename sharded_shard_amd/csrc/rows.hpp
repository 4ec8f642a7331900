// Column sums over the N rows of an [N, S] buffer of bf16 gradient
// contributions, added in rank order from row 0 (the reduction and the
// fused step share them), and the schedule of 8-element groups over a
// block's lanes.
#pragma once

#include "device.hpp"

// rows in flight per lane of the bf16 reduction on aligned rows (2: 0.4%
// ahead of 1 at 8 ranks with both rows' loads issued together; more rows
// spread each wave over more DRAM pages), and on misaligned rows (2
// measured 2.5% slower than 1)
#ifndef FSDP_REDUCE_ROW_BATCH
#define FSDP_REDUCE_ROW_BATCH 2
#endif
#ifndef FSDP_REDUCE_MIS_ROW_BATCH
#define FSDP_REDUCE_MIS_ROW_BATCH 1
#endif

namespace fsdp {

namespace {

// Sum of rows 0..N-1 at element offset `e` (from row 0's base), in order.
__device__ __forceinline__ float sum_rows_scalar(const uint16_t *src0, int64_t S, int32_t N,
                                                 int64_t e) {
    float acc = widen(src0[e]);
    for (int32_t j = 1; j < N; ++j) acc = acc + widen(src0[static_cast<int64_t>(j) * S + e]);
    return acc;
}

__device__ __forceinline__ void acc8(float (&acc)[8], u32x4 x) {
    acc[0] = acc[0] + bf16_lo(x.x);
    acc[1] = acc[1] + bf16_hi(x.x);
    acc[2] = acc[2] + bf16_lo(x.y);
    acc[3] = acc[3] + bf16_hi(x.y);
    acc[4] = acc[4] + bf16_lo(x.z);
    acc[5] = acc[5] + bf16_hi(x.z);
    acc[6] = acc[6] + bf16_lo(x.w);
    acc[7] = acc[7] + bf16_hi(x.w);
}

__device__ __forceinline__ void init8(float (&acc)[8], u32x4 x) {
    acc[0] = bf16_lo(x.x);
    acc[1] = bf16_hi(x.x);
    acc[2] = bf16_lo(x.y);
    acc[3] = bf16_hi(x.y);
    acc[4] = bf16_lo(x.z);
    acc[5] = bf16_hi(x.z);
    acc[6] = bf16_lo(x.w);
    acc[7] = bf16_hi(x.w);
}

// Aligned rows, C groups per lane: row by row from row 0, the C chunks of a
// row in flight together, so a wave reads C KB of one row before it moves to
// the next (at 64 ranks this keeps each wave on one DRAM region at a time:
// measured 5.99 vs 5.31 TB/s for one chunk of four rows in flight).  Pass c
// of this lane sits at byte offset offb + c * 1024.  Each row's buffer range
// covers exactly the 16-byte chunks holding its dbytes data bytes, so a lane
// past the end of the data reads zeros and never touches memory beyond the
// last chunk.  kRoll (the fused step) reloads each chunk's register with the
// next row's chunk as soon as it has been added, so the wave never drains
// its loads between rows: the 64-rank fused step 5.70 -> 5.93 TB/s on
// MI355X; the plain reduction stays without (6.31 vs 6.19 TB/s).
template <int NT, int C, bool kRoll = false>
__device__ __forceinline__ void sum_rows_wide(const uint16_t *base, uint32_t offb, uint32_t dbytes,
                                              int64_t S, int32_t N, float (&acc)[C][8]) {
    const char *r = reinterpret_cast<const char *>(base);
    const int64_t Sb = S * 2;
    const uint32_t nb = (dbytes + 15u) & ~15u;
    if constexpr (kRoll) {
        // chunk c of row j is added, then its register is reloaded with chunk
        // c of row j + 1: the wave waits for its oldest load only, and about
        // C loads stay in flight through the whole row loop.  Row 1 is read
        // with an empty range when N == 1 (zeros, no memory access).
        u32x4 x[C];
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = bload16<NT>(r, offb + c * 1024u, nb);
        const uint32_t nb1 = N > 1 ? nb : 0u;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            init8(acc[c], x[c]);
            x[c] = bload16<NT>(r + Sb, offb + c * 1024u, nb1);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int32_t j = 2; j < N; ++j) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                acc8(acc[c], x[c]);
                x[c] = bload16<NT>(r + j * Sb, offb + c * 1024u, nb);
                // in this order: hoisting the loads above the adds would
                // need a second set of chunk registers
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (N > 1) {
#pragma unroll
            for (int c = 0; c < C; ++c) acc8(acc[c], x[c]);
        }
        return;
    }
    {
        u32x4 x[C];
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = bload16<NT>(r, offb + c * 1024u, nb);
#pragma unroll
        for (int c = 0; c < C; ++c) init8(acc[c], x[c]);
    }
    for (int32_t j = 1; j < N; ++j) {
        u32x4 x[C];
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = bload16<NT>(r + j * Sb, offb + c * 1024u, nb);
#pragma unroll
        for (int c = 0; c < C; ++c) acc8(acc[c], x[c]);
    }
}

// Column sums of four consecutive elements (a quad) at QP places per lane,
// byte offsets offb + 512 h (h < QP) from row 0 at base (16-byte aligned
// rows, uniform), over the N rows of [N, S] bf16, in rank order from row 0;
// rows RB at a time, each row QP 8-byte loads per lane.  Buffer ranges as in
// sum_rows_wide (8-byte granules).  Lanes past the data read zeros.
template <int NT, int RB, int QP>
__device__ __forceinline__ void sum_rows_quad(const uint16_t *base, uint32_t offb, uint32_t dbytes,
                                              int64_t S, int32_t N, float (&acc)[QP][4]) {
    const char *r = reinterpret_cast<const char *>(base);
    const int64_t Sb = S * 2;
    const uint32_t nb = (dbytes + 7u) & ~7u;
    // whole batches of RB rows, then the last N mod RB rows one at a time:
    // no guard sits between a batch's loads and its adds (a guard per row let
    // the compiler issue each row's loads only after the previous row's had
    // returned, so a batch of 2 ran as 1)
    int32_t j = 0;
    for (; j + RB <= N; j += RB) {
        u32x2 x[RB][QP];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int h = 0; h < QP; ++h)
                x[i][h] = bload8<NT>(r + (j + i) * Sb, offb + 512u * h, nb);
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int h = 0; h < QP; ++h) {
                const float y[4] = {bf16_lo(x[i][h].x), bf16_hi(x[i][h].x), bf16_lo(x[i][h].y),
                                    bf16_hi(x[i][h].y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[h][e] = j + i == 0 ? y[e] : acc[h][e] + y[e];
            }
    }
    for (; j < N; ++j) {
        u32x2 x[QP];
#pragma unroll
        for (int h = 0; h < QP; ++h) x[h] = bload8<NT>(r + j * Sb, offb + 512u * h, nb);
#pragma unroll
        for (int h = 0; h < QP; ++h) {
            const float y[4] = {bf16_lo(x[h].x), bf16_hi(x[h].x), bf16_lo(x[h].y), bf16_hi(x[h].y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h][e] = j == 0 ? y[e] : acc[h][e] + y[e];
        }
    }
}

// The same sums over misaligned rows: row j starts k_j = (k0 + j kS) & 7
// bytes past an 8-byte boundary.  Lane l loads the 8-byte word holding the
// start of its quad, takes the next word from lane l + 1 (DPP; lane 63 loads
// its own, from a load whose other lanes sit at the end of the buffer
// range), and funnel-shifts by k_j: every word of a row is read once.  The
// whole wave must run this (the DPP reads every lane).
template <int NT, int RB>
__device__ __forceinline__ void sum_rows_quad_mis(const uint16_t *base, uint32_t offb,
                                                  uint32_t dbytes, int64_t S, int32_t N,
                                                  uint32_t k0, uint32_t kS, float (&acc)[2][4]) {
    const char *r = reinterpret_cast<const char *>(base);
    const int64_t Sb = S * 2;
    const bool last = (threadIdx.x & 63) == 63;
    for (int32_t j = 0; j < N; j += RB) {
        u32x2 a[RB][2], e[RB][2];
        uint32_t kk[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            kk[i] = (k0 + static_cast<uint32_t>(j + i) * kS) & 7u;
            const char *al = r + (j + i) * Sb - kk[i];
            const uint32_t n = j + i < N ? (kk[i] + dbytes + 7u) & ~7u : 0u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t o = offb + 512u * h;
                a[i][h] = bload8<NT>(al, o, n);
                e[i][h] = bload8<kBoundaryNT>(al, last ? o + 8u : n, n);
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const bool s4 = kk[i] >= 4u;
            const uint32_t sh = kk[i] & 3u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x2 b = next_or_own(a[i][h], e[i][h]);
                // bytes [k, k + 8) of a:b
                const uint32_t u0 = s4 ? a[i][h].y : a[i][h].x, u1 = s4 ? b.x : a[i][h].y;
                const uint32_t u2 = s4 ? b.y : b.x;
                const uint32_t w0 = __builtin_amdgcn_alignbyte(u1, u0, sh);
                const uint32_t w1 = __builtin_amdgcn_alignbyte(u2, u1, sh);
                if (j + i >= N) continue;
                const float y[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[h][q] = j + i == 0 ? y[q] : acc[h][q] + y[q];
            }
        }
    }
}

// Group schedule of the wide row kernels (16-byte aligned rows): 8-element
// groups [0, ngrp), C per lane per pass; pass c of lane l of wave w takes
// group (w*C + c)*64 + l, then all step by the block.  Every lane runs the
// same number of iterations, and `own` says whether its group exists.
template <int C = 1>
struct GroupWalk {
    int64_t g, step;
    __device__ GroupWalk() {
        const int64_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        g = wave * 64 * C + lane;
        step = static_cast<int64_t>(blockDim.x >> 6) * 64 * C;
    }
    // the wave still has work
    __device__ bool more(int64_t ngrp) const {
        return g - static_cast<int64_t>(threadIdx.x & 63) < ngrp;
    }
    // group of pass c
    __device__ int64_t at(int c) const { return g + c * 64; }
    __device__ bool own(int64_t ngrp, int c = 0) const { return at(c) < ngrp; }
    __device__ void next() { g += step; }
};

}  // namespace

}  // namespace fsdp
