// AdamW on the fp32 shards, AdamW fused with the copy-in, and the fused
// sharded step (reduce -> AdamW -> copy-in in one pass), bit-identical to the
// separate kernels: the same device functions in the same order, one fp32
// rounding per operation.
#include "launch.hpp"
#include "rows.hpp"

// AdamW per group: plain loads and stores (non-temporal ones make the
// kernel faster but the step slower: on the Llama 70B shape, per group,
// 73.4 against 72.3 ms, the next group's reduction losing 3%)
#ifndef FSDP_ADAMW_POL
#define FSDP_ADAMW_POL 0
#endif
// AdamW as one launch over every group, and AdamW fused with the copy-in
// (also one launch over a group set): non-temporal loads and stores (the
// AdamW launch 5.25 -> 5.55 TB/s on the Llama 7B shape, the step 14.71 ->
// 14.57 ms; the fused launch's step 14.17 -> 14.04 ms, and 73.3 -> 73.05 ms
// on the 70B shape)
#ifndef FSDP_ADAMW_SET_POL
#define FSDP_ADAMW_SET_POL 3
#endif
#ifndef FSDP_ADAMW_PACK_POL
#define FSDP_ADAMW_PACK_POL 3
#endif
// elements per block of AdamW fused with the copy-in: one vector per lane
// and array, as AdamW (against 4096: 5.3-5.4 -> 5.5-5.8 TB/s; 2048 in
// between)
#ifndef FSDP_ADAMW_PACK_SUB
#define FSDP_ADAMW_PACK_SUB 1024
#endif
// shard policy of the wide fused step (plain: its lanes store two halves
// of a 32-byte span, which non-temporal stores split into partial writes)
#ifndef FSDP_STEP_POL
#define FSDP_STEP_POL 0
#endif
// shard policy of the aligned fused step (a quad per lane: every wave
// instruction contiguous, so non-temporal stores write whole lines)
#ifndef FSDP_STEP_QUAD_POL
#define FSDP_STEP_QUAD_POL 3
#endif
// the aligned fused step's bf16 output: plain stores (the copy-out that
// follows reads that row)
#ifndef FSDP_STEP_OUT_NT
#define FSDP_STEP_OUT_NT 0
#endif
// rows in flight per lane of the aligned fused step up to 8 ranks (1: with
// both rows' loads issued together, 2 measured 0.5% slower per 7B step, 4
// 0.6%), and of both narrow fused-step variants from 9 to 15 ranks
#ifndef FSDP_STEP_ROW_BATCH
#define FSDP_STEP_ROW_BATCH 1
#endif
#ifndef FSDP_STEP_ROW_BATCH_WIDE
#define FSDP_STEP_ROW_BATCH_WIDE 4
#endif
// rows in flight of the fused step on misaligned rows up to 8 ranks
#ifndef FSDP_STEP_GEN_ROW_BATCH
#define FSDP_STEP_GEN_ROW_BATCH 1
#endif
// Groups per lane (at least 1) of the fused step's wide kernel, used on
// aligned rows from FSDP_STEP_WIDE_MIN_N ranks (a larger world size than any
// in use turns it off).
#ifndef FSDP_STEP_WIDE
#define FSDP_STEP_WIDE 8
#endif
#ifndef FSDP_STEP_WIDE_MIN_N
#define FSDP_STEP_WIDE_MIN_N 16
#endif
// the wide fused step's bf16 output: plain stores (the copy-out that follows
// reads that row; non-temporal stores measured 1.3% slower per step at 64
// ranks)
#ifndef FSDP_WIDE_OUT_NT
#define FSDP_WIDE_OUT_NT 0
#endif
// register budget of the wide fused step: at least this many waves per SIMD
// (amdgpu_waves_per_eu; capping it at 3 with an LDS reservation, below,
// measured 1.6% slower per 70B step)
#ifndef FSDP_STEP_WIDE_WAVES
#define FSDP_STEP_WIDE_WAVES 4
#endif
// register budget of the aligned fused step: at least this many waves per
// SIMD (amdgpu_waves_per_eu; 6 measured ahead of 7 and 8)
#ifndef FSDP_STEP_WAVES
#define FSDP_STEP_WAVES 6
#endif
// Occupancy caps.  A block that reserves LDS it never touches limits how many
// blocks share a CU (160 KB of LDS per CU).  The aligned fused step reserves
// 28 KB, so 5 of its 256-thread blocks (5 waves per SIMD) share a CU: 7B step
// 11.63-11.65 -> 11.54-11.55 ms and one block 0.3585-0.3596 -> 0.3556 ms at 8
// ranks (24 KB, 6 blocks, measured no change; 36 KB, 4 blocks, 0.3% slower;
// the misaligned fused step measured no gain at 6 or 5 blocks and 1.7% loss
// at 4).  AdamW as one launch over a group set and AdamW fused with the
// copy-in reserve 48 KB, 3 blocks per CU: AdamW 6.0 -> 6.1 TB/s on the 7B
// shape and 5.7 -> 6.2 on the 70B shape, the fused AdamW + copy-in 5.8 -> 6.1
// and 5.5 -> 6.2 (group-set steps 0.4-2% faster; 64 KB, 2 blocks, slower).
// Per group, AdamW keeps no cap: 48 KB measured 1.3% faster per 7B step but
// 0.4% slower per 70B step, whose per-group launches are short.
#ifndef FSDP_STEP_LDS
#define FSDP_STEP_LDS 28672
#endif
#ifndef FSDP_ADAMW_SET_LDS
#define FSDP_ADAMW_SET_LDS 49152
#endif
// the fused step reads its N gradient rows with non-temporal loads
#ifndef FSDP_STEP_ROW_NT
#define FSDP_STEP_ROW_NT 1
#endif

namespace fsdp {

namespace {

// ---------------------------------------------------------------------------
// AdamW on fp32 shards
// ---------------------------------------------------------------------------

struct AdamwScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps, decay, step_size, bc2_sqrt;
};

__device__ __forceinline__ void adamw_elem(float &p, float g, float &m, float &v,
                                           const AdamwScalars &c) {
    p = p * c.decay;
    m = c.beta1 * m + c.one_minus_beta1 * g;
    v = c.beta2 * v + c.one_minus_beta2 * (g * g);
    const float d = __builtin_sqrtf(v) / c.bc2_sqrt + c.eps;
    p = p - c.step_size * (m / d);
}

__device__ __forceinline__ void adamw_vec(f32x4 &p, f32x4 g, f32x4 &m, f32x4 &v,
                                          const AdamwScalars &c) {
    float pe[4] = {p.x, p.y, p.z, p.w}, me[4] = {m.x, m.y, m.z, m.w}, ve[4] = {v.x, v.y, v.z, v.w};
    const float ge[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw_elem(pe[k], ge[k], me[k], ve[k], c);
    p = f32x4{pe[0], pe[1], pe[2], pe[3]};
    m = f32x4{me[0], me[1], me[2], me[3]};
    v = f32x4{ve[0], ve[1], ve[2], ve[3]};
}

__device__ __forceinline__ void adamw_scalar_at(float *P, const float *G, float *M, float *Vv,
                                                int64_t i, const AdamwScalars &c) {
    float p = P[i], m = M[i], v = Vv[i];
    adamw_elem(p, G[i], m, v, c);
    P[i] = p;
    M[i] = m;
    Vv[i] = v;
}

template <int POL>
__device__ __forceinline__ void adamw_run(float *P, const float *G, float *M, float *Vv, int64_t len,
                                          const AdamwScalars &c) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    const uint32_t ap = lo32(P) & 15u;
    const bool same = ap == (lo32(G) & 15u) && ap == (lo32(M) & 15u) && ap == (lo32(Vv) & 15u);
    if (!same) {
        for (int64_t i = tid; i < len; i += kBlock) adamw_scalar_at(P, G, M, Vv, i, c);
        return;
    }
    int64_t head = ((16u - ap) & 15u) >> 2;
    if (head > len) head = len;
    if (tid < head) adamw_scalar_at(P, G, M, Vv, tid, c);
    const int64_t nvec = (len - head) >> 2;
    f32x4 *pv = reinterpret_cast<f32x4 *>(P + head);
    const f32x4 *gv = reinterpret_cast<const f32x4 *>(G + head);
    f32x4 *mv = reinterpret_cast<f32x4 *>(M + head);
    f32x4 *vv = reinterpret_cast<f32x4 *>(Vv + head);
    int64_t i = tid;
    for (; i + kBlock < nvec; i += 2 * kBlock) {
        const int64_t i1 = i + kBlock;
        f32x4 p0 = ldp<LN>(pv + i), m0 = ldp<LN>(mv + i), v0 = ldp<LN>(vv + i);
        f32x4 p1 = ldp<LN>(pv + i1), m1 = ldp<LN>(mv + i1), v1 = ldp<LN>(vv + i1);
        const f32x4 g0 = ldp<LN>(gv + i), g1 = ldp<LN>(gv + i1);
        adamw_vec(p0, g0, m0, v0, c);
        adamw_vec(p1, g1, m1, v1, c);
        stp<SN>(pv + i, p0);
        stp<SN>(mv + i, m0);
        stp<SN>(vv + i, v0);
        stp<SN>(pv + i1, p1);
        stp<SN>(mv + i1, m1);
        stp<SN>(vv + i1, v1);
    }
    if (i < nvec) {
        f32x4 p0 = ldp<LN>(pv + i), m0 = ldp<LN>(mv + i), v0 = ldp<LN>(vv + i);
        const f32x4 g0 = ldp<LN>(gv + i);
        adamw_vec(p0, g0, m0, v0, c);
        stp<SN>(pv + i, p0);
        stp<SN>(mv + i, m0);
        stp<SN>(vv + i, v0);
    }
    const int64_t e = head + (nvec << 2) + tid;
    if (e < len) adamw_scalar_at(P, G, M, Vv, e, c);
}

template <int POL>
__global__ __launch_bounds__(kBlock) void adamw_kernel(
    const EwTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, AdamwScalars c) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const EwTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        const DevEntry en = ents[tl.entry];
        const int64_t o = tl.off + b;
        adamw_run<POL>(en.master + o, en.grad + o, en.exp_avg + o, en.exp_avg_sq + o, len, c);
    }
}

// ---------------------------------------------------------------------------
// fused step: reduce -> AdamW -> copy-in, one pass over this rank's pieces
// ---------------------------------------------------------------------------

// One element: the three steps exactly as the separate kernels compute them.
template <bool kWriteGrad>
__device__ __forceinline__ void step_scalar_at(const uint16_t *rs0, int64_t S, int32_t N, float fN,
                                               float *P, float *M, float *Vv, float *G,
                                               uint16_t *dst, int64_t e, const AdamwScalars &c) {
    const float g = sum_rows_scalar(rs0, S, N, e) / fN;
    if (kWriteGrad) G[e] = g;
    float p = P[e], m = M[e], v = Vv[e];
    adamw_elem(p, g, m, v, c);
    P[e] = p;
    M[e] = m;
    Vv[e] = v;
    dst[e] = static_cast<uint16_t>(bf16_rne(p));
}

// The fused step on 16-byte aligned rows at many ranks (the wide kernel):
// valid elements [0, valid), then zeros up to len.  rs0 is row 0 of the
// gradient contributions at this run's first segment position; dst is ag_in
// at the same position; P, M, Vv, G are the shards at this run's first
// element.  The vector path aligns on the fp32 shards (the bulk of the
// bytes); the bf16 output is stored whole, by dwords or by halves, as its
// address allows.  C groups of 8 elements per lane, the rows read row by
// row with the lane's C chunks in flight (sum_rows_wide, rolling).
template <int POL, int C, bool kWriteGrad>
__device__ __forceinline__ void step_run_wide(const uint16_t *__restrict__ rs0, int64_t S,
                                              int32_t N, float fN, float *P, float *M, float *Vv,
                                              float *G, uint16_t *dst, int64_t len,
                                              int64_t valid, const AdamwScalars &c) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    const uint32_t ap = lo32(P) & 15u;
    int64_t head = ((16u - ap) & 15u) >> 2;
    if (head > valid) head = valid;
    const uint32_t kS = static_cast<uint32_t>((S * 2) & 15);
    const uint32_t k0 = lo32(rs0 + head) & 15u;
    // the vector path needs the shards equally aligned and the rows 16-byte
    // aligned at the first vector element
    const bool same = ap == (lo32(M) & 15u) && ap == (lo32(Vv) & 15u) &&
                      (!kWriteGrad || ap == (lo32(G) & 15u)) && (k0 | kS) == 0;
    if (!same) {
        for (int64_t e = tid; e < valid; e += static_cast<int64_t>(blockDim.x))
            step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, e, c);
    } else {
        if (tid < head) step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, tid, c);
        const int64_t ngrp = (valid - head) >> 3;
        const uint32_t ka = lo32(dst + head) & 15u;
        const uint32_t dbytes = static_cast<uint32_t>(2 * (valid - head));
        for (GroupWalk<C> w; w.more(ngrp); w.next()) {
            float acc[C][8];
            sum_rows_wide<FSDP_STEP_ROW_NT, C, true>(rs0 + head, static_cast<uint32_t>(w.g) << 4,
                                                     dbytes, S, N, acc);
#pragma unroll
            for (int q = 0; q < C; ++q) {
                if (!w.own(ngrp, q)) continue;
                const int64_t e0 = head + (w.at(q) << 3);
                f32x4 *pv = reinterpret_cast<f32x4 *>(P + e0);
                f32x4 *mv = reinterpret_cast<f32x4 *>(M + e0);
                f32x4 *vv = reinterpret_cast<f32x4 *>(Vv + e0);
                f32x4 p0 = ldp<LN>(pv), p1 = ldp<LN>(pv + 1);
                f32x4 m0 = ldp<LN>(mv), m1 = ldp<LN>(mv + 1);
                f32x4 v0 = ldp<LN>(vv), v1 = ldp<LN>(vv + 1);
                const f32x4 g0{acc[q][0] / fN, acc[q][1] / fN, acc[q][2] / fN, acc[q][3] / fN};
                const f32x4 g1{acc[q][4] / fN, acc[q][5] / fN, acc[q][6] / fN, acc[q][7] / fN};
                if (kWriteGrad) {
                    f32x4 *gv = reinterpret_cast<f32x4 *>(G + e0);
                    stp<SN>(gv, g0);
                    stp<SN>(gv + 1, g1);
                }
                adamw_vec(p0, g0, m0, v0, c);
                adamw_vec(p1, g1, m1, v1, c);
                stp<SN>(pv, p0);
                stp<SN>(pv + 1, p1);
                stp<SN>(mv, m0);
                stp<SN>(mv + 1, m1);
                stp<SN>(vv, v0);
                stp<SN>(vv + 1, v1);
                const float pb[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                store16_at<FSDP_WIDE_OUT_NT>(dst + e0, ka, pack8(pb));
            }
        }
        const int64_t done = head + (ngrp << 3);
        if (tid < valid - done)
            step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, done + tid, c);
    }
    zero_bf16<1>(dst, valid, len);
}

// Store 4 bf16 (one u32x2) at p, whose address modulo 8 is k (even, uniform):
// one 8-byte store when aligned, else dword and short stores.
template <int NT>
__device__ __forceinline__ void store8_at(uint16_t *p, uint32_t k, u32x2 w) {
    if (k == 0) {
        stp<NT>(reinterpret_cast<u32x2 *>(p), w);
    } else if (k == 4) {
        uint32_t *d = reinterpret_cast<uint32_t *>(p);
        d[0] = w.x;
        d[1] = w.y;
    } else {
        p[0] = static_cast<uint16_t>(w.x);
        *reinterpret_cast<uint32_t *>(p + 1) = alignbyte2(w.y, w.x);
        p[3] = static_cast<uint16_t>(w.y >> 16);
    }
}

// ---------------------------------------------------------------------------
// AdamW fused with the copy-in: the optimizer step that also writes the next
// all-gather's bf16 segment, with the gradient from the grad shards
// ---------------------------------------------------------------------------

__device__ __forceinline__ void adamw_pack_scalar_at(float *P, const float *G, float *M,
                                                     float *Vv, uint16_t *dst, int64_t i,
                                                     const AdamwScalars &c) {
    float p = P[i], m = M[i], v = Vv[i];
    adamw_elem(p, G[i], m, v, c);
    P[i] = p;
    M[i] = m;
    Vv[i] = v;
    dst[i] = static_cast<uint16_t>(bf16_rne(p));
}

// Valid elements [0, valid) of one run: AdamW exactly as adamw_run, then
// the bf16 cast of the new master into dst as pack_run writes it; zeros in
// dst from valid to len.  Four elements per lane and vector (one vector per
// lane in a sub-range of FSDP_ADAMW_PACK_SUB elements, longer ones two a
// block apart per iteration); the bf16 output stored by its own 8-byte phase.
template <int POL>
__device__ __forceinline__ void adamw_pack_run(float *P, const float *G, float *M, float *Vv,
                                               uint16_t *dst, int64_t len, int64_t valid,
                                               const AdamwScalars &c) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    const uint32_t ap = lo32(P) & 15u;
    const bool same = ap == (lo32(G) & 15u) && ap == (lo32(M) & 15u) && ap == (lo32(Vv) & 15u);
    if (!same) {
        for (int64_t i = tid; i < valid; i += kBlock) adamw_pack_scalar_at(P, G, M, Vv, dst, i, c);
    } else {
        int64_t head = ((16u - ap) & 15u) >> 2;
        if (head > valid) head = valid;
        if (tid < head) adamw_pack_scalar_at(P, G, M, Vv, dst, tid, c);
        const int64_t nvec = (valid - head) >> 2;
        f32x4 *pv = reinterpret_cast<f32x4 *>(P + head);
        const f32x4 *gv = reinterpret_cast<const f32x4 *>(G + head);
        f32x4 *mv = reinterpret_cast<f32x4 *>(M + head);
        f32x4 *vv = reinterpret_cast<f32x4 *>(Vv + head);
        uint16_t *d = dst + head;
        const uint32_t k8 = lo32(d) & 7u;
        int64_t i = tid;
        for (; i + kBlock < nvec; i += 2 * kBlock) {
            const int64_t i1 = i + kBlock;
            f32x4 p0 = ldp<LN>(pv + i), m0 = ldp<LN>(mv + i), v0 = ldp<LN>(vv + i);
            f32x4 p1 = ldp<LN>(pv + i1), m1 = ldp<LN>(mv + i1), v1 = ldp<LN>(vv + i1);
            const f32x4 g0 = ldp<LN>(gv + i), g1 = ldp<LN>(gv + i1);
            adamw_vec(p0, g0, m0, v0, c);
            adamw_vec(p1, g1, m1, v1, c);
            stp<SN>(pv + i, p0);
            stp<SN>(mv + i, m0);
            stp<SN>(vv + i, v0);
            stp<SN>(pv + i1, p1);
            stp<SN>(mv + i1, m1);
            stp<SN>(vv + i1, v1);
            store8_at<SN>(d + (i << 2), k8, u32x2{pack2(p0.x, p0.y), pack2(p0.z, p0.w)});
            store8_at<SN>(d + (i1 << 2), k8, u32x2{pack2(p1.x, p1.y), pack2(p1.z, p1.w)});
        }
        if (i < nvec) {
            f32x4 p0 = ldp<LN>(pv + i), m0 = ldp<LN>(mv + i), v0 = ldp<LN>(vv + i);
            const f32x4 g0 = ldp<LN>(gv + i);
            adamw_vec(p0, g0, m0, v0, c);
            stp<SN>(pv + i, p0);
            stp<SN>(mv + i, m0);
            stp<SN>(vv + i, v0);
            store8_at<SN>(d + (i << 2), k8, u32x2{pack2(p0.x, p0.y), pack2(p0.z, p0.w)});
        }
        const int64_t e = head + (nvec << 2) + tid;
        if (e < valid) adamw_pack_scalar_at(P, G, M, Vv, dst, e, c);
    }
    zero_bf16<SN>(dst, valid, len);
}

// Over copy-in tiles: AdamW of the tile's valid elements and their bf16
// copy into ag_in (the set's arena), zeros in the padding.
template <int POL>
__global__ __launch_bounds__(kBlock) void adamw_pack_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, uint16_t *__restrict__ ag_in, AdamwScalars c) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        const DevEntry en = ents[tl.entry];
        const int64_t o = tl.src + b;
        adamw_pack_run<POL>(en.master + o, en.grad + o, en.exp_avg + o, en.exp_avg_sq + o,
                            ag_in + tl.dst + b, len, valid, c);
    }
}

// The fused step, a quad per lane and pass: lane l of a wave takes quads
// l + 64 h (h < QP) of the wave's 64 QP, so every load and store instruction
// of the wave is contiguous (rows 512 bytes, shards 1 KB, the bf16 output 512
// bytes).  That lets the shards use non-temporal loads and stores without
// partial writes (a lane storing two halves of 32 bytes splits them).  Rows
// 16-byte aligned, or with kMis at any even byte phase (sum_rows_quad_mis,
// QP = 2).  Same arithmetic, in the same order, as step_run_wide and the
// separate kernels.
template <int POL, int RB, int QP, bool kWriteGrad, bool kMis = false>
__device__ __forceinline__ void step_run_quad(const uint16_t *__restrict__ rs0, int64_t S,
                                              int32_t N, float fN, float *P, float *M, float *Vv,
                                              float *G, uint16_t *dst, int64_t len, int64_t valid,
                                              const AdamwScalars &c) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    const uint32_t ap = lo32(P) & 15u;
    int64_t head = ((16u - ap) & 15u) >> 2;
    if (head > valid) head = valid;
    const uint32_t kS = static_cast<uint32_t>((S * 2) & 15);
    const uint32_t k0 = lo32(rs0 + head) & 15u;
    const bool same = ap == (lo32(M) & 15u) && ap == (lo32(Vv) & 15u) &&
                      (!kWriteGrad || ap == (lo32(G) & 15u)) && (kMis || (k0 | kS) == 0);
    if (!same) {
        for (int64_t e = tid; e < valid; e += static_cast<int64_t>(blockDim.x))
            step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, e, c);
    } else {
        static_assert(!kMis || QP == 2, "misaligned rows: two quads per lane");
        if (tid < head) step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, tid, c);
        const int64_t nq = (valid - head) >> 2;
        const uint32_t k8 = lo32(dst + head) & 7u;
        const uint32_t dbytes = static_cast<uint32_t>(2 * (valid - head));
        const int64_t lane = tid & 63;
        const int64_t qstep = static_cast<int64_t>(blockDim.x >> 6) * 64 * QP;
        char *pb = reinterpret_cast<char *>(P + head), *mb = reinterpret_cast<char *>(M + head);
        char *vb = reinterpret_cast<char *>(Vv + head);
        char *gb = kWriteGrad ? reinterpret_cast<char *>(G + head) : nullptr;
        const uint32_t sb = static_cast<uint32_t>(nq) << 4;
        for (int64_t qb = (tid >> 6) * 64 * QP; qb < nq; qb += qstep) {
            float acc[QP][4];
            if constexpr (kMis)
                sum_rows_quad_mis<FSDP_STEP_ROW_NT, RB>(rs0 + head,
                                                        static_cast<uint32_t>(qb + lane) << 3,
                                                        dbytes, S, N, k0 & 7u, kS & 7u, acc);
            else
                sum_rows_quad<FSDP_STEP_ROW_NT, RB, QP>(
                    rs0 + head, static_cast<uint32_t>(qb + lane) << 3, dbytes, S, N, acc);
            // p, m and v of every quad of the pass through buffer ranges of
            // the run's vectors: all loads leave before the first wait (with
            // a guard per quad they went one quad at a time), and lanes past
            // the end read zeros and have their stores dropped
            f32x4 pq[QP], mq[QP], vq[QP];
#pragma unroll
            for (int h = 0; h < QP; ++h) {
                const uint32_t o = static_cast<uint32_t>(qb + lane + 64 * h) << 4;
                pq[h] = __builtin_bit_cast(f32x4, bload16<LN>(pb, o, sb));
                mq[h] = __builtin_bit_cast(f32x4, bload16<LN>(mb, o, sb));
                vq[h] = __builtin_bit_cast(f32x4, bload16<LN>(vb, o, sb));
            }
#pragma unroll
            for (int h = 0; h < QP; ++h) {
                const uint32_t o = static_cast<uint32_t>(qb + lane + 64 * h) << 4;
                const f32x4 g{acc[h][0] / fN, acc[h][1] / fN, acc[h][2] / fN, acc[h][3] / fN};
                if (kWriteGrad) bstore16<SN>(gb, o, sb, __builtin_bit_cast(u32x4, g));
                adamw_vec(pq[h], g, mq[h], vq[h], c);
                bstore16<SN>(pb, o, sb, __builtin_bit_cast(u32x4, pq[h]));
                bstore16<SN>(mb, o, sb, __builtin_bit_cast(u32x4, mq[h]));
                bstore16<SN>(vb, o, sb, __builtin_bit_cast(u32x4, vq[h]));
                const int64_t q = qb + lane + 64 * h;
                if (q < nq)
                    store8_at<FSDP_STEP_OUT_NT>(
                        dst + head + (q << 2), k8,
                        u32x2{pack2(pq[h].x, pq[h].y), pack2(pq[h].z, pq[h].w)});
            }
        }
        const int64_t done = head + (nq << 2);
        if (tid < valid - done)
            step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, done + tid, c);
    }
    zero_bf16<1>(dst, valid, len);
}

template <int POL, int RB, int C, bool kChunkAligned, bool kWriteGrad, int QP = 0>
__device__ __forceinline__ void step_tiles(const PackTile *__restrict__ tiles, int64_t n_tiles,
                                           int32_t split, int64_t sub,
                                           const DevEntry *__restrict__ ents,
                                           const uint16_t *__restrict__ rs_in,
                                           uint16_t *__restrict__ ag_in, int64_t S, int32_t N,
                                           float fN, const AdamwScalars &c) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        const DevEntry en = ents[tl.entry];
        const int64_t o = tl.src + b;
        if constexpr (QP > 0)
            step_run_quad<POL, RB, QP, kWriteGrad, !kChunkAligned>(rs_in + tl.dst + b, S, N, fN, en.master + o,
                                               en.exp_avg + o, en.exp_avg_sq + o,
                                               kWriteGrad ? en.grad + o : nullptr,
                                               ag_in + tl.dst + b, len, valid, c);
        else
            step_run_wide<POL, C, kWriteGrad>(
                rs_in + tl.dst + b, S, N, fN, en.master + o, en.exp_avg + o, en.exp_avg_sq + o,
                kWriteGrad ? en.grad + o : nullptr, ag_in + tl.dst + b, len, valid, c);
    }
}

// Aligned rows, a quad per lane and pass (step_run_quad) with the shard
// policy FSDP_STEP_QUAD_POL, scheduled for FSDP_STEP_WAVES waves per SIMD.
template <int RB, bool kWriteGrad>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(FSDP_STEP_WAVES)))
void step_kernel_aligned(const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split,
                         int64_t sub, const DevEntry *__restrict__ ents,
                         const uint16_t *__restrict__ rs_in, uint16_t *__restrict__ ag_in,
                         int64_t S, int32_t N, float fN, AdamwScalars c) {
    step_tiles<FSDP_STEP_QUAD_POL, RB, 1, true, kWriteGrad, 2>(tiles, n_tiles, split, sub, ents,
                                                                rs_in, ag_in, S, N, fN, c);
}

// Aligned rows at many ranks: one wave per block, FSDP_STEP_WIDE groups per
// lane read row by row (sum_rows_wide).
template <int POL, bool kWriteGrad>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(FSDP_STEP_WIDE_WAVES)))
void step_kernel_wide(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ rs_in,
    uint16_t *__restrict__ ag_in, int64_t S, int32_t N, float fN, AdamwScalars c) {
    step_tiles<POL, 1, FSDP_STEP_WIDE, true, kWriteGrad>(tiles, n_tiles, split, sub, ents, rs_in,
                                                         ag_in, S, N, fN, c);
}

// Misaligned rows: a quad per lane and pass as the aligned kernel, each row
// funnel-shifted by its own phase (sum_rows_quad_mis).
template <int RB, bool kWriteGrad>
__global__ __launch_bounds__(kBlock) void step_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents,
    const uint16_t *__restrict__ rs_in, uint16_t *__restrict__ ag_in, int64_t S, int32_t N,
    float fN, AdamwScalars c) {
    step_tiles<FSDP_STEP_QUAD_POL, RB, 1, false, kWriteGrad, 2>(tiles, n_tiles, split, sub, ents,
                                                                 rs_in, ag_in, S, N, fN, c);
}

AdamwScalars to_scalars(const float s[8]) {
    return AdamwScalars{s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]};
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------

hipError_t launch_adamw(const EwTile *tiles, int64_t n, const DevEntry *ents,
                        const float scal[8], bool one_launch, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileAdamw, FSDP_ADAMW_SUB);
    if (one_launch)
        adamw_kernel<FSDP_ADAMW_SET_POL><<<grid_for(n, sp), kBlock, FSDP_ADAMW_SET_LDS, st>>>(
            tiles, n, sp, kTileAdamw / sp, ents, to_scalars(scal));
    else
        adamw_kernel<FSDP_ADAMW_POL><<<grid_for(n, sp), kBlock, 0, st>>>(
            tiles, n, sp, kTileAdamw / sp, ents, to_scalars(scal));
    return hipGetLastError();
}

hipError_t launch_adamw_pack(const PackTile *tiles, int64_t n, const DevEntry *ents,
                             uint16_t *ag_in, const float scal[8], hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTilePack, FSDP_ADAMW_PACK_SUB);
    adamw_pack_kernel<FSDP_ADAMW_PACK_POL><<<grid_for(n, sp), kBlock, FSDP_ADAMW_SET_LDS, st>>>(
        tiles, n, sp, kTilePack / sp, ents, ag_in, to_scalars(scal));
    return hipGetLastError();
}

template <int RB, int RBG>
void launch_step_rb(bool aligned, bool write_grad, unsigned grid, unsigned thr, hipStream_t st,
                    const PackTile *tiles, int64_t n, int32_t sp, int64_t sub, const DevEntry *ents,
                    const uint16_t *rs_in, uint16_t *ag_in, int64_t S, int32_t N, float fN,
                    const AdamwScalars &c) {
    if (aligned && write_grad)
        step_kernel_aligned<RB, true><<<grid, thr, FSDP_STEP_LDS, st>>>(
            tiles, n, sp, sub, ents, rs_in, ag_in, S, N, fN, c);
    else if (aligned)
        step_kernel_aligned<RB, false><<<grid, thr, FSDP_STEP_LDS, st>>>(
            tiles, n, sp, sub, ents, rs_in, ag_in, S, N, fN, c);
    else if (write_grad)
        step_kernel<RBG, true><<<grid, thr, 0, st>>>(tiles, n, sp, sub, ents, rs_in, ag_in, S, N,
                                                    fN, c);
    else
        step_kernel<RBG, false><<<grid, thr, 0, st>>>(tiles, n, sp, sub, ents, rs_in, ag_in, S, N,
                                                     fN, c);
}

hipError_t launch_step(const PackTile *tiles, int64_t n, const DevEntry *ents,
                       const uint16_t *rs_in, uint16_t *ag_in, int64_t S, int32_t N,
                       const float scal[8], bool write_grad, bool chunk_aligned,
                       hipStream_t st) {
    if (n == 0) return hipSuccess;
    const float fN = static_cast<float>(N);
    const AdamwScalars c = to_scalars(scal);
    // p, m, v read and written: six more streams per element besides the N rows;
    // both variants run whole waves of 128 quads, so sub-ranges are powers of two
    const int32_t sp = split_rows(kTilePack, N, 6);
    const int64_t sub = kTilePack / sp;
    const unsigned grid = grid_for(n, sp);
    const unsigned thr = kBlock;
    const bool aligned = chunk_aligned;
    constexpr int P = FSDP_STEP_POL;
    if (aligned && N >= FSDP_STEP_WIDE_MIN_N) {
        // one wave per block, each block one sub-range of 64 * 8 * FSDP_STEP_WIDE elements
        constexpr int64_t wsub = 64 * 8 * FSDP_STEP_WIDE;
        static_assert(kTilePack % wsub == 0, "wide sub-range must divide the tile");
        const int32_t wsp = static_cast<int32_t>(kTilePack / wsub);
        const unsigned wgrid = grid_for(n, wsp);
        if (write_grad)
            step_kernel_wide<P, true><<<wgrid, 64, 0, st>>>(tiles, n, wsp, wsub, ents, rs_in, ag_in,
                                                            S, N, fN, c);
        else
            step_kernel_wide<P, false><<<wgrid, 64, 0, st>>>(tiles, n, wsp, wsub, ents, rs_in, ag_in,
                                                             S, N, fN, c);
        return hipGetLastError();
    }
    if (N <= 8)
        launch_step_rb<FSDP_STEP_ROW_BATCH, FSDP_STEP_GEN_ROW_BATCH>(
            aligned, write_grad, grid, thr, st, tiles, n, sp, sub, ents, rs_in, ag_in, S, N, fN, c);
    else
        launch_step_rb<FSDP_STEP_ROW_BATCH_WIDE, FSDP_STEP_ROW_BATCH_WIDE>(
            aligned, write_grad, grid, thr, st, tiles, n, sp, sub, ents, rs_in, ag_in, S, N, fN, c);
    return hipGetLastError();
}

}  // namespace fsdp
