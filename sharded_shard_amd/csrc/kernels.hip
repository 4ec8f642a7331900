// HIP kernels of one rank's FSDP2 sharded step, written for CDNA4 (gfx950).
//
// All four kernels stream HBM and do (almost) no arithmetic, so the design
// rules are the memory-bound ones: 16-byte (dwordx4) coalesced loads and
// stores, several independent loads in flight per lane, non-temporal hints
// on data that is touched once, and no LDS.  Work is a table of tiles built
// on the host (plan.cpp): block b takes tiles b, b + grid, ...; each tile is
// one contiguous run of one parameter, so a block reads one tile record and
// one entry record with scalar loads and then streams.
//
// Alignment.  Pieces of a group sit back to back with no gap by default, so a
// run can start at any 2-byte (bf16) or 4-byte (fp32) address.  Destinations
// are handled in 16-byte vectors after a short element-wise head; sources
// that are misaligned relative to the destination are read as aligned 16-byte
// vectors and funnel-shifted in registers (v_alignbyte).  A 16-byte aligned
// vector never crosses a page, and every vector loaded holds at least one byte
// of the run, so the extra reads never touch unmapped memory.
//
// Numerics (built with -ffp-contract=off and correctly rounded fp32 divide
// and square root): reductions add rank contributions in rank order starting
// from rank 0's value, then divide once by N; AdamW performs each operation
// as one fp32 rounding in the order documented in the C header.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace fsdp {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) {
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void st_nt(T *p, T v) {
    __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ uint32_t alignbyte2(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// Bytes [k, k + 16) of the 32-byte little-endian concatenation a:b, k even.
__device__ __forceinline__ u32x4 funnel_bytes(u32x4 a, u32x4 b, uint32_t k) {
    u32x4 lo, hi;
    switch (k >> 2) {
        case 0:
            lo = a;
            hi = u32x4{a.y, a.z, a.w, b.x};
            break;
        case 1:
            lo = u32x4{a.y, a.z, a.w, b.x};
            hi = u32x4{a.z, a.w, b.x, b.y};
            break;
        case 2:
            lo = u32x4{a.z, a.w, b.x, b.y};
            hi = u32x4{a.w, b.x, b.y, b.z};
            break;
        default:
            lo = u32x4{a.w, b.x, b.y, b.z};
            hi = u32x4{b.x, b.y, b.z, b.w};
            break;
    }
    if (k & 2u) {
        return u32x4{alignbyte2(hi.x, lo.x), alignbyte2(hi.y, lo.y),
                     alignbyte2(hi.z, lo.z), alignbyte2(hi.w, lo.w)};
    }
    return lo;
}

// 16 bytes at byte address `addr` (even).  k = addr & 15 must be uniform
// across the wave for the branch to stay scalar.
__device__ __forceinline__ u32x4 load16_at(const uint16_t *p, uint32_t k) {
    if (k == 0) return ld_nt(reinterpret_cast<const u32x4 *>(p));
    const u32x4 *al = reinterpret_cast<const u32x4 *>(
        reinterpret_cast<uintptr_t>(p) - k);
    const u32x4 a = ld_nt(al);
    const u32x4 b = ld_nt(al + 1);
    return funnel_bytes(a, b, k);
}

// Eight fp32 starting at p, whose dword index modulo 4 is q (uniform).
__device__ __forceinline__ void load8f_at(const float *p, uint32_t q, f32x4 &o0,
                                          f32x4 &o1) {
    const f32x4 *al = reinterpret_cast<const f32x4 *>(p - q);
    if (q == 0) {
        o0 = ld_nt(al);
        o1 = ld_nt(al + 1);
        return;
    }
    const f32x4 a = ld_nt(al), b = ld_nt(al + 1), c = ld_nt(al + 2);
    switch (q) {
        case 1:
            o0 = f32x4{a.y, a.z, a.w, b.x};
            o1 = f32x4{b.y, b.z, b.w, c.x};
            break;
        case 2:
            o0 = f32x4{a.z, a.w, b.x, b.y};
            o1 = f32x4{b.z, b.w, c.x, c.y};
            break;
        default:
            o0 = f32x4{a.w, b.x, b.y, b.z};
            o1 = f32x4{b.w, c.x, c.y, c.z};
            break;
    }
}

// fp32 -> bf16 bits, round to nearest even.  bf16 is the top half of an
// fp32; adding 0x7FFF plus the lowest kept bit and truncating rounds the
// dropped half to nearest with ties to even, and carries the largest finite
// values into infinity.  A NaN keeps its sign and leading payload bits and
// gets the quiet bit.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float widen(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// ---------------------------------------------------------------------------
// copy-out: [N, S] bf16 -> full parameters
// ---------------------------------------------------------------------------

__device__ __forceinline__ void copy_run_bf16(uint16_t *dst, const uint16_t *src,
                                              int64_t len) {
    const int tid = threadIdx.x;
    const uint32_t da = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
    int64_t head = ((16u - (da & 15u)) & 15u) >> 1;
    if (head > len) head = len;
    if (tid < head) dst[tid] = src[tid];
    const int64_t rem = len - head;
    const int64_t nvec = rem >> 3;
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    const uint16_t *s = src + head;
    const uint32_t k = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s)) & 15u;
    if (k == 0) {
        const u32x4 *sv = reinterpret_cast<const u32x4 *>(s);
        int64_t v = tid;
        for (; v + 3 * kBlock < nvec; v += 4 * kBlock) {
            const u32x4 x0 = ld_nt(sv + v);
            const u32x4 x1 = ld_nt(sv + v + kBlock);
            const u32x4 x2 = ld_nt(sv + v + 2 * kBlock);
            const u32x4 x3 = ld_nt(sv + v + 3 * kBlock);
            st_nt(dv + v, x0);
            st_nt(dv + v + kBlock, x1);
            st_nt(dv + v + 2 * kBlock, x2);
            st_nt(dv + v + 3 * kBlock, x3);
        }
        for (; v < nvec; v += kBlock) st_nt(dv + v, ld_nt(sv + v));
    } else {
        const u32x4 *sv = reinterpret_cast<const u32x4 *>(
            reinterpret_cast<uintptr_t>(s) - k);
        int64_t v = tid;
        for (; v + kBlock < nvec; v += 2 * kBlock) {
            const u32x4 a0 = ld_nt(sv + v), b0 = ld_nt(sv + v + 1);
            const u32x4 a1 = ld_nt(sv + v + kBlock), b1 = ld_nt(sv + v + kBlock + 1);
            st_nt(dv + v, funnel_bytes(a0, b0, k));
            st_nt(dv + v + kBlock, funnel_bytes(a1, b1, k));
        }
        for (; v < nvec; v += kBlock)
            st_nt(dv + v, funnel_bytes(ld_nt(sv + v), ld_nt(sv + v + 1), k));
    }
    const int64_t done = head + (nvec << 3);
    if (tid < len - done) dst[done + tid] = src[done + tid];
}

__global__ __launch_bounds__(kBlock) void unpack_kernel(
    const UnpackTile *__restrict__ tiles, int64_t n_tiles,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ ag_out) {
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const UnpackTile tl = tiles[t];
        uint16_t *dst = ents[tl.entry].full + tl.dst;
        copy_run_bf16(dst, ag_out + tl.src, tl.len);
    }
}

// ---------------------------------------------------------------------------
// copy-in: fp32 master shards -> bf16 segment (zeros in padding)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void pack_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles,
    const DevEntry *__restrict__ ents, uint16_t *__restrict__ ag_in) {
    const int tid = threadIdx.x;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const PackTile tl = tiles[t];
        uint16_t *dst = ag_in + tl.dst;
        const float *src = ents[tl.entry].master + tl.src;
        const int64_t len = tl.len, valid = tl.valid;
        const uint32_t da = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
        int64_t head = ((16u - (da & 15u)) & 15u) >> 1;
        if (head > len) head = len;
        if (tid < head) dst[tid] = tid < valid ? static_cast<uint16_t>(bf16_rne(src[tid])) : 0;
        const int64_t nvec = (len - head) >> 3;
        u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
        const float *s = src + head;
        const uint32_t q = (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s)) >> 2) & 3u;
        // vectors wholly inside the valid part, then the straddling one, then zeros
        const int64_t vfull = valid > head ? (valid - head) >> 3 : 0;
        int64_t v = tid;
        for (; v + kBlock < vfull; v += 2 * kBlock) {
            f32x4 a0, a1, b0, b1;
            load8f_at(s + (v << 3), q, a0, a1);
            load8f_at(s + ((v + kBlock) << 3), q, b0, b1);
            st_nt(dv + v, u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w),
                                pack2(a1.x, a1.y), pack2(a1.z, a1.w)});
            st_nt(dv + v + kBlock, u32x4{pack2(b0.x, b0.y), pack2(b0.z, b0.w),
                                         pack2(b1.x, b1.y), pack2(b1.z, b1.w)});
        }
        for (; v < vfull; v += kBlock) {
            f32x4 a0, a1;
            load8f_at(s + (v << 3), q, a0, a1);
            st_nt(dv + v, u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w),
                                pack2(a1.x, a1.y), pack2(a1.z, a1.w)});
        }
        for (v = vfull + tid; v < nvec; v += kBlock) {
            const int64_t e0 = head + (v << 3);
            if (e0 >= valid) {
                st_nt(dv + v, u32x4{0u, 0u, 0u, 0u});
            } else {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t e = e0 + 2 * i;
                    const uint32_t lo = e < valid ? bf16_rne(src[e]) : 0u;
                    const uint32_t hi = e + 1 < valid ? bf16_rne(src[e + 1]) : 0u;
                    w[i] = lo | (hi << 16);
                }
                st_nt(dv + v, u32x4{w[0], w[1], w[2], w[3]});
            }
        }
        const int64_t done = head + (nvec << 3);
        const int64_t e = done + tid;
        if (e < len) dst[e] = e < valid ? static_cast<uint16_t>(bf16_rne(src[e])) : 0;
    }
}

// ---------------------------------------------------------------------------
// reduce: [N, S] bf16 contributions -> fp32 mean, this rank's pieces
// ---------------------------------------------------------------------------

// Sum of rows 0..N-1 at element offset `e` (from row 0's base), in order.
__device__ __forceinline__ float sum_rows_scalar(const uint16_t *src0, int64_t S,
                                                 int32_t N, int64_t e) {
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

template <bool kRowsAligned>
__global__ __launch_bounds__(kBlock) void reduce_kernel(
    const ReduceTile *__restrict__ tiles, int64_t n_tiles,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ rs_in,
    int64_t S, int32_t N, float fN) {
    const int tid = threadIdx.x;
    const uint32_t kS = static_cast<uint32_t>((S * 2) & 15);
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const ReduceTile tl = tiles[t];
        float *dst = ents[tl.entry].grad + tl.dst;
        const uint16_t *src0 = rs_in + tl.src;
        const int64_t len = tl.len;
        const uint32_t da = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
        int64_t head = ((16u - (da & 15u)) & 15u) >> 2;
        if (head > len) head = len;
        if (tid < head) dst[tid] = sum_rows_scalar(src0, S, N, tid) / fN;
        const int64_t ngrp = (len - head) >> 3;
        const uint16_t *s0 = src0 + head;
        const uint32_t k0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s0)) & 15u;
        f32x4 *dv = reinterpret_cast<f32x4 *>(dst + head);
        for (int64_t g = tid; g < ngrp; g += kBlock) {
            const uint16_t *p = s0 + (g << 3);
            float acc[8];
            if (kRowsAligned) {
                // every row starts at the same offset modulo 16 bytes
                init8(acc, load16_at(p, k0));
                int32_t j = 1;
                for (; j + 7 < N; j += 8) {
                    u32x4 x[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = load16_at(p + static_cast<int64_t>(j + i) * S, k0);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc8(acc, x[i]);
                }
                for (; j < N; ++j) acc8(acc, load16_at(p + static_cast<int64_t>(j) * S, k0));
            } else {
                init8(acc, load16_at(p, k0));
                uint32_t k = k0;
                for (int32_t j = 1; j < N; ++j) {
                    k = (k + kS) & 15u;
                    acc8(acc, load16_at(p + static_cast<int64_t>(j) * S, k));
                }
            }
            const f32x4 o0{acc[0] / fN, acc[1] / fN, acc[2] / fN, acc[3] / fN};
            const f32x4 o1{acc[4] / fN, acc[5] / fN, acc[6] / fN, acc[7] / fN};
            st_nt(dv + 2 * g, o0);
            st_nt(dv + 2 * g + 1, o1);
        }
        const int64_t done = head + (ngrp << 3);
        const int64_t e = done + tid;
        if (e < len) dst[e] = sum_rows_scalar(src0, S, N, e) / fN;
    }
}

// ---------------------------------------------------------------------------
// AdamW on fp32 shards
// ---------------------------------------------------------------------------

struct AdamwScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps, decay, step_size,
        bc2_sqrt;
};

__device__ __forceinline__ void adamw_elem(float &p, float g, float &m, float &v,
                                           const AdamwScalars &c) {
    p = p * c.decay;
    m = c.beta1 * m + c.one_minus_beta1 * g;
    v = c.beta2 * v + c.one_minus_beta2 * (g * g);
    const float d = __builtin_sqrtf(v) / c.bc2_sqrt + c.eps;
    p = p - c.step_size * (m / d);
}

__global__ __launch_bounds__(kBlock) void adamw_kernel(
    const EwTile *__restrict__ tiles, int64_t n_tiles,
    const DevEntry *__restrict__ ents, AdamwScalars c) {
    const int tid = threadIdx.x;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const EwTile tl = tiles[t];
        const DevEntry en = ents[tl.entry];
        float *P = en.master + tl.off;
        const float *G = en.grad + tl.off;
        float *M = en.exp_avg + tl.off;
        float *Vv = en.exp_avg_sq + tl.off;
        const int64_t len = tl.len;
        const uint32_t ap = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(P)) & 15u;
        const bool same = ap == (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(G)) & 15u) &&
                          ap == (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(M)) & 15u) &&
                          ap == (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(Vv)) & 15u);
        if (!same) {
            for (int64_t i = tid; i < len; i += kBlock) {
                float p = P[i], m = M[i], v = Vv[i];
                adamw_elem(p, G[i], m, v, c);
                P[i] = p;
                M[i] = m;
                Vv[i] = v;
            }
            continue;
        }
        int64_t head = ((16u - ap) & 15u) >> 2;
        if (head > len) head = len;
        if (tid < head) {
            float p = P[tid], m = M[tid], v = Vv[tid];
            adamw_elem(p, G[tid], m, v, c);
            P[tid] = p;
            M[tid] = m;
            Vv[tid] = v;
        }
        const int64_t nvec = (len - head) >> 2;
        f32x4 *pv = reinterpret_cast<f32x4 *>(P + head);
        const f32x4 *gv = reinterpret_cast<const f32x4 *>(G + head);
        f32x4 *mv = reinterpret_cast<f32x4 *>(M + head);
        f32x4 *vv = reinterpret_cast<f32x4 *>(Vv + head);
        for (int64_t i = tid; i < nvec; i += kBlock) {
            const f32x4 g = ld_nt(gv + i);
            f32x4 p = ld_nt(pv + i), m = ld_nt(mv + i), v = ld_nt(vv + i);
            float pe[4] = {p.x, p.y, p.z, p.w}, me[4] = {m.x, m.y, m.z, m.w},
                  ve[4] = {v.x, v.y, v.z, v.w};
            const float ge[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) adamw_elem(pe[k], ge[k], me[k], ve[k], c);
            st_nt(pv + i, f32x4{pe[0], pe[1], pe[2], pe[3]});
            st_nt(mv + i, f32x4{me[0], me[1], me[2], me[3]});
            st_nt(vv + i, f32x4{ve[0], ve[1], ve[2], ve[3]});
        }
        const int64_t e = head + (nvec << 2) + tid;
        if (e < len) {
            float p = P[e], m = M[e], v = Vv[e];
            adamw_elem(p, G[e], m, v, c);
            P[e] = p;
            M[e] = m;
            Vv[e] = v;
        }
    }
}

inline unsigned grid_for(int64_t n_tiles) {
    constexpr int64_t kMaxGrid = 1 << 20;
    return static_cast<unsigned>(n_tiles < kMaxGrid ? n_tiles : kMaxGrid);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------

hipError_t launch_pack(const PackTile *tiles, int64_t n, const DevEntry *ents,
                       uint16_t *ag_in, hipStream_t st) {
    if (n == 0) return hipSuccess;
    pack_kernel<<<grid_for(n), kBlock, 0, st>>>(tiles, n, ents, ag_in);
    return hipGetLastError();
}

hipError_t launch_unpack(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *ag_out, hipStream_t st) {
    if (n == 0) return hipSuccess;
    unpack_kernel<<<grid_for(n), kBlock, 0, st>>>(tiles, n, ents, ag_out);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *rs_in, int64_t S, int32_t N, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const float fN = static_cast<float>(N);
    if (((S * 2) & 15) == 0)
        reduce_kernel<true><<<grid_for(n), kBlock, 0, st>>>(tiles, n, ents, rs_in, S, N, fN);
    else
        reduce_kernel<false><<<grid_for(n), kBlock, 0, st>>>(tiles, n, ents, rs_in, S, N, fN);
    return hipGetLastError();
}

hipError_t launch_adamw(const EwTile *tiles, int64_t n, const DevEntry *ents,
                        const float scal[8], hipStream_t st) {
    if (n == 0) return hipSuccess;
    AdamwScalars c{scal[0], scal[1], scal[2], scal[3], scal[4], scal[5], scal[6], scal[7]};
    adamw_kernel<<<grid_for(n), kBlock, 0, st>>>(tiles, n, ents, c);
    return hipGetLastError();
}

}  // namespace fsdp
