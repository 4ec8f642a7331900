// Copies of the sharded step: the all-gather copy-out ([N, S] bf16 -> full
// parameters), the reduce-scatter copy-ins (full gradients or fp32
// accumulators -> [N, S]), the FP8 copy-out and the resharding executor.
// Pure data movement at the HBM roofline: 16-byte vectors, raw buffer loads
// from one descriptor per run, misaligned sources funnel-shifted in
// registers with each chunk read once.
#include "device.hpp"
#include "launch.hpp"

// copy-out and the two-byte copies: non-temporal loads and stores
#ifndef FSDP_UNPACK_POL
#define FSDP_UNPACK_POL 3
#endif
// copy-out blocks: 2048 elements over 128 threads when every row piece is
// 16-byte aligned, 4096 over 256 otherwise; the other two-byte copies (bf16
// reduce-scatter copy-in, resharding) and the FP8 copy-out (4096 bytes) take
// the 128-thread shape.  Copy-out measured on MI355X, two chunks per lane,
// Llama 7B and 70B shapes: 128 threads 6.26 and 6.60 TB/s, 64 threads 6.18
// and 6.52, 256 threads 6.05 and 6.41, 512 threads 6.12 and 6.36; misaligned
// ragged rows: 256 threads 5.77-5.89, 128 threads 5.62-5.73.
#ifndef FSDP_UNPACK_SUB
#define FSDP_UNPACK_SUB 2048
#endif
#ifndef FSDP_UNPACK_THREADS
#define FSDP_UNPACK_THREADS 128
#endif
#ifndef FSDP_UNPACK_MIS_SUB
#define FSDP_UNPACK_MIS_SUB 4096
#endif
#ifndef FSDP_UNPACK_MIS_THREADS
#define FSDP_UNPACK_MIS_THREADS 256
#endif
// LDS the copy-out and the bf16 reduce-scatter copy-in reserve, and never
// touch, on misaligned rows, so that 6 of their 256-thread blocks share a CU
// (160 KB of LDS per CU): on the ragged MoE rows the copy-out 6.09-6.14 ->
// 6.24-6.29 TB/s, the copy-in 6.00-6.03 -> 6.13-6.19 and the step
// 1.072-1.077 -> 1.062-1.070 ms (7 blocks alike, 5 in between; on aligned
// rows the 128-thread copies gained nothing at 6 waves per SIMD and the FP8
// copy-out lost 3.5%)
#ifndef FSDP_COPY_MIS_LDS
#define FSDP_COPY_MIS_LDS 24576
#endif
// 16-byte chunks each lane of an aligned copy loads before storing them (4
// or 8 with correspondingly larger blocks measured 9-16% slower)
#ifndef FSDP_UNPACK_UNROLL
#define FSDP_UNPACK_UNROLL 2
#endif
// reduce-scatter copy-ins widening to fp32 and from the fp32 accumulators,
// and the accumulation itself: non-temporal loads and stores
#ifndef FSDP_RSPACK_F32_POL
#define FSDP_RSPACK_F32_POL 3
#endif
#ifndef FSDP_RSPACK_ACC_POL
#define FSDP_RSPACK_ACC_POL 3
#endif
// LDS the copy-in from the accumulators reserves and never touches, so that
// 6 of its 256-thread blocks share a CU (160 KB of LDS per CU): 6.07 -> 6.37
// TB/s on the 70B shape, +1.5% on the 7B shape and +1.8% on the ragged MoE
// rows.  The reductions, the accumulation, the other copy-ins and the FP8
// copy-in measured slower at 6, 5, 4 or 3 blocks per CU.
#ifndef FSDP_RSPACK_ACC_LDS
#define FSDP_RSPACK_ACC_LDS 24576
#endif
// the same for the fp32 reduce-scatter copy-in on misaligned rows, 5 blocks
// per CU: 5.42-5.47 -> 5.70-5.74 TB/s on the ragged MoE rows (6 blocks
// +3%, 4 +2%, 3 -10%)
#ifndef FSDP_RSPACK_F32_MIS_LDS
#define FSDP_RSPACK_F32_MIS_LDS 28672
#endif

namespace fsdp {

namespace {

// ---------------------------------------------------------------------------
// copy-out: [N, S] bf16 -> full parameters
// ---------------------------------------------------------------------------

// TB threads per block (whole waves).
template <int POL, int TB = kBlock>
__device__ __forceinline__ void copy_run_bf16(uint16_t *__restrict__ dst,
                                              const uint16_t *__restrict__ src, int64_t len) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = ((16u - (lo32(dst) & 15u)) & 15u) >> 1;
    if (head > len) head = len;
    if (tid < head) dst[tid] = src[tid];
    const int64_t nvec = (len - head) >> 3;
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    const uint16_t *s = src + head;
    const uint32_t k = lo32(s) & 15u;
    if (k == 0) {
        // raw buffer loads from one SGPR descriptor per run (measured faster
        // than per-lane 64-bit addresses on MI355X)
        // FSDP_UNPACK_UNROLL chunks in flight per lane before their stores
        constexpr int U = FSDP_UNPACK_UNROLL;
        const char *sb = reinterpret_cast<const char *>(s);
        const uint32_t nb = static_cast<uint32_t>(nvec) << 4;
        int64_t v = tid;
        for (; v + (U - 1) * TB < nvec; v += U * TB) {
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[u] = bload16<LN>(sb, static_cast<uint32_t>(v + u * TB) << 4, nb);
#pragma unroll
            for (int u = 0; u < U; ++u) stp<SN>(dv + v + u * TB, x[u]);
        }
        for (; v < nvec; v += TB)
            stp<SN>(dv + v, bload16<LN>(sb, static_cast<uint32_t>(v) << 4, nb));
    } else {
        // Every aligned 16-byte source chunk is read once: a lane's second
        // chunk is the next lane's first (DPP), and lane 63 of each wave
        // loads its own with a load whose other lanes sit at the end of the
        // buffer range (they read zero and touch no memory).  The range is
        // exactly the chunks holding data, and whole waves iterate together.
        // Lane 63's chunk opens the span another wave reads, so it is loaded
        // with a temporal hint and stays in L2 for that wave (kBoundaryNT).
        const char *al = reinterpret_cast<const char *>(s) - k;
        const uint32_t nb = (k + 2 * static_cast<uint32_t>(len - head) + 15u) & ~15u;
        // stores through a buffer range of exactly the run's vectors: lanes
        // past the end are dropped without a branch, which would let the
        // compiler sink a boundary load under it (see next_or_own)
        char *db = reinterpret_cast<char *>(dv);
        const uint32_t dn = static_cast<uint32_t>(nvec) << 4;
        const uint32_t lane = tid & 63;
        const bool last = lane == 63;
        for (int64_t w0 = tid - lane; w0 < nvec; w0 += 2 * TB) {
            const int64_t v0 = w0 + lane, v1 = v0 + TB;
            const uint32_t o0 = static_cast<uint32_t>(v0) << 4, o1 = static_cast<uint32_t>(v1) << 4;
            const u32x4 a0 = bload16<LN>(al, o0, nb), a1 = bload16<LN>(al, o1, nb);
            const u32x4 h0 = bload16<kBoundaryNT>(al, last ? o0 + 16 : nb, nb);
            const u32x4 h1 = bload16<kBoundaryNT>(al, last ? o1 + 16 : nb, nb);
            const u32x4 b0 = next_or_own(a0, h0), b1 = next_or_own(a1, h1);
            bstore16<SN>(db, o0, dn, funnel(a0, b0, k));
            bstore16<SN>(db, o1, dn, funnel(a1, b1, k));
        }
    }
    const int64_t done = head + (nvec << 3);
    if (tid < len - done) dst[done + tid] = src[done + tid];
}

template <int POL, int TB, bool kRemap>
__global__ __launch_bounds__(TB) void unpack_kernel(
    const UnpackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ ag_out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt<kRemap>(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const UnpackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        copy_run_bf16<POL, TB>(ents[tl.entry].full + tl.dst + b, ag_out + tl.src + b, len);
    }
}

// Resharding: runs of 2-byte units between absolute addresses.
template <int POL, int TB>
__global__ __launch_bounds__(TB) void copy_runs_kernel(const CopyTile *__restrict__ tiles,
                                                           int64_t n_tiles, int32_t split,
                                                           int64_t sub) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const CopyTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        copy_run_bf16<POL, TB>(tl.dst + b, tl.src + b, len);
    }
}

// ---------------------------------------------------------------------------
// reduce-scatter copy-in: full bf16 gradients -> [N, S] (bf16 or fp32)
// ---------------------------------------------------------------------------

template <int POL, int TB, bool kRemap>
__global__ __launch_bounds__(TB) void rspack_bf16_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, uint16_t *__restrict__ out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt<kRemap>(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        uint16_t *dst = out + tl.dst + b;
        if (valid > 0) copy_run_bf16<POL, TB>(dst, ents[tl.entry].full_grad + tl.src + b, valid);
        zero_bf16<(POL >> 1) & 1>(dst, valid, len);
    }
}

// dst[e] = 0.0f for e in [from, len), 16-byte stores where aligned.
template <int SN>
__device__ __forceinline__ void zero_f32(float *dst, int64_t from, int64_t len) {
    const int tid = threadIdx.x;
    if (from >= len) return;
    float *d = dst + from;
    const int64_t n = len - from;
    int64_t head = ((16u - (lo32(d) & 15u)) & 15u) >> 2;
    if (head > n) head = n;
    if (tid < head) d[tid] = 0.0f;
    const int64_t nvec = (n - head) >> 2;
    f32x4 *dv = reinterpret_cast<f32x4 *>(d + head);
    for (int64_t v = tid; v < nvec; v += kBlock) stp<SN>(dv + v, f32x4{0.f, 0.f, 0.f, 0.f});
    const int64_t done = head + (nvec << 2);
    if (tid < n - done) d[done + tid] = 0.0f;
}

// dst[i] = fp32(src[i]) for i < valid (exact widening), zeros up to len.
// dst is aligned to 16 bytes after a short head; every lane then widens four
// elements into one 16-byte store, so each wave instruction is contiguous.
// An 8-byte aligned source is one 8-byte load per lane.  Otherwise lane l
// loads the 8-byte word holding its first element, takes the next word from
// lane l + 1 (DPP; lane 63 loads its own from a load whose other lanes sit
// at the end of the buffer range), and funnel-shifts: every source word is
// read once, and whole waves iterate together.
template <int POL>
__device__ __forceinline__ void widen_run(float *__restrict__ dst, const uint16_t *__restrict__ src,
                                          int64_t len, int64_t valid) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = ((16u - (lo32(dst) & 15u)) & 15u) >> 2;
    if (head > valid) head = valid;
    if (tid < head) dst[tid] = widen(src[tid]);
    const uint16_t *s = src + head;
    const uint32_t k = lo32(s) & 15u;
    f32x4 *dv = reinterpret_cast<f32x4 *>(dst + head);
    int64_t done;
    if ((k & 7u) == 0) {
        const int64_t nq = (valid - head) >> 2;
        const u32x2 *sv = reinterpret_cast<const u32x2 *>(s);
        // two loads a block apart before their stores (+1-2%; the fp32 copy
        // from the accumulators measured 5% slower that way and keeps one)
        int64_t q = tid;
        for (; q + kBlock < nq; q += 2 * kBlock) {
            const u32x2 w0 = ldp<LN>(sv + q), w1 = ldp<LN>(sv + q + kBlock);
            stp<SN>(dv + q, f32x4{bf16_lo(w0.x), bf16_hi(w0.x), bf16_lo(w0.y), bf16_hi(w0.y)});
            stp<SN>(dv + q + kBlock,
                    f32x4{bf16_lo(w1.x), bf16_hi(w1.x), bf16_lo(w1.y), bf16_hi(w1.y)});
        }
        for (; q < nq; q += kBlock) {
            const u32x2 w = ldp<LN>(sv + q);
            stp<SN>(dv + q, f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)});
        }
        done = head + (nq << 2);
    } else {
        const uint32_t k8 = k & 7u;                     // 2, 4 or 6
        const char *al = reinterpret_cast<const char *>(s) - k8;
        const int64_t nq = (valid - head) >> 2;
        const uint32_t nb = (k8 + 2 * static_cast<uint32_t>(valid - head) + 7u) & ~7u;
        const uint32_t lane = tid & 63;
        const bool last = lane == 63, s4 = k8 >= 4u;
        const uint32_t sh = k8 & 3u;
        char *db = reinterpret_cast<char *>(dv);     // bounded stores, as in copy_run_bf16
        const uint32_t dn = static_cast<uint32_t>(nq) << 4;
        // two words a block apart per lane, both loaded before either is
        // used (one per iteration measured 6% slower on the ragged MoE rows)
        for (int64_t w0 = tid - lane; w0 < nq; w0 += 2 * kBlock) {
            u32x2 a[2], h[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t o = static_cast<uint32_t>(w0 + lane + u * kBlock) << 3;
                a[u] = bload8<LN>(al, o, nb);
                h[u] = bload8<kBoundaryNT>(al, last ? o + 8 : nb, nb);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t q = static_cast<uint32_t>(w0 + lane + u * kBlock);
                const u32x2 b = next_or_own(a[u], h[u]);
                // bytes [k8, k8 + 8) of a:b
                const uint32_t u0 = s4 ? a[u].y : a[u].x, u1 = s4 ? b.x : a[u].y;
                const uint32_t u2 = s4 ? b.y : b.x;
                const uint32_t r0 = __builtin_amdgcn_alignbyte(u1, u0, sh);
                const uint32_t r1 = __builtin_amdgcn_alignbyte(u2, u1, sh);
                bstore16<SN>(db, q << 4, dn,
                             __builtin_bit_cast(u32x4, f32x4{bf16_lo(r0), bf16_hi(r0),
                                                             bf16_lo(r1), bf16_hi(r1)}));
            }
        }
        done = head + (nq << 2);
    }
    if (tid < valid - done) dst[done + tid] = widen(src[done + tid]);
    zero_f32<SN>(dst, valid, len);
}

template <int POL, bool kRemap>
__global__ __launch_bounds__(kBlock) void rspack_f32_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, float *__restrict__ out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt<kRemap>(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        widen_run<POL>(out + tl.dst + b, ents[tl.entry].full_grad + tl.src + b, len, valid);
    }
}

template <int POL, int TB = kBlock>
__device__ __forceinline__ void copy_run_u8(uint8_t *__restrict__ dst, const uint8_t *__restrict__ src,
                                            int64_t len) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = (16u - (lo32(dst) & 15u)) & 15u;
    if (head > len) head = len;
    if (tid < head) dst[tid] = src[tid];
    const int64_t nvec = (len - head) >> 4;
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    const uint8_t *s = src + head;
    const uint32_t k = lo32(s) & 15u;
    // raw buffer loads over exactly the 16-byte chunks holding the run; a
    // misaligned run reads every chunk once, a lane's second chunk coming
    // from the next lane (lane 63 loads its own), as in copy_run_bf16
    const char *al = reinterpret_cast<const char *>(s) - k;
    const uint32_t nb = (k + static_cast<uint32_t>(len - head) + 15u) & ~15u;
    if (k == 0) {
        for (int64_t v = tid; v < nvec; v += TB)
            stp<SN>(dv + v, bload16<LN>(al, static_cast<uint32_t>(v) << 4, nb));
    } else {
        char *db = reinterpret_cast<char *>(dv);     // bounded stores, as in copy_run_bf16
        const uint32_t dn = static_cast<uint32_t>(nvec) << 4;
        const uint32_t lane = tid & 63;
        const bool last = lane == 63;
        for (int64_t w0 = tid - lane; w0 < nvec; w0 += TB) {
            const uint32_t o = static_cast<uint32_t>(w0 + lane) << 4;
            const u32x4 a = bload16<LN>(al, o, nb);
            const u32x4 h = bload16<kBoundaryNT>(al, last ? o + 16 : nb, nb);
            const u32x4 b = next_or_own(a, h);
            bstore16<SN>(db, o, dn, funnel(a, b, k));
        }
    }
    const int64_t done = head + (nvec << 4);
    if (tid < len - done) dst[done + tid] = src[done + tid];
}

template <int POL, int TB, bool kRemap>
__global__ __launch_bounds__(TB) void unpack_fp8_kernel(
    const UnpackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint8_t *__restrict__ ag_out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt<kRemap>(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const UnpackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        copy_run_u8<POL, TB>(ents[tl.entry].full_fp8 + tl.dst + b, ag_out + tl.src + b, len);
    }
}

// Reduce-scatter copy-in from the fp32 accumulators: copy fp32 runs, zeros
// in padding.  dst is aligned to 16 bytes after a short head; every lane then
// stores one 16-byte vector, so each wave instruction is contiguous.  An
// aligned source is one load per lane; otherwise lane l loads the aligned
// chunk holding its first element, takes the next chunk from lane l + 1
// (DPP; lane 63 loads its own) and shifts by whole dwords.
template <int POL>
__device__ __forceinline__ void copy_f32_run(float *__restrict__ dst, const float *__restrict__ src,
                                             int64_t len, int64_t valid) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = ((16u - (lo32(dst) & 15u)) & 15u) >> 2;
    if (head > valid) head = valid;
    if (tid < head) dst[tid] = src[tid];
    const float *s = src + head;
    const uint32_t q = (lo32(s) >> 2) & 3u;
    f32x4 *dv = reinterpret_cast<f32x4 *>(dst + head);
    int64_t done;
    if (q == 0) {
        const int64_t nq = (valid - head) >> 2;
        const f32x4 *sv = reinterpret_cast<const f32x4 *>(s);
        for (int64_t v = tid; v < nq; v += kBlock) stp<SN>(dv + v, ldp<LN>(sv + v));
        done = head + (nq << 2);
    } else {
        const char *al = reinterpret_cast<const char *>(s) - 4 * q;
        const int64_t nv = (valid - head) >> 2;
        const uint32_t nb = (4 * q + 4 * static_cast<uint32_t>(valid - head) + 15u) & ~15u;
        char *db = reinterpret_cast<char *>(dv);     // bounded stores, as in copy_run_bf16
        const uint32_t dn = static_cast<uint32_t>(nv) << 4;
        const uint32_t lane = tid & 63;
        const bool last = lane == 63;
        // two chunks a block apart per lane, as in widen_run (one per
        // iteration measured 5% slower on the ragged MoE rows)
        for (int64_t w0 = tid - lane; w0 < nv; w0 += 2 * kBlock) {
            u32x4 a[2], h[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t o = static_cast<uint32_t>(w0 + lane + u * kBlock) << 4;
                a[u] = bload16<LN>(al, o, nb);
                h[u] = bload16<kBoundaryNT>(al, last ? o + 16 : nb, nb);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t v = static_cast<uint32_t>(w0 + lane + u * kBlock);
                const u32x4 b = next_or_own(a[u], h[u]);
                bstore16<SN>(db, v << 4, dn, funnel(a[u], b, 4 * q));
            }
        }
        done = head + (nv << 2);
    }
    if (tid < valid - done) dst[done + tid] = src[done + tid];
    zero_f32<SN>(dst, valid, len);
}

template <int POL, bool kRemap>
__global__ __launch_bounds__(kBlock) void rspack_acc_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, float *__restrict__ out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = first_vt<kRemap>(); vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        copy_f32_run<POL>(out + tl.dst + b, ents[tl.entry].grad_acc + tl.src + b, len, valid);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------

// Row pieces 16-byte aligned: FSDP_UNPACK_THREADS threads per block over
// FSDP_UNPACK_SUB elements; otherwise FSDP_UNPACK_MIS_THREADS over
// FSDP_UNPACK_MIS_SUB (both correct for any alignment; measured per case).
hipError_t launch_unpack(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *ag_out, bool chunk_aligned, hipStream_t st) {
    if (n == 0) return hipSuccess;
    if (chunk_aligned) {
        const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_SUB);
        unpack_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS, false>
            <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp,
                                                              ents, ag_out);
    } else {
        const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_MIS_SUB);
        unpack_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_MIS_THREADS, true>
            <<<grid_for(n, sp), FSDP_UNPACK_MIS_THREADS, FSDP_COPY_MIS_LDS, st>>>(
                tiles, n, sp, kTileUnpack / sp, ents, ag_out);
    }
    return hipGetLastError();
}

hipError_t launch_copy_runs(const CopyTile *tiles, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_SUB);
    copy_runs_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS>
        <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp);
    return hipGetLastError();
}

hipError_t launch_unpack_fp8(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                             const uint8_t *ag_out, bool chunk_aligned, hipStream_t st) {
    if (n == 0) return hipSuccess;
    // 16 bytes per lane move 16 elements: twice the elements per block of bf16
    const int32_t sp = split_for(kTileUnpack, 2 * FSDP_UNPACK_SUB);
    if (chunk_aligned)
        unpack_fp8_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS, false>
            <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp,
                                                              ents, ag_out);
    else
        unpack_fp8_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS, true>
            <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp,
                                                              ents, ag_out);
    return hipGetLastError();
}

hipError_t launch_rspack_acc(const PackTile *tiles, int64_t n, const DevEntry *ents, float *out,
                             bool chunk_aligned, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_SUB);
    if (chunk_aligned)
        rspack_acc_kernel<FSDP_RSPACK_ACC_POL, false><<<grid_for(n, sp), kBlock, FSDP_RSPACK_ACC_LDS, st>>>(
            tiles, n, sp, kTileUnpack / sp, ents, out);
    else
        rspack_acc_kernel<FSDP_RSPACK_ACC_POL, true><<<grid_for(n, sp), kBlock, FSDP_RSPACK_ACC_LDS, st>>>(
            tiles, n, sp, kTileUnpack / sp, ents, out);
    return hipGetLastError();
}

// Block shapes as the copy-out's, chosen by whether every row piece of the
// output is 16-byte aligned; misaligned rows take the XCD remap (first_vt).
hipError_t launch_rspack(const PackTile *tiles, int64_t n, const DevEntry *ents, void *out,
                         bool f32, bool chunk_aligned, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileUnpack, chunk_aligned ? FSDP_UNPACK_SUB : FSDP_UNPACK_MIS_SUB);
    const unsigned grid = grid_for(n, sp);
    if (f32 && chunk_aligned)
        rspack_f32_kernel<FSDP_RSPACK_F32_POL, false><<<grid, kBlock, 0, st>>>(
            tiles, n, sp, kTileUnpack / sp, ents, static_cast<float *>(out));
    else if (f32)
        rspack_f32_kernel<FSDP_RSPACK_F32_POL, true><<<grid, kBlock, FSDP_RSPACK_F32_MIS_LDS, st>>>(
            tiles, n, sp, kTileUnpack / sp, ents, static_cast<float *>(out));
    else if (chunk_aligned)
        rspack_bf16_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS, false>
            <<<grid, FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp, ents,
                                                   static_cast<uint16_t *>(out));
    else
        rspack_bf16_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_MIS_THREADS, true>
            <<<grid, FSDP_UNPACK_MIS_THREADS, FSDP_COPY_MIS_LDS, st>>>(
                tiles, n, sp, kTileUnpack / sp, ents, static_cast<uint16_t *>(out));
    return hipGetLastError();
}

}  // namespace fsdp
