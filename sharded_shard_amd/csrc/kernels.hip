// HIP kernels of one rank's FSDP2 sharded step, written for CDNA4 (gfx950).
//
// All kernels stream HBM and do little arithmetic, so the design rules are the
// memory-bound ones: 16-byte (dwordx4) coalesced loads and stores, several
// independent loads in flight per lane, a cache policy chosen per stream
// (non-temporal for data touched once, where it measured faster), no LDS.
//
// Work decomposition.  The host planner (plan.cpp) cuts every run of every
// parameter into tiles of kTile* elements and uploads the tile table once.  A
// launch has `split` blocks per tile: block b serves tile b / split,
// sub-range b % split of kTile / split elements.  The table stays small (one 16- or
// 32-byte record per tile) while each block moves only a few KB, which keeps
// all 256 CUs busy to the end of the launch.  Blocks read their tile record
// and one entry record with scalar loads, then stream.  Grids are
// grid-strided, so any grid size is correct.
//
// Alignment.  Pieces of a group sit back to back with no gap by default, so a
// run can start at any 2-byte (bf16) or 4-byte (fp32) address.  Destinations
// are written in 16-byte vectors after a short element-wise head; sources
// that are misaligned relative to the destination are read as aligned 16-byte
// vectors and funnel-shifted in registers (v_alignbyte).  A 16-byte aligned
// vector never crosses a page, and every vector loaded holds at least one byte
// of the run, so these reads never touch unmapped memory.
//
// Numerics (built with -ffp-contract=off and correctly rounded fp32 divide
// and square root): reductions add rank contributions in rank order starting
// from rank 0's value, then divide once by N; AdamW performs each operation
// as one fp32 rounding in the order documented in the C header; bf16 casts
// round to nearest even.  The fused step uses the same device functions in
// the same order, so its results equal the three separate calls bit for bit.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

// Cache policy per kernel: bit 0 = non-temporal loads, bit 1 = non-temporal
// stores.  Elements per block (sub-range) per kernel; for the kernels that
// read all N rows per element, the sub-range shrinks as N grows
// (FSDP_ROWS_BUDGET row-elements per block, at least FSDP_MIN_SUB).  Rows in
// flight per lane: the fused step keeps FSDP_STEP_ROW_BATCH rows (aligned)
// or FSDP_STEP_GEN_ROW_BATCH rows (misaligned) outstanding up to 8 ranks and
// FSDP_STEP_ROW_BATCH_WIDE beyond, the plain reductions
// FSDP_REDUCE_ROW_BATCH (measured on MI355X: more rows in flight per wave
// spread each wave over more DRAM pages).
#ifndef FSDP_UNPACK_POL
#define FSDP_UNPACK_POL 3
#endif
#ifndef FSDP_REDUCE_POL
#define FSDP_REDUCE_POL 1
#endif
// the bf16 reduction on aligned rows below the wide threshold: a quad per
// lane, non-temporal loads and stores
#ifndef FSDP_REDUCE_QUAD_POL
#define FSDP_REDUCE_QUAD_POL 3
#endif
// Lanes of the fp32 reduction store two 16-byte halves of a 32-byte span per
// group: non-temporal stores of that pattern cost extra HBM writes (measured
// 1.1-1.7x the algorithmic bytes), plain stores do not.  The fp32 copy-ins
// and the accumulation move four elements per lane, so every store
// instruction of a wave writes 1 KB contiguously, and take non-temporal
// loads and stores.
#ifndef FSDP_REDUCE_F32_POL
#define FSDP_REDUCE_F32_POL 0
#endif
// the fp32 reduction on aligned rows: a vector per lane, non-temporal loads
// and stores
#ifndef FSDP_REDUCE_F32_QUAD_POL
#define FSDP_REDUCE_F32_QUAD_POL 3
#endif
#ifndef FSDP_RSPACK_F32_POL
#define FSDP_RSPACK_F32_POL 3
#endif
#ifndef FSDP_RSPACK_ACC_POL
#define FSDP_RSPACK_ACC_POL 3
#endif
#ifndef FSDP_ACC_POL
#define FSDP_ACC_POL 3
#endif
// AdamW: plain loads and stores (non-temporal ones measured faster for the
// kernel itself but slowed the copy-in and copy-out after it by more)
#ifndef FSDP_ADAMW_POL
#define FSDP_ADAMW_POL 0
#endif
#ifndef FSDP_PACK_POL
#define FSDP_PACK_POL 3
#endif
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
// 16-byte chunks each lane of an aligned copy loads before storing them (4
// or 8 with correspondingly larger blocks measured 9-16% slower)
#ifndef FSDP_UNPACK_UNROLL
#define FSDP_UNPACK_UNROLL 2
#endif
#ifndef FSDP_ADAMW_SUB
#define FSDP_ADAMW_SUB 4096
#endif
#ifndef FSDP_PACK_SUB
#define FSDP_PACK_SUB 2048
#endif
#ifndef FSDP_FP8_POL
#define FSDP_FP8_POL 0
#endif
#ifndef FSDP_FP8_SUB
#define FSDP_FP8_SUB 4096
#endif
#ifndef FSDP_ROWS_BUDGET
#define FSDP_ROWS_BUDGET 32768
#endif
#ifndef FSDP_MIN_SUB
#define FSDP_MIN_SUB 512
#endif
#ifndef FSDP_STEP_ROW_BATCH
#define FSDP_STEP_ROW_BATCH 2
#endif
#ifndef FSDP_STEP_ROW_BATCH_WIDE
#define FSDP_STEP_ROW_BATCH_WIDE 4
#endif
// rows in flight of the fused step on misaligned rows up to 8 ranks
#ifndef FSDP_STEP_GEN_ROW_BATCH
#define FSDP_STEP_GEN_ROW_BATCH 1
#endif
#ifndef FSDP_REDUCE_ROW_BATCH
#define FSDP_REDUCE_ROW_BATCH 2
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
// occupancy target of the wide fused step (waves per SIMD)
#ifndef FSDP_STEP_WIDE_WAVES
#define FSDP_STEP_WIDE_WAVES 4
#endif
// The same for the plain reduction of bf16 contributions (fp32
// contributions measured slower read this way: 5.65 vs 5.87 TB/s at N = 64).
#ifndef FSDP_REDUCE_WIDE
#define FSDP_REDUCE_WIDE 4
#endif
#ifndef FSDP_REDUCE_WIDE_MIN_N
#define FSDP_REDUCE_WIDE_MIN_N 16
#endif
// threads per block of the fused step below the wide kernel (at most kBlock)
#ifndef FSDP_STEP_THREADS
#define FSDP_STEP_THREADS 256
#endif
#ifndef FSDP_STEP_WAVES
#define FSDP_STEP_WAVES 6
#endif
// the fused step reads its N gradient rows with non-temporal loads
#ifndef FSDP_STEP_ROW_NT
#define FSDP_STEP_ROW_NT 1
#endif
// occupancy target of the fused step on misaligned rows (0: the default)
#ifndef FSDP_STEP_GEN_WAVES
#define FSDP_STEP_GEN_WAVES 0
#endif
#if FSDP_STEP_GEN_WAVES > 0
#define FSDP_STEP_GEN_ATTR __attribute__((amdgpu_waves_per_eu(FSDP_STEP_GEN_WAVES)))
#else
#define FSDP_STEP_GEN_ATTR
#endif
// occupancy target of the AdamW kernel (0: the compiler's default)
#ifndef FSDP_ADAMW_WAVES
#define FSDP_ADAMW_WAVES 0
#endif
#if FSDP_ADAMW_WAVES > 0
#define FSDP_ADAMW_ATTR __attribute__((amdgpu_waves_per_eu(FSDP_ADAMW_WAVES)))
#else
#define FSDP_ADAMW_ATTR
#endif
#ifndef FSDP_ROW_BLOCK_FIT
#define FSDP_ROW_BLOCK_FIT 0
#endif

namespace fsdp {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef FSDP_BLOCK
#define FSDP_BLOCK 256
#endif
constexpr int kBlock = FSDP_BLOCK;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

template <int NT, typename T>
__device__ __forceinline__ T ldp(const T *p) {
    if constexpr (NT != 0) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int NT, typename T>
__device__ __forceinline__ void stp(T *p, T v) {
    if constexpr (NT != 0) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__device__ __forceinline__ uint32_t lo32(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ uint32_t alignbyte2(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// Bytes [k, k + 16) of the 32-byte little-endian concatenation a:b, for a
// wave-uniform k in [0, 16), without branches: an 8-byte and a 4-byte select
// step, then a byte align of the remaining 0..3 bytes.  Branch-free so that
// no wait for the loads lands between them and the next iteration's loads.
__device__ __forceinline__ u32x4 funnel(u32x4 a, u32x4 b, uint32_t k) {
    const bool s8 = (k & 8u) != 0, s4 = (k & 4u) != 0;
    const uint32_t u0 = s8 ? a.z : a.x, u1 = s8 ? a.w : a.y, u2 = s8 ? b.x : a.z;
    const uint32_t u3 = s8 ? b.y : a.w, u4 = s8 ? b.z : b.x, u5 = s8 ? b.w : b.y;
    const uint32_t v0 = s4 ? u1 : u0, v1 = s4 ? u2 : u1, v2 = s4 ? u3 : u2;
    const uint32_t v3 = s4 ? u4 : u3, v4 = s4 ? u5 : u4;
    const uint32_t sh = k & 3u;
    return u32x4{__builtin_amdgcn_alignbyte(v1, v0, sh), __builtin_amdgcn_alignbyte(v2, v1, sh),
                 __builtin_amdgcn_alignbyte(v3, v2, sh), __builtin_amdgcn_alignbyte(v4, v3, sh)};
}

// Dwords [q, q + 8) of the 12 dwords a:b:c, q in [0, 4) wave-uniform,
// without branches.
__device__ __forceinline__ void select8f(f32x4 a, f32x4 b, f32x4 c, uint32_t q, f32x4 &o0,
                                         f32x4 &o1) {
    const bool s2 = (q & 2u) != 0, s1 = (q & 1u) != 0;
    // u = dwords [2*s2, 2*s2 + 10), then o = u[s1 .. s1 + 8)
    const float u0 = s2 ? a.z : a.x, u1 = s2 ? a.w : a.y, u2 = s2 ? b.x : a.z;
    const float u3 = s2 ? b.y : a.w, u4 = s2 ? b.z : b.x, u5 = s2 ? b.w : b.y;
    const float u6 = s2 ? c.x : b.z, u7 = s2 ? c.y : b.w, u8 = s2 ? c.z : c.x;
    const float u9 = s2 ? c.w : c.y;
    o0 = f32x4{s1 ? u1 : u0, s1 ? u2 : u1, s1 ? u3 : u2, s1 ? u4 : u3};
    o1 = f32x4{s1 ? u5 : u4, s1 ? u6 : u5, s1 ? u7 : u6, s1 ? u8 : u7};
    (void)u9;
}

// Raw buffer load of 16 bytes at byte offset voff from a 16-byte aligned,
// wave-uniform base.  The descriptor (base, nbytes) lives in SGPRs, so each
// row of [N, S] costs one shared 32-bit lane offset instead of a 64-bit
// address per row, which keeps VGPR use and occupancy where the row batch
// needs them.  Reads at or past nbytes return zero instead of touching memory.
// Descriptor word 3 is the gfx9-family raw-buffer format; aux bit 1 = nt.
template <int NT>
__device__ __forceinline__ u32x4 bload16(const char *al, uint32_t voff, uint32_t nbytes) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(al), 0, nbytes, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, NT ? 2 : 0);
}

// The same for 8 bytes from an 8-byte aligned, wave-uniform base.
template <int NT>
__device__ __forceinline__ u32x2 bload8(const char *al, uint32_t voff, uint32_t nbytes) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(al), 0, nbytes, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, NT ? 2 : 0);
}

// The same register of the next lane of the wave (wave_shl:1 DPP); the last
// lane gets 0.
__device__ __forceinline__ uint32_t next_lane(uint32_t x) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x130, 0xF, 0xF, false);
}

__device__ __forceinline__ u32x4 next_lane16(u32x4 a) {
    return u32x4{next_lane(a.x), next_lane(a.y), next_lane(a.z), next_lane(a.w)};
}

// Eight fp32 starting at p, whose dword index modulo 4 is q (wave-uniform).
// kAl: q == 0, two aligned loads; else three aligned loads and a select.
template <int NT, bool kAl>
__device__ __forceinline__ void load8f(const float *p, uint32_t q, f32x4 &o0, f32x4 &o1) {
    if (kAl) {
        const f32x4 *v = reinterpret_cast<const f32x4 *>(p);
        o0 = ldp<NT>(v);
        o1 = ldp<NT>(v + 1);
        return;
    }
    const f32x4 *al = reinterpret_cast<const f32x4 *>(p - q);
    select8f(ldp<NT>(al), ldp<NT>(al + 1), ldp<NT>(al + 2), q, o0, o1);
}

// Store 8 bf16 (one u32x4) at p, whose address modulo 16 is ka (even,
// uniform): one 16-byte store when aligned, else dword and short stores.
template <int NT>
__device__ __forceinline__ void store16_at(uint16_t *p, uint32_t ka, u32x4 w) {
    if (ka == 0) {
        stp<NT>(reinterpret_cast<u32x4 *>(p), w);
    } else if ((ka & 3u) == 0) {
        uint32_t *d = reinterpret_cast<uint32_t *>(p);
        d[0] = w.x;
        d[1] = w.y;
        d[2] = w.z;
        d[3] = w.w;
    } else {
        p[0] = static_cast<uint16_t>(w.x);
        uint32_t *d = reinterpret_cast<uint32_t *>(p + 1);
        d[0] = alignbyte2(w.y, w.x);
        d[1] = alignbyte2(w.z, w.y);
        d[2] = alignbyte2(w.w, w.z);
        p[7] = static_cast<uint16_t>(w.w >> 16);
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

__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
    return u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float widen(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Tile t and first element b of virtual tile vt: `split` blocks per tile,
// `sub` elements each (a multiple of 8, so every sub-range keeps the tile's
// phase modulo 16 bytes).
__device__ __forceinline__ void sub_range(int64_t vt, int32_t split, int64_t sub, int64_t *t,
                                          int64_t *b) {
    *t = vt / split;
    *b = (vt - *t * split) * sub;
}

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
        const char *al = reinterpret_cast<const char *>(s) - k;
        const uint32_t nb = (k + 2 * static_cast<uint32_t>(len - head) + 15u) & ~15u;
        const uint32_t lane = tid & 63;
        const bool last = lane == 63;
        for (int64_t w0 = tid - lane; w0 < nvec; w0 += 2 * TB) {
            const int64_t v0 = w0 + lane, v1 = v0 + TB;
            const uint32_t o0 = static_cast<uint32_t>(v0) << 4, o1 = static_cast<uint32_t>(v1) << 4;
            const u32x4 a0 = bload16<LN>(al, o0, nb), a1 = bload16<LN>(al, o1, nb);
            const u32x4 h0 = bload16<LN>(al, last ? o0 + 16 : nb, nb);
            const u32x4 h1 = bload16<LN>(al, last ? o1 + 16 : nb, nb);
            u32x4 b0 = next_lane16(a0), b1 = next_lane16(a1);
            if (last) {
                b0 = h0;
                b1 = h1;
            }
            if (v0 < nvec) stp<SN>(dv + v0, funnel(a0, b0, k));
            if (v1 < nvec) stp<SN>(dv + v1, funnel(a1, b1, k));
        }
    }
    const int64_t done = head + (nvec << 3);
    if (tid < len - done) dst[done + tid] = src[done + tid];
}

template <int POL, int TB>
__global__ __launch_bounds__(TB) void unpack_kernel(
    const UnpackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ ag_out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const CopyTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        copy_run_bf16<POL, TB>(tl.dst + b, tl.src + b, len);
    }
}

// ---------------------------------------------------------------------------
// copy-in: fp32 master shards -> bf16 segment (zeros in padding)
// ---------------------------------------------------------------------------

// dst[e] = 0 for e in [from, len), 16-byte stores where aligned.
template <int SN>
__device__ __forceinline__ void zero_bf16(uint16_t *dst, int64_t from, int64_t len) {
    const int tid = threadIdx.x;
    if (from >= len) return;
    uint16_t *d = dst + from;
    const int64_t n = len - from;
    int64_t head = ((16u - (lo32(d) & 15u)) & 15u) >> 1;
    if (head > n) head = n;
    if (tid < head) d[tid] = 0;
    const int64_t nvec = (n - head) >> 3;
    u32x4 *dv = reinterpret_cast<u32x4 *>(d + head);
    const int nthr = blockDim.x;
    for (int64_t v = tid; v < nvec; v += nthr) stp<SN>(dv + v, u32x4{0u, 0u, 0u, 0u});
    const int64_t done = head + (nvec << 3);
    if (tid < n - done) d[done + tid] = 0;
}

// Copy-in vectors: dv[v] = bf16 of s[8v .. 8v + 8) for v < nvec.
template <int LN, int SN, bool kAl>
__device__ __forceinline__ void pack_vec(u32x4 *__restrict__ dv, const float *__restrict__ s,
                                         int64_t nvec, uint32_t q) {
    int64_t v = threadIdx.x;
    for (; v + kBlock < nvec; v += 2 * kBlock) {
        f32x4 a0, a1, b0, b1;
        load8f<LN, kAl>(s + (v << 3), q, a0, a1);
        load8f<LN, kAl>(s + ((v + kBlock) << 3), q, b0, b1);
        stp<SN>(dv + v, u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w), pack2(a1.x, a1.y),
                              pack2(a1.z, a1.w)});
        stp<SN>(dv + v + kBlock, u32x4{pack2(b0.x, b0.y), pack2(b0.z, b0.w), pack2(b1.x, b1.y),
                                       pack2(b1.z, b1.w)});
    }
    if (v < nvec) {
        f32x4 a0, a1;
        load8f<LN, kAl>(s + (v << 3), q, a0, a1);
        stp<SN>(dv + v, u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w), pack2(a1.x, a1.y),
                              pack2(a1.z, a1.w)});
    }
}

template <int POL>
__device__ __forceinline__ void pack_run(uint16_t *__restrict__ dst, const float *__restrict__ src,
                                         int64_t len, int64_t valid) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = ((16u - (lo32(dst) & 15u)) & 15u) >> 1;
    if (head > valid) head = valid;
    if (tid < head) dst[tid] = static_cast<uint16_t>(bf16_rne(src[tid]));
    const int64_t nvec = (valid - head) >> 3;
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    const float *s = src + head;
    const uint32_t q = (lo32(s) >> 2) & 3u;
    if (q == 0) pack_vec<LN, SN, true>(dv, s, nvec, 0u);
    else pack_vec<LN, SN, false>(dv, s, nvec, q);
    const int64_t done = head + (nvec << 3);
    if (tid < valid - done) dst[done + tid] = static_cast<uint16_t>(bf16_rne(src[done + tid]));
    zero_bf16<SN>(dst, valid, len);
}

template <int POL>
__global__ __launch_bounds__(kBlock) void pack_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, uint16_t *__restrict__ ag_in) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        pack_run<POL>(ag_in + tl.dst + b, ents[tl.entry].master + tl.src + b, len, valid);
    }
}

// ---------------------------------------------------------------------------
// reduce: [N, S] bf16 contributions -> fp32 mean, this rank's pieces
// ---------------------------------------------------------------------------

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

// Eight consecutive column sums of the N rows of [N, S] bf16 whose row 0
// starts at base (uniform) plus this lane's byte offset offb, added in rank
// order from row 0; k0 = (base + offb) & 15, kS = (2S) & 15.  Each row's
// buffer range covers exactly the 16-byte chunks that hold its dbytes data
// bytes, so a lane past the end of the data reads zeros and never touches
// memory beyond the last chunk.  Rows are loaded RB at a time.
//
// kChunkAligned: every row starts 16-byte aligned here (k0 = 0, kS = 0), so
// each row is one aligned 16-byte load.  Otherwise a row is read as aligned
// 16-byte chunks and funnel-shifted; the caller gives the lanes of a wave
// consecutive chunks (offb = 16 * (lane + const)), so a lane's second chunk
// is the next lane's first, and lane 63's sums are not valid.
template <int NT, int RB, bool kChunkAligned>
__device__ __forceinline__ void sum_rows8(const uint16_t *base, uint32_t offb, uint32_t dbytes,
                                          int64_t S, int32_t N, uint32_t k0, uint32_t kS,
                                          float (&acc)[8]) {
    const char *r = reinterpret_cast<const char *>(base);
    const int64_t Sb = S * 2;
    for (int32_t j = 0; j < N; j += RB) {
        // rows past N get an empty range: their loads read zero and are
        // never added
        u32x4 x[RB];
        if (kChunkAligned) {
            const uint32_t nb = (dbytes + 15u) & ~15u;
#pragma unroll
            for (int i = 0; i < RB; ++i)
                x[i] = bload16<NT>(r + (j + i) * Sb, offb, j + i < N ? nb : 0u);
        } else {
            uint32_t kk[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                kk[i] = (k0 + static_cast<uint32_t>(j + i) * kS) & 15u;
                x[i] = bload16<NT>(r + (j + i) * Sb - kk[i], offb,
                                   j + i < N ? (kk[i] + dbytes + 15u) & ~15u : 0u);
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) x[i] = funnel(x[i], next_lane16(x[i]), kk[i]);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (j + i < N) {
                if (j + i == 0) init8(acc, x[i]);
                else acc8(acc, x[i]);
            }
        }
    }
}

// Aligned rows, C groups per lane: row by row from row 0, the C chunks of a
// row in flight together, so a wave reads C KB of one row before it moves to
// the next (at 64 ranks this keeps each wave on one DRAM region at a time:
// measured 5.99 vs 5.31 TB/s for one chunk of four rows in flight).  Pass c
// of this lane sits at byte offset offb + c * 1024; same buffer ranges as
// sum_rows8.  kRoll (the fused step) reloads each chunk's register with the
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
// sum_rows8.
template <int NT, int RB, int QP>
__device__ __forceinline__ void sum_rows_quad(const uint16_t *base, uint32_t offb, uint32_t dbytes,
                                              int64_t S, int32_t N, float (&acc)[QP][4]) {
    const char *r = reinterpret_cast<const char *>(base);
    const int64_t Sb = S * 2;
    const uint32_t nb = (dbytes + 7u) & ~7u;
    for (int32_t j = 0; j < N; j += RB) {
        u32x2 x[RB][QP];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const char *row = r + (j + i) * Sb;
            const uint32_t n = j + i < N ? nb : 0u;
#pragma unroll
            for (int h = 0; h < QP; ++h) x[i][h] = bload8<NT>(row, offb + 512u * h, n);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (j + i >= N) continue;
#pragma unroll
            for (int h = 0; h < QP; ++h) {
                const float y[4] = {bf16_lo(x[i][h].x), bf16_hi(x[i][h].x), bf16_lo(x[i][h].y),
                                    bf16_hi(x[i][h].y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[h][e] = j + i == 0 ? y[e] : acc[h][e] + y[e];
            }
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
                e[i][h] = bload8<NT>(al, last ? o + 8u : n, n);
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const bool s4 = kk[i] >= 4u;
            const uint32_t sh = kk[i] & 3u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x2 b{next_lane(a[i][h].x), next_lane(a[i][h].y)};
                if (last) b = e[i][h];
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

// Group schedule of the row kernels: 8-element groups [0, ngrp), C per lane
// per pass, a wave's lanes on consecutive groups.  Aligned rows: pass c of
// lane l of wave w takes group (w*C + c)*64 + l, then all step by the block.
// Misaligned rows (C = 1 only): a wave covers 63 groups and its lane 63 only
// loads the chunk after lane 62's (see sum_rows8); every lane runs the same
// number of iterations, and `own` says whether its group is to be written.
template <bool kChunkAligned, int C = 1>
struct GroupWalk {
    static_assert(kChunkAligned || C == 1, "several groups per lane need aligned rows");
    static constexpr int64_t kPer = kChunkAligned ? 64 : 63;
    int64_t g, step;
    __device__ GroupWalk() {
        const int64_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        g = wave * kPer * C + lane;
        step = static_cast<int64_t>(blockDim.x >> 6) * kPer * C;
    }
    // the wave still has work
    __device__ bool more(int64_t ngrp) const {
        return g - static_cast<int64_t>(threadIdx.x & 63) < ngrp;
    }
    // group of pass c
    __device__ int64_t at(int c) const { return g + c * kPer; }
    __device__ bool own(int64_t ngrp, int c = 0) const {
        return at(c) < ngrp && (kChunkAligned || (threadIdx.x & 63) != 63);
    }
    __device__ void next() { g += step; }
};

template <int POL, int C, bool kChunkAligned>
__device__ __forceinline__ void reduce_run(float *__restrict__ dst, const uint16_t *__restrict__ src0,
                                           int64_t len, int64_t S, int32_t N, float fN) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
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
    if constexpr (kChunkAligned && C == 1) {
        // a quad per lane and pass, two passes 64 quads apart: every wave
        // instruction contiguous, so the stores take FSDP_REDUCE_QUAD_POL
        constexpr int QS = (FSDP_REDUCE_QUAD_POL >> 1) & 1;
        const int64_t nq = (len - head) >> 2;
        const int64_t lane = tid & 63;
        const int64_t qstep = static_cast<int64_t>(blockDim.x >> 6) * 128;
        for (int64_t qb = (tid >> 6) * 128; qb < nq; qb += qstep) {
            float acc[2][4];
            sum_rows_quad<FSDP_REDUCE_QUAD_POL & 1, FSDP_REDUCE_ROW_BATCH, 2>(
                s0, static_cast<uint32_t>(qb + lane) << 3, dbytes, S, N, acc);
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
    }
    const int64_t ngrp = (len - head) >> 3;
    for (GroupWalk<kChunkAligned, C> w; w.more(ngrp); w.next()) {
        float acc[C][8];
        if constexpr (C == 1)
            sum_rows8<LN, FSDP_REDUCE_ROW_BATCH, kChunkAligned>(
                s0, static_cast<uint32_t>(w.g) << 4, dbytes, S, N, k0, kS, acc[0]);
        else
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

template <int POL, int C, bool kChunkAligned>
__global__ __launch_bounds__(kBlock) void reduce_kernel(
    const ReduceTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint16_t *__restrict__ rs_in,
    int64_t S, int32_t N, float fN) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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
__global__ __launch_bounds__(kBlock) FSDP_ADAMW_ATTR void adamw_kernel(
    const EwTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, AdamwScalars c) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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
// reduce-scatter copy-in: full bf16 gradients -> [N, S] (bf16 or fp32)
// ---------------------------------------------------------------------------

template <int POL, int TB>
__global__ __launch_bounds__(TB) void rspack_bf16_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, uint16_t *__restrict__ out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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
        for (int64_t q = tid; q < nq; q += kBlock) {
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
        for (int64_t w0 = tid - lane; w0 < nq; w0 += kBlock) {
            const int64_t q = w0 + lane;
            const uint32_t o = static_cast<uint32_t>(q) << 3;
            const u32x2 a = bload8<LN>(al, o, nb);
            const u32x2 h = bload8<LN>(al, last ? o + 8 : nb, nb);
            u32x2 b{next_lane(a.x), next_lane(a.y)};
            if (last) b = h;
            // bytes [k8, k8 + 8) of a:b
            const uint32_t u0 = s4 ? a.y : a.x, u1 = s4 ? b.x : a.y, u2 = s4 ? b.y : b.x;
            const uint32_t r0 = __builtin_amdgcn_alignbyte(u1, u0, sh);
            const uint32_t r1 = __builtin_amdgcn_alignbyte(u2, u1, sh);
            if (q < nq) stp<SN>(dv + q, f32x4{bf16_lo(r0), bf16_hi(r0), bf16_lo(r1), bf16_hi(r1)});
        }
        done = head + (nq << 2);
    }
    if (tid < valid - done) dst[done + tid] = widen(src[done + tid]);
    zero_f32<SN>(dst, valid, len);
}

template <int POL>
__global__ __launch_bounds__(kBlock) void rspack_f32_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, float *__restrict__ out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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

// ---------------------------------------------------------------------------
// FP8 E4M3 all-gather: scaled saturating copy-in, byte copy-out, amax
// ---------------------------------------------------------------------------

// fp32 -> OCP e4m3fn code, round to nearest even, magnitudes >= 448 (and
// infinities) saturate to +-448, NaN -> NaN code with its sign.  Normal
// codes keep 3 of the 23 mantissa bits of the fp32 pattern (ties to even,
// exponent rebiased from 127 to 7); below 2^-6 the code is the subnormal
// m/8 * 2^-6 with m the significand shifted to 2^-9 units, ties to even.
__device__ __forceinline__ uint32_t e4m3_sat(float f) {
    // Every case is computed and the right one selected, so a wave never
    // diverges on the value class.
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7FFFFFFFu;
    // normal: round the fp32 pattern to 3 mantissa bits, rebias 127 -> 7
    uint32_t cn = ((mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20) - (120u << 3);
    cn = cn > 0x7Eu ? 0x7Eu : cn;
    // subnormal (exponent field 120 or less): shifts of 32 or more leave 0,
    // and so does 31 for a 24-bit significand, so the shift is capped there
    const uint32_t E = mag >> 23;
    const uint32_t shift = E - 110u <= 10u ? 141u - E : 31u;
    const uint32_t M = (mag & 0x7FFFFFu) | 0x800000u;
    const uint32_t cs = (M + (1u << (shift - 1u)) - 1u + ((M >> shift) & 1u)) >> shift;
    uint32_t r = mag >= 0x3C800000u ? cn : cs;
    r = mag >= 0x43E00000u ? 0x7Eu : r;
    r = mag > 0x7F800000u ? 0x7Fu : r;
    return sign | r;
}

// Four e4m3_sat(x * s) codes packed little-endian, on the gfx950 converter
// (v_cvt_pk_fp8_f32: e4m3fn, round to nearest even, two values per
// instruction).  Inputs are first clamped to +-448 by compares, which keeps
// NaN; the converter writes 0xFF for every NaN, so a positive NaN gets its
// top bit cleared.  Checked equal to e4m3_sat over all 2^32 fp32 inputs.
__device__ __forceinline__ float clamp448(float v) {
    return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);
}

__device__ __forceinline__ uint32_t pos_nan_bit(float x, uint32_t bit) {
    return __float_as_uint(x) - 0x7F800001u < 0x007FFFFFu ? bit : 0u;
}

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d, float s) {
    const float x0 = a * s, x1 = b * s, x2 = c * s, x3 = d * s;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(x0), clamp448(x1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(x2), clamp448(x3), w, true);
    const uint32_t clr = pos_nan_bit(x0, 0x80u) | pos_nan_bit(x1, 0x8000u) |
                         pos_nan_bit(x2, 0x800000u) | pos_nan_bit(x3, 0x80000000u);
    return static_cast<uint32_t>(w) & ~clr;
}

// dst[e] = 0 for e in [from, len) bytes, 16-byte stores where aligned.
__device__ __forceinline__ void zero_u8(uint8_t *dst, int64_t from, int64_t len) {
    const int tid = threadIdx.x;
    if (from >= len) return;
    uint8_t *d = dst + from;
    const int64_t n = len - from;
    int64_t head = (16u - (lo32(d) & 15u)) & 15u;
    if (head > n) head = n;
    if (tid < head) d[tid] = 0;
    const int64_t nvec = (n - head) >> 4;
    u32x4 *dv = reinterpret_cast<u32x4 *>(d + head);
    for (int64_t v = tid; v < nvec; v += kBlock) stp<1>(dv + v, u32x4{0u, 0u, 0u, 0u});
    const int64_t done = head + (nvec << 4);
    if (tid < n - done) d[done + tid] = 0;
}

// dv[g] = e4m3 of scale * s[16g .. 16g + 16) for g < ngrp; two groups per
// lane per iteration when the source is aligned (the misaligned variant's
// extra loads and selects would cost the whole kernel occupancy).
template <int LN, int SN, bool kAl>
__device__ __forceinline__ void pack_fp8_vec(u32x4 *__restrict__ dv, const float *__restrict__ s,
                                             int64_t ngrp, uint32_t q, float scale) {
    int64_t g = threadIdx.x;
    for (; kAl && g + kBlock < ngrp; g += 2 * kBlock) {
        f32x4 a0, a1, a2, a3, b0, b1, b2, b3;
        load8f<LN, kAl>(s + (g << 4), q, a0, a1);
        load8f<LN, kAl>(s + (g << 4) + 8, q, a2, a3);
        load8f<LN, kAl>(s + ((g + kBlock) << 4), q, b0, b1);
        load8f<LN, kAl>(s + ((g + kBlock) << 4) + 8, q, b2, b3);
        stp<SN>(dv + g, u32x4{pack4_e4m3(a0.x, a0.y, a0.z, a0.w, scale),
                              pack4_e4m3(a1.x, a1.y, a1.z, a1.w, scale),
                              pack4_e4m3(a2.x, a2.y, a2.z, a2.w, scale),
                              pack4_e4m3(a3.x, a3.y, a3.z, a3.w, scale)});
        stp<SN>(dv + g + kBlock, u32x4{pack4_e4m3(b0.x, b0.y, b0.z, b0.w, scale),
                                       pack4_e4m3(b1.x, b1.y, b1.z, b1.w, scale),
                                       pack4_e4m3(b2.x, b2.y, b2.z, b2.w, scale),
                                       pack4_e4m3(b3.x, b3.y, b3.z, b3.w, scale)});
    }
    for (; g < ngrp; g += kBlock) {
        f32x4 a0, a1, a2, a3;
        load8f<LN, kAl>(s + (g << 4), q, a0, a1);
        load8f<LN, kAl>(s + (g << 4) + 8, q, a2, a3);
        stp<SN>(dv + g, u32x4{pack4_e4m3(a0.x, a0.y, a0.z, a0.w, scale),
                              pack4_e4m3(a1.x, a1.y, a1.z, a1.w, scale),
                              pack4_e4m3(a2.x, a2.y, a2.z, a2.w, scale),
                              pack4_e4m3(a3.x, a3.y, a3.z, a3.w, scale)});
    }
}

template <int POL>
__device__ __forceinline__ void pack_fp8_run(uint8_t *__restrict__ dst, const float *__restrict__ src,
                                             int64_t len, int64_t valid, float scale) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    int64_t head = (16u - (lo32(dst) & 15u)) & 15u;
    if (head > valid) head = valid;
    if (tid < head) dst[tid] = static_cast<uint8_t>(e4m3_sat(src[tid] * scale));
    const int64_t ngrp = (valid - head) >> 4;
    const float *s = src + head;
    const uint32_t q = (lo32(s) >> 2) & 3u;
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    if (q == 0) pack_fp8_vec<LN, SN, true>(dv, s, ngrp, 0u, scale);
    else pack_fp8_vec<LN, SN, false>(dv, s, ngrp, q, scale);
    const int64_t done = head + (ngrp << 4);
    if (tid < valid - done)
        dst[done + tid] = static_cast<uint8_t>(e4m3_sat(src[done + tid] * scale));
    zero_u8(dst, valid, len);
}

template <int POL>
__global__ __launch_bounds__(kBlock) void pack_fp8_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, uint8_t *__restrict__ ag_in,
    const float *__restrict__ scales) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const PackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        int64_t valid = tl.valid - b;
        valid = valid < 0 ? 0 : (valid > len ? len : valid);
        pack_fp8_run<POL>(ag_in + tl.dst + b, ents[tl.entry].master + tl.src + b, len, valid,
                          scales[tl.entry]);
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
        const uint32_t lane = tid & 63;
        const bool last = lane == 63;
        for (int64_t w0 = tid - lane; w0 < nvec; w0 += TB) {
            const int64_t v = w0 + lane;
            const uint32_t o = static_cast<uint32_t>(v) << 4;
            const u32x4 a = bload16<LN>(al, o, nb);
            const u32x4 h = bload16<LN>(al, last ? o + 16 : nb, nb);
            u32x4 b = next_lane16(a);
            if (last) b = h;
            if (v < nvec) stp<SN>(dv + v, funnel(a, b, k));
        }
    }
    const int64_t done = head + (nvec << 4);
    if (tid < len - done) dst[done + tid] = src[done + tid];
}

template <int POL, int TB>
__global__ __launch_bounds__(TB) void unpack_fp8_kernel(
    const UnpackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const uint8_t *__restrict__ ag_out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const UnpackTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        copy_run_u8<POL, TB>(ents[tl.entry].full_fp8 + tl.dst + b, ag_out + tl.src + b, len);
    }
}

__global__ __launch_bounds__(kBlock) void zero_floats_kernel(float *p, int32_t n) {
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Largest |x| per parameter as the maximum of the bit patterns of |x|
// (monotone for non-negative floats; a NaN wins), merged across blocks with
// an unsigned atomic max on the result's bits.
__global__ __launch_bounds__(kBlock) void amax_kernel(const EwTile *__restrict__ tiles,
                                                      int64_t n_tiles, int32_t split, int64_t sub,
                                                      const DevEntry *__restrict__ ents,
                                                      uint32_t *__restrict__ amax_bits) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    const int tid = threadIdx.x;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const EwTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        const float *P = ents[tl.entry].master + tl.off + b;
        uint32_t m = 0;
        for (int64_t i = tid; i < len; i += kBlock) {
            const uint32_t x = __float_as_uint(P[i]) & 0x7FFFFFFFu;
            m = x > m ? x : m;
        }
        for (int off = 32; off > 0; off >>= 1) {
            const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 64));
            m = o > m ? o : m;
        }
        if ((tid & 63) == 0 && m != 0) atomicMax(amax_bits + tl.entry, m);
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
    for (int64_t v = tid; v < nvec; v += kBlock) {
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
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const EwTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        const DevEntry en = ents[tl.entry];
        accumulate_run<POL, kReset>(en.grad_acc + tl.off + b, en.full_grad + tl.off + b, len);
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
        const uint32_t lane = tid & 63;
        const bool last = lane == 63;
        for (int64_t w0 = tid - lane; w0 < nv; w0 += kBlock) {
            const int64_t v = w0 + lane;
            const uint32_t o = static_cast<uint32_t>(v) << 4;
            const u32x4 a = bload16<LN>(al, o, nb);
            const u32x4 h = bload16<LN>(al, last ? o + 16 : nb, nb);
            u32x4 b = next_lane16(a);
            if (last) b = h;
            if (v < nv) stp<SN>(dv + v, __builtin_bit_cast(f32x4, funnel(a, b, 4 * q)));
        }
        done = head + (nv << 2);
    }
    if (tid < valid - done) dst[done + tid] = src[done + tid];
    zero_f32<SN>(dst, valid, len);
}

template <int POL>
__global__ __launch_bounds__(kBlock) void rspack_acc_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, float *__restrict__ out) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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

// ---------------------------------------------------------------------------
// reduce of fp32 contributions: [N, S] fp32 -> fp32 mean, this rank's pieces
// ---------------------------------------------------------------------------

__device__ __forceinline__ float sum_rows_scalar_f32(const float *src0, int64_t S, int32_t N,
                                                     int64_t e) {
    float acc = src0[e];
    for (int32_t j = 1; j < N; ++j) acc = acc + src0[static_cast<int64_t>(j) * S + e];
    return acc;
}

// Eight consecutive column sums of the N rows of [N, S] fp32 whose row 0
// starts at base (uniform) plus this lane's byte offset offb (32 bytes per
// group), added in rank order from row 0; q0 = dword index of base + offb
// modulo 4, qS = S modulo 4.  Buffer ranges cover exactly the 16-byte chunks
// holding each row's dbytes data bytes.  Same scheme as sum_rows8: with
// kChunkAligned (q0 = qS = 0) each row is two aligned loads; otherwise a
// lane's third chunk is the next lane's first (waves of 63 groups).
template <int NT, int RB, bool kChunkAligned>
__device__ __forceinline__ void sum_rows8f(const float *base, uint32_t offb, uint32_t dbytes,
                                           int64_t S, int32_t N, uint32_t q0, uint32_t qS,
                                           float (&acc)[8]) {
    const char *r = reinterpret_cast<const char *>(base);
    const int64_t Sb = S * 4;
    for (int32_t j = 0; j < N; j += RB) {
        f32x4 lo[RB], hi[RB];
        if (kChunkAligned) {
            const uint32_t nb = (dbytes + 15u) & ~15u;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const char *row = r + (j + i) * Sb;
                const uint32_t n = j + i < N ? nb : 0u;
                lo[i] = __builtin_bit_cast(f32x4, bload16<NT>(row, offb, n));
                hi[i] = __builtin_bit_cast(f32x4, bload16<NT>(row, offb + 16, n));
            }
        } else {
            uint32_t qq[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                qq[i] = (q0 + static_cast<uint32_t>(j + i) * qS) & 3u;
                const char *al = r + (j + i) * Sb - 4 * qq[i];
                const uint32_t n = j + i < N ? (4 * qq[i] + dbytes + 15u) & ~15u : 0u;
                lo[i] = __builtin_bit_cast(f32x4, bload16<NT>(al, offb, n));
                hi[i] = __builtin_bit_cast(f32x4, bload16<NT>(al, offb + 16, n));
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const f32x4 c = __builtin_bit_cast(
                    f32x4, next_lane16(__builtin_bit_cast(u32x4, lo[i])));
                select8f(lo[i], hi[i], c, qq[i], lo[i], hi[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (j + i < N) {
                const float x[8] = {lo[i].x, lo[i].y, lo[i].z, lo[i].w,
                                    hi[i].x, hi[i].y, hi[i].z, hi[i].w};
                if (j + i == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = x[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
                }
            }
        }
    }
}

template <int POL, bool kChunkAligned>
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
    if constexpr (kChunkAligned) {
        // four elements (one vector) per lane and pass, two passes 64
        // vectors apart: every wave instruction contiguous, so loads and
        // stores take FSDP_REDUCE_F32_QUAD_POL
        constexpr int QL = FSDP_REDUCE_F32_QUAD_POL & 1, QS = (FSDP_REDUCE_F32_QUAD_POL >> 1) & 1;
        const char *r = reinterpret_cast<const char *>(s0);
        const int64_t Sb = S * 4;
        const uint32_t nb = (dbytes + 15u) & ~15u;
        const int64_t nq = (len - head) >> 2;
        const int64_t lane = tid & 63;
        const int64_t qstep = static_cast<int64_t>(blockDim.x >> 6) * 128;
        for (int64_t qb = (tid >> 6) * 128; qb < nq; qb += qstep) {
            const uint32_t off = static_cast<uint32_t>(qb + lane) << 4;
            f32x4 acc[2];
            for (int32_t j = 0; j < N; j += FSDP_REDUCE_ROW_BATCH) {
                f32x4 x[FSDP_REDUCE_ROW_BATCH][2];
#pragma unroll
                for (int i = 0; i < FSDP_REDUCE_ROW_BATCH; ++i) {
                    const char *row = r + (j + i) * Sb;
                    const uint32_t n = j + i < N ? nb : 0u;
                    x[i][0] = __builtin_bit_cast(f32x4, bload16<QL>(row, off, n));
                    x[i][1] = __builtin_bit_cast(f32x4, bload16<QL>(row, off + 1024u, n));
                }
#pragma unroll
                for (int i = 0; i < FSDP_REDUCE_ROW_BATCH; ++i) {
                    if (j + i >= N) continue;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f32x4 y = x[i][h];
                        acc[h] = j + i == 0 ? y
                                            : f32x4{acc[h].x + y.x, acc[h].y + y.y,
                                                    acc[h].z + y.z, acc[h].w + y.w};
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t q = qb + lane + 64 * h;
                if (q < nq)
                    stp<QS>(dv + q, f32x4{acc[h].x / fN, acc[h].y / fN, acc[h].z / fN,
                                          acc[h].w / fN});
            }
        }
        const int64_t done = head + (nq << 2);
        if (tid < len - done) dst[done + tid] = sum_rows_scalar_f32(src0, S, N, done + tid) / fN;
        return;
    }
    const int64_t ngrp = (len - head) >> 3;
    for (GroupWalk<kChunkAligned> w; w.more(ngrp); w.next()) {
        float acc[8];
        sum_rows8f<LN, FSDP_REDUCE_ROW_BATCH, kChunkAligned>(
            s0, static_cast<uint32_t>(w.g) << 5, dbytes, S, N, q0, qS, acc);
        if (w.own(ngrp)) {
            const int64_t g = w.g;
            stp<SN>(dv + 2 * g, f32x4{acc[0] / fN, acc[1] / fN, acc[2] / fN, acc[3] / fN});
            stp<SN>(dv + 2 * g + 1, f32x4{acc[4] / fN, acc[5] / fN, acc[6] / fN, acc[7] / fN});
        }
    }
    const int64_t done = head + (ngrp << 3);
    if (tid < len - done) dst[done + tid] = sum_rows_scalar_f32(src0, S, N, done + tid) / fN;
}

template <int POL, bool kChunkAligned>
__global__ __launch_bounds__(kBlock) void reduce_f32_kernel(
    const ReduceTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents, const float *__restrict__ rs_in, int64_t S, int32_t N,
    float fN) {
    const int64_t L = sub;
    const int64_t nvt = n_tiles * split;
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
        int64_t t, b;
        sub_range(vt, split, L, &t, &b);
        const ReduceTile tl = tiles[t];
        if (b >= tl.len) continue;
        const int64_t len = tl.len - b < L ? tl.len - b : L;
        reduce_f32_run<POL, kChunkAligned>(ents[tl.entry].grad + tl.dst + b, rs_in + tl.src + b,
                                          len, S, N, fN);
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

// Valid elements [0, valid) then zeros up to len.  rs0 is row 0 of the
// gradient contributions at this run's first segment position; dst is ag_in
// at the same position; P, M, Vv, G are the shards at this run's first
// element.  The vector path aligns on the fp32 shards (the bulk of the
// bytes); contributions are funnel-shifted per row and the bf16 output is
// stored whole, by dwords or by halves, as its address allows.  C groups per
// lane per pass (C > 1: aligned rows, read row by row).
template <int POL, int RB, int C, bool kChunkAligned, bool kWriteGrad>
__device__ __forceinline__ void step_run(const uint16_t *__restrict__ rs0, int64_t S, int32_t N,
                                         float fN, float *P, float *M, float *Vv, float *G,
                                         uint16_t *dst, int64_t len, int64_t valid,
                                         const AdamwScalars &c) {
    constexpr int LN = POL & 1, SN = (POL >> 1) & 1;
    const int tid = threadIdx.x;
    const uint32_t ap = lo32(P) & 15u;
    int64_t head = ((16u - ap) & 15u) >> 2;
    if (head > valid) head = valid;
    const uint32_t kS = static_cast<uint32_t>((S * 2) & 15);
    const uint32_t k0 = lo32(rs0 + head) & 15u;
    // the vector path needs the shards equally aligned, and with
    // kChunkAligned the rows 16-byte aligned at the first vector element
    const bool same = ap == (lo32(M) & 15u) && ap == (lo32(Vv) & 15u) &&
                      (!kWriteGrad || ap == (lo32(G) & 15u)) &&
                      (!kChunkAligned || (k0 | kS) == 0);
    if (!same) {
        for (int64_t e = tid; e < valid; e += static_cast<int64_t>(blockDim.x))
            step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, e, c);
    } else {
        if (tid < head) step_scalar_at<kWriteGrad>(rs0, S, N, fN, P, M, Vv, G, dst, tid, c);
        const int64_t ngrp = (valid - head) >> 3;
        const uint32_t ka = lo32(dst + head) & 15u;
        const uint32_t dbytes = static_cast<uint32_t>(2 * (valid - head));
        for (GroupWalk<kChunkAligned, C> w; w.more(ngrp); w.next()) {
            float acc[C][8];
            if constexpr (C == 1)
                sum_rows8<FSDP_STEP_ROW_NT, RB, kChunkAligned>(
                    rs0 + head, static_cast<uint32_t>(w.g) << 4, dbytes, S, N, k0, kS, acc[0]);
            else
                sum_rows_wide<FSDP_STEP_ROW_NT, C, true>(
                    rs0 + head, static_cast<uint32_t>(w.g) << 4, dbytes, S, N, acc);
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

// The fused step, a quad per lane and pass: lane l of a wave takes quads
// l + 64 h (h < QP) of the wave's 64 QP, so every load and store instruction
// of the wave is contiguous (rows 512 bytes, shards 1 KB, the bf16 output 512
// bytes).  That lets the shards use non-temporal loads and stores without
// partial writes (a lane storing two halves of 32 bytes splits them).  Rows
// 16-byte aligned, or with kMis at any even byte phase (sum_rows_quad_mis,
// QP = 2).  Same arithmetic, in the same order, as step_run.
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
        for (int64_t qb = (tid >> 6) * 64 * QP; qb < nq; qb += qstep) {
            float acc[QP][4];
            if constexpr (kMis)
                sum_rows_quad_mis<FSDP_STEP_ROW_NT, RB>(rs0 + head,
                                                        static_cast<uint32_t>(qb + lane) << 3,
                                                        dbytes, S, N, k0 & 7u, kS & 7u, acc);
            else
                sum_rows_quad<FSDP_STEP_ROW_NT, RB, QP>(
                    rs0 + head, static_cast<uint32_t>(qb + lane) << 3, dbytes, S, N, acc);
#pragma unroll
            for (int h = 0; h < QP; ++h) {
                const int64_t q = qb + lane + 64 * h;
                if (q >= nq) continue;
                const int64_t e0 = head + (q << 2);
                f32x4 *pv = reinterpret_cast<f32x4 *>(P + e0);
                f32x4 *mv = reinterpret_cast<f32x4 *>(M + e0);
                f32x4 *vv = reinterpret_cast<f32x4 *>(Vv + e0);
                f32x4 pq = ldp<LN>(pv), mq = ldp<LN>(mv), vq = ldp<LN>(vv);
                const f32x4 g{acc[h][0] / fN, acc[h][1] / fN, acc[h][2] / fN, acc[h][3] / fN};
                if (kWriteGrad) stp<SN>(reinterpret_cast<f32x4 *>(G + e0), g);
                adamw_vec(pq, g, mq, vq, c);
                stp<SN>(pv, pq);
                stp<SN>(mv, mq);
                stp<SN>(vv, vq);
                store8_at<FSDP_STEP_OUT_NT>(dst + e0, k8, u32x2{pack2(pq.x, pq.y), pack2(pq.z, pq.w)});
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
    for (int64_t vt = blockIdx.x; vt < nvt; vt += gridDim.x) {
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
            step_run<POL, RB, C, kChunkAligned, kWriteGrad>(
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
__global__ __launch_bounds__(kBlock) FSDP_STEP_GEN_ATTR void step_kernel(
    const PackTile *__restrict__ tiles, int64_t n_tiles, int32_t split, int64_t sub,
    const DevEntry *__restrict__ ents,
    const uint16_t *__restrict__ rs_in, uint16_t *__restrict__ ag_in, int64_t S, int32_t N,
    float fN, AdamwScalars c) {
    step_tiles<FSDP_STEP_QUAD_POL, RB, 1, false, kWriteGrad, 2>(tiles, n_tiles, split, sub, ents,
                                                                 rs_in, ag_in, S, N, fN, c);
}

inline unsigned grid_for(int64_t n_tiles, int32_t split) {
    constexpr int64_t kMaxGrid = 1 << 22;
    const int64_t n = n_tiles * split;
    return static_cast<unsigned>(n < kMaxGrid ? n : kMaxGrid);
}

// Blocks per tile for a wanted sub-range: the largest power of two not above
// `want`, within [8, kTile]; tiles are powers of two, so it divides them.
inline int32_t split_for(int64_t tile, int64_t want) {
    int64_t sub = 8;
    while (sub * 2 <= want && sub * 2 <= tile) sub *= 2;
    return static_cast<int32_t>(tile / sub);
}

// Sub-range for kernels that read all N rows per element (reduce, fused step):
// about FSDP_ROWS_BUDGET row-elements per block.
inline int32_t split_rows(int64_t tile, int32_t N, int32_t extra_rows) {
    int64_t want = FSDP_ROWS_BUDGET / (N + extra_rows);
    if (want < FSDP_MIN_SUB) want = FSDP_MIN_SUB;
    return split_for(tile, want);
}

// Threads for the row kernels: one 8-element group per lane, whole waves,
// at most kBlock (so a small sub-range does not leave idle waves).
inline unsigned row_threads(int64_t sub) {
#if FSDP_ROW_BLOCK_FIT
    int64_t t = (sub / 8 + 63) / 64 * 64;
    return static_cast<unsigned>(t < 64 ? 64 : (t > kBlock ? kBlock : t));
#else
    (void)sub;
    return kBlock;
#endif
}

// Misaligned rows: a wave covers 63 groups (504 elements), so sub-ranges are
// cut in whole such waves; a power-of-two sub-range would leave one wave a
// second pass through all N rows for a handful of groups.
struct RowSplit {
    int32_t split;
    int64_t sub;
};
inline RowSplit row_split(int64_t tile, int32_t sp, bool aligned) {
    const int64_t sub = tile / sp;
    if (aligned) return RowSplit{sp, sub};
    const int64_t msub = sub / 512 * 504;
    return RowSplit{static_cast<int32_t>((tile + msub - 1) / msub), msub};
}

AdamwScalars to_scalars(const float s[8]) {
    return AdamwScalars{s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]};
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------

hipError_t launch_pack(const PackTile *tiles, int64_t n, const DevEntry *ents, uint16_t *ag_in,
                       hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTilePack, FSDP_PACK_SUB);
    pack_kernel<FSDP_PACK_POL>
        <<<grid_for(n, sp), kBlock, 0, st>>>(tiles, n, sp, kTilePack / sp, ents, ag_in);
    return hipGetLastError();
}

// Row pieces 16-byte aligned: FSDP_UNPACK_THREADS threads per block over
// FSDP_UNPACK_SUB elements; otherwise FSDP_UNPACK_MIS_THREADS over
// FSDP_UNPACK_MIS_SUB (both correct for any alignment; measured per case).
hipError_t launch_unpack(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                         const uint16_t *ag_out, bool chunk_aligned, hipStream_t st) {
    if (n == 0) return hipSuccess;
    if (chunk_aligned) {
        const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_SUB);
        unpack_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS>
            <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp,
                                                              ents, ag_out);
    } else {
        const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_MIS_SUB);
        unpack_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_MIS_THREADS>
            <<<grid_for(n, sp), FSDP_UNPACK_MIS_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp,
                                                                  ents, ag_out);
    }
    return hipGetLastError();
}

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
    const RowSplit rsp = row_split(kTileReduce, split_rows(kTileReduce, N, 0), chunk_aligned);
    const unsigned grid = grid_for(n, rsp.split);
    const unsigned thr = row_threads(rsp.sub);
    if (chunk_aligned)
        reduce_kernel<FSDP_REDUCE_POL, 1, true>
            <<<grid, thr, 0, st>>>(tiles, n, rsp.split, rsp.sub, ents, rs_in, S, N, fN);
    else
        reduce_kernel<FSDP_REDUCE_POL, 1, false>
            <<<grid, thr, 0, st>>>(tiles, n, rsp.split, rsp.sub, ents, rs_in, S, N, fN);
    return hipGetLastError();
}

hipError_t launch_adamw(const EwTile *tiles, int64_t n, const DevEntry *ents,
                        const float scal[8], hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileAdamw, FSDP_ADAMW_SUB);
    adamw_kernel<FSDP_ADAMW_POL><<<grid_for(n, sp), kBlock, 0, st>>>(
        tiles, n, sp, kTileAdamw / sp, ents, to_scalars(scal));
    return hipGetLastError();
}

hipError_t launch_copy_runs(const CopyTile *tiles, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_SUB);
    copy_runs_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS>
        <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp);
    return hipGetLastError();
}

hipError_t launch_pack_fp8(const PackTile *tiles, int64_t n, const DevEntry *ents, uint8_t *ag_in,
                           const float *scales, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTilePack, FSDP_FP8_SUB);
    pack_fp8_kernel<FSDP_FP8_POL><<<grid_for(n, sp), kBlock, 0, st>>>(
        tiles, n, sp, kTilePack / sp, ents, ag_in, scales);
    return hipGetLastError();
}

hipError_t launch_unpack_fp8(const UnpackTile *tiles, int64_t n, const DevEntry *ents,
                             const uint8_t *ag_out, hipStream_t st) {
    if (n == 0) return hipSuccess;
    // 16 bytes per lane move 16 elements: twice the elements per block of bf16
    const int32_t sp = split_for(kTileUnpack, 2 * FSDP_UNPACK_SUB);
    unpack_fp8_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS>
        <<<grid_for(n, sp), FSDP_UNPACK_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp, ents,
                                                          ag_out);
    return hipGetLastError();
}

hipError_t launch_amax(const EwTile *tiles, int64_t n, const DevEntry *ents, float *amax,
                       int32_t n_params, hipStream_t st) {
    if (n_params == 0) return hipSuccess;
    zero_floats_kernel<<<(n_params + kBlock - 1) / kBlock, kBlock, 0, st>>>(amax, n_params);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    const int32_t sp = split_for(kTileAdamw, FSDP_ADAMW_SUB);
    amax_kernel<<<grid_for(n, sp), kBlock, 0, st>>>(tiles, n, sp, kTileAdamw / sp, ents,
                                                    reinterpret_cast<uint32_t *>(amax));
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

hipError_t launch_rspack_acc(const PackTile *tiles, int64_t n, const DevEntry *ents, float *out,
                             hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileUnpack, FSDP_UNPACK_SUB);
    rspack_acc_kernel<FSDP_RSPACK_ACC_POL><<<grid_for(n, sp), kBlock, 0, st>>>(
        tiles, n, sp, kTileUnpack / sp, ents, out);
    return hipGetLastError();
}

// Block shapes as the copy-out's, chosen by whether every row piece of the
// output is 16-byte aligned.
hipError_t launch_rspack(const PackTile *tiles, int64_t n, const DevEntry *ents, void *out,
                         bool f32, bool chunk_aligned, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTileUnpack, chunk_aligned ? FSDP_UNPACK_SUB : FSDP_UNPACK_MIS_SUB);
    const unsigned grid = grid_for(n, sp);
    if (f32)
        rspack_f32_kernel<FSDP_RSPACK_F32_POL><<<grid, kBlock, 0, st>>>(
            tiles, n, sp, kTileUnpack / sp, ents, static_cast<float *>(out));
    else if (chunk_aligned)
        rspack_bf16_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_THREADS><<<grid, FSDP_UNPACK_THREADS, 0, st>>>(
            tiles, n, sp, kTileUnpack / sp, ents, static_cast<uint16_t *>(out));
    else
        rspack_bf16_kernel<FSDP_UNPACK_POL, FSDP_UNPACK_MIS_THREADS>
            <<<grid, FSDP_UNPACK_MIS_THREADS, 0, st>>>(tiles, n, sp, kTileUnpack / sp, ents,
                                                       static_cast<uint16_t *>(out));
    return hipGetLastError();
}

hipError_t launch_reduce_f32(const ReduceTile *tiles, int64_t n, const DevEntry *ents,
                             const float *rs_in, int64_t S, int32_t N, bool chunk_aligned,
                             hipStream_t st) {
    if (n == 0) return hipSuccess;
    const float fN = static_cast<float>(N);
    // fp32 rows carry twice the bytes of bf16 rows per element
    const RowSplit rsp = row_split(kTileReduce, split_rows(kTileReduce, 2 * N, 0), chunk_aligned);
    const unsigned grid = grid_for(n, rsp.split);
    const unsigned thr = row_threads(rsp.sub);
    if (chunk_aligned)
        reduce_f32_kernel<FSDP_REDUCE_F32_POL, true>
            <<<grid, thr, 0, st>>>(tiles, n, rsp.split, rsp.sub, ents, rs_in, S, N, fN);
    else
        reduce_f32_kernel<FSDP_REDUCE_F32_POL, false>
            <<<grid, thr, 0, st>>>(tiles, n, rsp.split, rsp.sub, ents, rs_in, S, N, fN);
    return hipGetLastError();
}

template <int RB, int RBG>
void launch_step_rb(bool aligned, bool write_grad, unsigned grid, unsigned thr, hipStream_t st,
                    const PackTile *tiles, int64_t n, int32_t sp, int64_t sub, const DevEntry *ents,
                    const uint16_t *rs_in, uint16_t *ag_in, int64_t S, int32_t N, float fN,
                    const AdamwScalars &c) {
    if (aligned && write_grad)
        step_kernel_aligned<RB, true><<<grid, thr, 0, st>>>(tiles, n, sp, sub, ents, rs_in, ag_in,
                                                           S, N, fN, c);
    else if (aligned)
        step_kernel_aligned<RB, false><<<grid, thr, 0, st>>>(tiles, n, sp, sub, ents, rs_in,
                                                            ag_in, S, N, fN, c);
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
    const RowSplit rsp = row_split(kTilePack, split_rows(kTilePack, N, 6), true);
    const int32_t sp = rsp.split;
    const int64_t sub = rsp.sub;
    const unsigned grid = grid_for(n, sp);
    const unsigned thr = row_threads(sub) < FSDP_STEP_THREADS ? row_threads(sub) : FSDP_STEP_THREADS;
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
