// Device code shared by the HIP kernels of one rank's FSDP2 sharded step,
// written for CDNA4 (gfx950).  The kernels live in copy.hip (copy-out,
// reduce-scatter copy-ins, FP8 copy-out, resharding), pack.hip (copy-in, FP8
// copy-in, amax), reduce.hip (reductions, accumulation) and step.hip (AdamW
// and the fused step); rows.hpp holds the column sums over the N rows.
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
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

// Knobs.  Each kernel family's tuning constants sit in its own file as
// FSDP_* macros (a build can override one with -D to measure an
// alternative); the values are the ones measured fastest on MI355X.  Cache
// policy constants: bit 0 = non-temporal loads, bit 1 = non-temporal stores.

// Elements per block of the kernels that read all N rows per element (the
// reductions and the narrow fused step): about FSDP_ROWS_BUDGET
// row-elements per block, at least FSDP_MIN_SUB elements.
#ifndef FSDP_ROWS_BUDGET
#define FSDP_ROWS_BUDGET 32768
#endif
#ifndef FSDP_MIN_SUB
#define FSDP_MIN_SUB 512
#endif
// elements per block of AdamW and the accumulation: one 16-byte vector per
// lane and array in a 256-thread block (against 4096 elements, two vectors
// a block apart twice: AdamW 5.4-5.5 -> 5.6-6.0 TB/s and the accumulation
// 5.9-6.0 -> 6.2-6.3 on the 7B and 70B shapes; 2048 in between)
#ifndef FSDP_ADAMW_SUB
#define FSDP_ADAMW_SUB 1024
#endif

namespace fsdp {

namespace {

// Cache policy of the extra load of a misaligned read: the chunk after a
// wave's span, which lane 63 loads for its funnel shift and another wave
// reads too, takes a temporal load.  Under the non-temporal hint of the rest
// of the run it was often evicted from L2 before the other wave's read and
// fetched twice (ragged MoE workload: fp32 reduce-scatter copy-in and
// copy-out +1%, misaligned fused step +0.6%).
constexpr int kBoundaryNT = 0;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// threads per block of most kernels (four waves)
constexpr int kBlock = 256;

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

// Raw buffer store of 16 bytes at byte offset voff from a 16-byte aligned,
// wave-uniform base; stores at or past nbytes are dropped, so a lane past
// the end of a run needs no branch around its store.
template <int NT>
__device__ __forceinline__ void bstore16(char *al, uint32_t voff, uint32_t nbytes, u32x4 w) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(al, 0, nbytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, 0, NT ? 2 : 0);
}

// The same register of the next lane of the wave (wave_shl:1 DPP); the last
// lane gets 0.
__device__ __forceinline__ uint32_t next_lane(uint32_t x) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x130, 0xF, 0xF, false);
}

__device__ __forceinline__ u32x4 next_lane16(u32x4 a) {
    return u32x4{next_lane(a.x), next_lane(a.y), next_lane(a.z), next_lane(a.w)};
}

// The next lane's register, lane 63 taking `own` instead (its load of the
// chunk past the wave's span): the DPP move's old value, which a lane
// without a source lane keeps.  Consumed by the move itself rather than by
// a select on the lane index, the load cannot be sunk by the compiler under
// a branch (a lane-63 select, or a guard on a later store or add), where it
// left only after the wave's other loads had returned: one more memory
// latency per iteration.
__device__ __forceinline__ uint32_t next_lane_or(uint32_t x, uint32_t own) {
    return __builtin_amdgcn_update_dpp(own, x, 0x130, 0xF, 0xF, false);
}
__device__ __forceinline__ u32x4 next_or_own(u32x4 a, u32x4 own) {
    return u32x4{next_lane_or(a.x, own.x), next_lane_or(a.y, own.y), next_lane_or(a.z, own.z),
                 next_lane_or(a.w, own.w)};
}
__device__ __forceinline__ u32x2 next_or_own(u32x2 a, u32x2 own) {
    return u32x2{next_lane_or(a.x, own.x), next_lane_or(a.y, own.y)};
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

// First virtual tile of this block.  kRemap renumbers the launch's blocks so
// that each of the GPU's 8 XCDs (which take blocks round-robin: block b runs
// on XCD b % 8) serves one contiguous eighth of the virtual tiles: a
// bijection on [0, gridDim.x), so every tile is still served exactly once.
// Used by the copies on misaligned rows, where neighbouring blocks share the
// 128-byte line at their boundary and the remap lets one XCD's L2 fetch it
// once (ragged MoE copy-out 5.74 -> 6.08 TB/s on MI355X); on aligned rows
// the round-robin order measured faster (7B step 11.65 vs 12.35 ms with
// every kernel remapped).
template <bool kRemap = false>
__device__ __forceinline__ int64_t first_vt() {
    const int64_t b = blockIdx.x;
    if constexpr (!kRemap) {
        return b;
    } else {
        const int64_t G = gridDim.x;
        const int64_t x = b & 7, per = G >> 3, rem = G & 7;
        return x * per + (x < rem ? x : rem) + (b >> 3);
    }
}

// Tile t and first element b of virtual tile vt: `split` blocks per tile,
// `sub` elements each (a multiple of 8, so every sub-range keeps the tile's
// phase modulo 16 bytes).
__device__ __forceinline__ void sub_range(int64_t vt, int32_t split, int64_t sub, int64_t *t,
                                          int64_t *b) {
    *t = vt / split;
    *b = (vt - *t * split) * sub;
}

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

// ---------------------------------------------------------------------------
// launch shapes (host)
// ---------------------------------------------------------------------------

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

}  // namespace

}  // namespace fsdp
