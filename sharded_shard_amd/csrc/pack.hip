// All-gather copy-ins of the sharded step: fp32 master shards -> bf16 (round
// to nearest even) or FP8 E4M3 (scaled, saturating) segment with zero
// padding, and the per-parameter amax that sets the FP8 scales.
#include "device.hpp"
#include "launch.hpp"

// copy-in: non-temporal loads and stores
#ifndef FSDP_PACK_POL
#define FSDP_PACK_POL 3
#endif
// elements per block of the copy-in (1024 and 4096 measured slower)
#ifndef FSDP_PACK_SUB
#define FSDP_PACK_SUB 2048
#endif
// FP8 copy-in: plain loads and stores (non-temporal loads cost it a third)
#ifndef FSDP_FP8_POL
#define FSDP_FP8_POL 0
#endif
// elements per block of the FP8 copy-in (2048 and 1024 measured 10% and 34%
// slower)
#ifndef FSDP_FP8_SUB
#define FSDP_FP8_SUB 4096
#endif
// elements per block of the amax
#ifndef FSDP_AMAX_SUB
#define FSDP_AMAX_SUB 4096
#endif

namespace fsdp {

namespace {

// ---------------------------------------------------------------------------
// copy-in: fp32 master shards -> bf16 segment (zeros in padding)
// ---------------------------------------------------------------------------

// Copy-in vectors: dv[v] = bf16 of s[8v .. 8v + 8) for v < nvec, s 16-byte
// aligned.
template <int LN, int SN>
__device__ __forceinline__ void pack_vec(u32x4 *__restrict__ dv, const float *__restrict__ s,
                                         int64_t nvec) {
    int64_t v = threadIdx.x;
    for (; v + kBlock < nvec; v += 2 * kBlock) {
        f32x4 a0, a1, b0, b1;
        load8f<LN, true>(s + (v << 3), 0u, a0, a1);
        load8f<LN, true>(s + ((v + kBlock) << 3), 0u, b0, b1);
        stp<SN>(dv + v, u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w), pack2(a1.x, a1.y),
                              pack2(a1.z, a1.w)});
        stp<SN>(dv + v + kBlock, u32x4{pack2(b0.x, b0.y), pack2(b0.z, b0.w), pack2(b1.x, b1.y),
                                       pack2(b1.z, b1.w)});
    }
    if (v < nvec) {
        f32x4 a0, a1;
        load8f<LN, true>(s + (v << 3), 0u, a0, a1);
        stp<SN>(dv + v, u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w), pack2(a1.x, a1.y),
                              pack2(a1.z, a1.w)});
    }
}

// The same from a source whose dword index modulo 4 is q (1..3): lane l
// loads the two aligned 16-byte chunks holding the start of its eight
// elements, takes the third from lane l + 1 (DPP; lane 63 loads its own with
// a load whose other lanes read nothing) and selects: every chunk is read
// once (a third load per lane instead measured 5% slower on the ragged MoE
// rows).  Whole waves iterate together.  The stores go through a buffer
// range of exactly the nvec vectors: with a branch around them instead the
// compiler issued the second load only after the first had returned, and
// under the non-temporal hint the lines the two loads share were often
// fetched twice (ragged MoE rows: reads 1.41x the algorithmic bytes by the
// request counters, now 1.02x; the copy-in 4.23 -> 4.79 TB/s).
template <int LN, int SN>
__device__ __forceinline__ void pack_vec_mis(u32x4 *__restrict__ dv, const float *__restrict__ s,
                                             int64_t nvec, uint32_t q) {
    const char *al = reinterpret_cast<const char *>(s - q);
    const uint32_t nb = (4u * (q + 8u * static_cast<uint32_t>(nvec)) + 15u) & ~15u;
    char *dst = reinterpret_cast<char *>(dv);
    const uint32_t db = static_cast<uint32_t>(nvec) << 4;
    const uint32_t lane = threadIdx.x & 63;
    const bool last = lane == 63;
    for (int64_t w0 = threadIdx.x - lane; w0 < nvec; w0 += kBlock) {
        const uint32_t v = static_cast<uint32_t>(w0 + lane);
        const uint32_t o = v << 5;
        const f32x4 c0 = __builtin_bit_cast(f32x4, bload16<LN>(al, o, nb));
        const f32x4 c1 = __builtin_bit_cast(f32x4, bload16<LN>(al, o + 16u, nb));
        const u32x4 e = bload16<kBoundaryNT>(al, last ? o + 32u : nb, nb);
        const u32x4 c2 = next_or_own(__builtin_bit_cast(u32x4, c0), e);
        f32x4 a0, a1;
        select8f(c0, c1, __builtin_bit_cast(f32x4, c2), q, a0, a1);
        bstore16<SN>(dst, v << 4, db,
                     u32x4{pack2(a0.x, a0.y), pack2(a0.z, a0.w), pack2(a1.x, a1.y),
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
    if (q == 0) pack_vec<LN, SN>(dv, s, nvec);
    else pack_vec_mis<LN, SN>(dv, s, nvec, q);
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
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
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
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
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
    for (int64_t vt = first_vt(); vt < nvt; vt += gridDim.x) {
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

hipError_t launch_pack_fp8(const PackTile *tiles, int64_t n, const DevEntry *ents, uint8_t *ag_in,
                           const float *scales, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int32_t sp = split_for(kTilePack, FSDP_FP8_SUB);
    pack_fp8_kernel<FSDP_FP8_POL><<<grid_for(n, sp), kBlock, 0, st>>>(
        tiles, n, sp, kTilePack / sp, ents, ag_in, scales);
    return hipGetLastError();
}

hipError_t launch_amax(const EwTile *tiles, int64_t n, const DevEntry *ents, float *amax,
                       int32_t n_params, hipStream_t st) {
    if (n_params == 0) return hipSuccess;
    zero_floats_kernel<<<(n_params + kBlock - 1) / kBlock, kBlock, 0, st>>>(amax, n_params);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    const int32_t sp = split_for(kTileAdamw, FSDP_AMAX_SUB);
    amax_kernel<<<grid_for(n, sp), kBlock, 0, st>>>(tiles, n, sp, kTileAdamw / sp, ents,
                                                    reinterpret_cast<uint32_t *>(amax));
    return hipGetLastError();
}

}  // namespace fsdp
