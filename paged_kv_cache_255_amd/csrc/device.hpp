// Device-side helpers for the gfx950 kernels: storage types, conversions,
// cross-lane reductions.  Everything here runs on the GPU only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kWave = 64;     // CDNA wavefront width
// Tokens per tile, the kernels' unit of work.  A cache block of block_size
// tokens (16, 32, 64, 128 or 256) is block_size / 16 consecutive tiles, each
// with the same layout as a 16-token block.
constexpr int kTile = 16;
constexpr float kLog2e = 1.4426950408889634f;

// Element of token u (0..15) and dim d inside one V tile (16 tokens x D dims,
// KE bytes per element), p = 4 / KE: each 16-byte piece holds p dims, 16
// apart, of 4 consecutive tokens.  Piece (d / 16p) * 64 + (u / 4) * 16 + d % 16
// holds the value at place ((d / 16) % p) * 4 + u % 4.  So one load
// instruction reads 1 KiB of the tile with lane L taking piece 64 q + L, and
// lane (col, grp) = (L % 16, L / 16) gets dims 16 (p q + i) + col (i < p) of
// tokens 4 grp .. 4 grp + 3: the V^T operand of the 16x16x16 MFMA, p
// products' worth per 16 bytes.  D is a multiple of 16 p.
template <int KE>
__host__ __device__ constexpr int v_tile_index(int u, int d)
{
    constexpr int p = 4 / KE;
    const int piece = (d / (16 * p)) * 64 + (u / 4) * 16 + d % 16;
    return piece * 4 * p + ((d / 16) % p) * 4 + u % 4;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- storage types ---------------------------------------------------------
template <int DT> struct Store;
template <> struct Store<PA_F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Store<PA_F16> { using T = _Float16; static constexpr int bytes = 2; };
template <> struct Store<PA_BF16> { using T = __bf16; static constexpr int bytes = 2; };
template <> struct Store<PA_FP8_E4M3> { using T = uint8_t; static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Two E4M3 bytes (word `hi` of w) -> two floats, hardware conversion.
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w, bool hi)
{
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

// Unpacks one 16-byte chunk of stored values into floats (16/bytes values).
template <int DT> struct Chunk;
template <> struct Chunk<PA_F32> {
    static constexpr int N = 4;
    __device__ static void unpack(const u32x4 c, float *o)
    {
        o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
        o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
    }
};
template <> struct Chunk<PA_BF16> {
    static constexpr int N = 8;
    __device__ static void unpack(const u32x4 c, float *o)
    {
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(w[i]); o[2 * i + 1] = bf16_hi(w[i]); }
    }
};
template <> struct Chunk<PA_F16> {
    static constexpr int N = 8;
    __device__ static void unpack(const u32x4 c, float *o)
    {
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[2 * i] = f16_lo(w[i]); o[2 * i + 1] = f16_hi(w[i]); }
    }
};
template <> struct Chunk<PA_FP8_E4M3> {
    static constexpr int N = 16;
    __device__ static void unpack(const u32x4 c, float *o)
    {
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 a = fp8x2_to_f32(w[i], false);
            f32x2 b = fp8x2_to_f32(w[i], true);
            o[4 * i] = a.x; o[4 * i + 1] = a.y; o[4 * i + 2] = b.x; o[4 * i + 3] = b.y;
        }
    }
};

// ---- scalar conversions ----------------------------------------------------
template <int DT> __device__ __forceinline__ float to_f32(typename Store<DT>::T x);
template <> __device__ __forceinline__ float to_f32<PA_F32>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<PA_F16>(_Float16 x) { return (float)x; }
template <> __device__ __forceinline__ float to_f32<PA_BF16>(__bf16 x) { return (float)x; }

// Round to nearest even (the compiler lowers these to v_cvt_*_f32, RNE).
template <int DT> __device__ __forceinline__ typename Store<DT>::T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<PA_F32>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<PA_F16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<PA_BF16>(float x) { return (__bf16)x; }

// fp32 -> E4M3FN, nearest value with ties to the even code, saturating at
// +-448, NaN -> 0x7F with the sign kept.  The conversion instruction
// (v_cvt_pk_fp8_f32) rounds to nearest even but neither saturates (an input
// past the largest code becomes NaN) nor keeps a NaN through the clamp that
// would make it saturate; so the input is clamped to +-448 (v_med3_f32) and
// a NaN input is encoded by hand.  Measured on MI355X over all 2^32 fp32 bit
// patterns: identical to a bit-level definition (keep the top 3 mantissa
// bits with round-half-even on the dropped ones, subnormals below 2^-6 as
// integer counts of 2^-9, saturation at 448), and clamp without the NaN case
// differs on every NaN, no clamp on every input past 464.
__device__ __forceinline__ float e4m3_clamp(float x)
{
    return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f);
}

__device__ __forceinline__ uint32_t e4m3_nan_code(float x)
{
    return ((__float_as_uint(x) >> 24) & 0x80u) | 0x7Fu;
}

// Four values, packed low byte first.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), (int)w, true);
    if (__builtin_isnan(a) || __builtin_isnan(b) || __builtin_isnan(c) || __builtin_isnan(d)) {
        const float x[4] = {a, b, c, d};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (__builtin_isnan(x[i]))
                w = (w & ~(0xFFu << (8 * i))) | (e4m3_nan_code(x[i]) << (8 * i));
    }
    return w;
}

__device__ __forceinline__ uint8_t f32_to_e4m3(float x)
{
    if (__builtin_isnan(x))
        return (uint8_t)e4m3_nan_code(x);
    const float c = e4m3_clamp(x);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFF);
}

// s_waitcnt operand that waits for vmcnt == 0 and leaves the expcnt and
// lgkmcnt fields at their maxima (no wait): gfx9 encoding.
constexpr int kWaitVmcnt0 = 0x0F70;

// ---- cross-lane ------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask)
{
    return __shfl_xor(v, mask, kWave);
}

// Max / sum of v over the lane pairs (l, l^16) and (l, l^32), with the
// gfx950 permlane swaps (plain VALU: no LDS queue, nothing for a wait
// counter).  Passing v as both operands, one result holds each lane's own row
// (or half) and the other its partner's, so combining them is the reduction.
__device__ __forceinline__ f32x2 pair_xor16(float v)
{
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 pair_xor32(float v)
{
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor16(float v) { const f32x2 p = pair_xor16(v); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float max_xor32(float v) { const f32x2 p = pair_xor32(v); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor16(float v) { const f32x2 p = pair_xor16(v); return p.x + p.y; }
__device__ __forceinline__ float sum_xor32(float v) { const f32x2 p = pair_xor32(v); return p.x + p.y; }

// Orders this wave's LDS accesses in program order for the compiler; the
// hardware already executes one wave's LDS instructions in order.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A value every lane of the wave reads from the same address, in memory the
// launch does not write (lengths, tables, plans), read with a scalar load.
// Its wait is on the scalar counter: a vector load's wait would also wait
// for every vector store the wave issued before it (the vector memory
// counter covers stores), such as the partial states a piece just wrote.
// The address goes through readfirstlane: computed from an index the
// compiler keeps in a vector register, it would otherwise become a vector
// load after all.
__device__ __forceinline__ int32_t uniform_load(const int32_t *p)
{
    using CI32 = __attribute__((address_space(4))) const int32_t;
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_readfirstlane(*(const CI32 *)((hi << 32) | lo));
}

__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Streaming loads (the nontemporal hint): for data read once per launch, the
// KV tiles.  Measured on MI355X, a read stream with this hint at one wave
// per SIMD and 8 x 16 B in flight per lane reached 7.27 TB/s, against
// 6.47 TB/s for plain loads.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Loads 16 bytes per lane from global memory straight into LDS (lane l's
// bytes land at lds + 16 l): a load the compiler keeps although no register
// receives it, used to bring data into the caches ahead of the loads that
// need it.  lds must be wave-uniform and hold 1 KiB.
__device__ __forceinline__ void load16_to_lds(const void *src, void *lds)
{
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)src,
        (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

} // namespace pa
