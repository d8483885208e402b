// Cache append kernel: one wave per (token, KV head) writes that token's K
// row and V column into its slot (store_token, append.hpp).  A slot outside
// [0, num_blocks * block_size) is skipped.
#include <algorithm>

#include "append.hpp"

namespace pa {

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void append_kernel(const void *k, const void *v, void *k_cache,
                                                     void *v_cache, const int32_t *slots,
                                                     int32_t num_tokens, int32_t num_kv_heads,
                                                     int32_t num_blocks, int32_t tile_shift,
                                                     float k_inv, float v_inv)
{
    using TQ = typename Store<QT>::T;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= (int64_t)num_tokens * num_kv_heads)
        return;
    const int32_t t = (int32_t)(w / num_kv_heads);
    const int32_t g = (int32_t)(w % num_kv_heads);
    const int32_t slot = slots[t];
    const int32_t bs = kTile << tile_shift;
    if (slot < 0 || (int64_t)slot >= (int64_t)num_blocks * bs)
        return;
    const TQ *ks = static_cast<const TQ *>(k) + ((size_t)t * num_kv_heads + g) * D;
    const TQ *vs = static_cast<const TQ *>(v) + ((size_t)t * num_kv_heads + g) * D;
    store_token<QT, KT, D>(ks, vs, k_cache, v_cache, slot / bs, slot % bs, tile_shift, g,
                           num_kv_heads, k_inv, v_inv, lane);
}

// Value of the low (hi = false) or high half of a word of two 16-bit
// activations.
template <int QT>
__device__ __forceinline__ float half_f32(uint32_t w, bool hi)
{
    using TQ = typename Store<QT>::T;
    return to_f32<QT>(__builtin_bit_cast(TQ, (uint16_t)(hi ? w >> 16 : w & 0xFFFFu)));
}

// The same append for calls that write whole 16-token tiles (a prefill): wave
// (w, g) takes window w of the token array (entries [16 w, 16 w + 16)) for KV
// head g.  From the slots of entries [16 w - 16, 16 w + 32), one per lane, it
// finds the complete tiles: 16 entries in a row whose slots run from a
// multiple of 16 to 15 past it, all inside the pool.  At most one starts in
// the window; the wave writes it whole, its 16 K rows with 16-byte loads
// and stores, its V tile through LDS: the 16 V rows are staged dim-major,
// and each lane then gathers the 16-byte pieces of the tile layout
// (v_tile_index) it stores.  A window entry inside a complete tile that
// starts in the window before is that window's wave's; any other entry is
// written on its own as by append_kernel.  The bytes are those append_kernel
// writes.
template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void append_tiles_kernel(const void *k, const void *v,
                                                           void *k_cache, void *v_cache,
                                                           const int32_t *slots,
                                                           int32_t num_tokens,
                                                           int32_t num_kv_heads,
                                                           int32_t num_blocks, int32_t tile_shift,
                                                           float k_inv, float v_inv)
{
    using TQ = typename Store<QT>::T;
    using TK = typename Store<KT>::T;
    constexpr int QB = Store<QT>::bytes, KE = Store<KT>::bytes;
    // LDS row of one dim: 16 tokens plus 4 of padding (fewer bank
    // conflicts; keeps each 4-token group aligned for its read)
    constexpr int ROW = 20 * KE;
    __shared__ __align__(16) uint8_t stage[4][D * ROW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t wid = (int64_t)blockIdx.x * 4 + wave;
    const int64_t windows = ((int64_t)num_tokens + kTile - 1) / kTile;
    if (wid >= windows * num_kv_heads)
        return;
    const int64_t w = wid / num_kv_heads;
    const int32_t g = (int32_t)(wid % num_kv_heads);
    const int32_t bs = kTile << tile_shift;
    const int64_t cap = (int64_t)num_blocks * bs;

    // lane i: slot of entry 16 w - 16 + i (i < 48), -1 outside the array or
    // the pool
    const int64_t e = kTile * w - kTile + lane;
    int32_t s = -1;
    if (lane < 3 * kTile && e >= 0 && e < num_tokens) {
        s = slots[e];
        if (s < 0 || (int64_t)s >= cap)
            s = -1;
    }
    const int32_t s_next = __shfl_down(s, 1, kWave);
    const uint64_t links = __ballot(s >= 0 && lane + 1 < 3 * kTile && s_next == s + 1);
    const bool starts_here = s >= 0 && s % kTile == 0 && lane + kTile <= 3 * kTile &&
                             ((links >> lane) & 0x7FFFull) == 0x7FFFull;
    const uint64_t starts = __ballot(starts_here);

    const uint64_t mine = (starts >> kTile) & 0xFFFFull;
    if (mine) {
        const int p = kTile + __ffsll((unsigned long long)mine) - 1;
        const int64_t t0 = kTile * w - kTile + p;
        const int32_t s0 = __builtin_amdgcn_readlane(s, p);
        const size_t tile = (((size_t)(s0 / bs) * num_kv_heads + g) << tile_shift) +
                            (size_t)((s0 % bs) / kTile);
        TK *kd = static_cast<TK *>(k_cache) + tile * kTile * D;
        uint8_t *vd = reinterpret_cast<uint8_t *>(static_cast<TK *>(v_cache) + tile * kTile * D);
        const size_t row = (size_t)num_kv_heads * D; // source stride between tokens
        const TQ *ks = static_cast<const TQ *>(k) + ((size_t)t0 * num_kv_heads + g) * D;
        const TQ *vs = static_cast<const TQ *>(v) + ((size_t)t0 * num_kv_heads + g) * D;

        // K: the tile's 16 rows are contiguous in the cache; chunk c holds
        // cache elements [16 c / KE, 16 (c + 1) / KE)
#pragma unroll
        for (int c = lane; c < D * KE; c += kWave) {
            const int el0 = c * (16 / KE);
            const TQ *src = ks + (size_t)(el0 / D) * row + el0 % D;
            if constexpr (KE == QB) {
                *reinterpret_cast<u32x4 *>(kd + el0) = load16(src);
            } else {
                // FP8 from 16-bit activations: 16 values from two loads
                const u32x4 a = load16(src), b = load16(src + 8);
                const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                uint32_t out[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[i] = e4m3x4(half_f32<QT>(wd[2 * i], false) * k_inv,
                                    half_f32<QT>(wd[2 * i], true) * k_inv,
                                    half_f32<QT>(wd[2 * i + 1], false) * k_inv,
                                    half_f32<QT>(wd[2 * i + 1], true) * k_inv);
                *reinterpret_cast<u32x4 *>(kd + el0) = u32x4{out[0], out[1], out[2], out[3]};
            }
        }

        // V: stage the 16 rows dim-major (token u of dim d at byte
        // d ROW + u KE), converted to the cache format
        uint8_t *st = stage[wave];
#pragma unroll
        for (int c = lane; c < D * QB; c += kWave) {
            const int el0 = c * (16 / QB);
            const int u = el0 / D, d0 = el0 % D;
            const u32x4 x = load16(vs + (size_t)u * row + d0);
            if constexpr (KT == PA_FP8_E4M3) {
                // 8 values of 16 bits: two words of four codes
                const uint32_t c0 = e4m3x4(half_f32<QT>(x.x, false) * v_inv,
                                           half_f32<QT>(x.x, true) * v_inv,
                                           half_f32<QT>(x.y, false) * v_inv,
                                           half_f32<QT>(x.y, true) * v_inv);
                const uint32_t c1 = e4m3x4(half_f32<QT>(x.z, false) * v_inv,
                                           half_f32<QT>(x.z, true) * v_inv,
                                           half_f32<QT>(x.w, false) * v_inv,
                                           half_f32<QT>(x.w, true) * v_inv);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    st[(d0 + i) * ROW + u] = (uint8_t)((i < 4 ? c0 : c1) >> (8 * (i % 4)));
            } else {
                const TQ *xe = reinterpret_cast<const TQ *>(&x);
#pragma unroll
                for (int i = 0; i < 16 / QB; ++i)
                    *reinterpret_cast<TK *>(st + (d0 + i) * ROW + u * KE) = xe[i];
            }
        }
        wave_lds_sync();
        // piece 64 q + L (L = col + 16 grp) holds, for i < 4 / KE, dim
        // 16 ((4 / KE) q + i) + col of tokens 4 grp .. 4 grp + 3
        const int col = lane & 15, grp = lane >> 4;
        constexpr int PD = 4 / KE;
#pragma unroll
        for (int q = 0; q < D * KE / kWave; ++q) {
            uint32_t wds[4];
#pragma unroll
            for (int i = 0; i < PD; ++i) {
                const uint8_t *src = st + (16 * (PD * q + i) + col) * ROW + 4 * grp * KE;
                if constexpr (KE == 1) {
                    wds[i] = *reinterpret_cast<const uint32_t *>(src);
                } else if constexpr (KE == 2) {
                    const u32x2 two = *reinterpret_cast<const u32x2 *>(src);
                    wds[2 * i] = two.x;
                    wds[2 * i + 1] = two.y;
                } else {
                    const u32x4 four = *reinterpret_cast<const u32x4 *>(src);
                    wds[0] = four.x;
                    wds[1] = four.y;
                    wds[2] = four.z;
                    wds[3] = four.w;
                }
            }
            *reinterpret_cast<u32x4 *>(vd + (size_t)(kWave * q + lane) * 16) =
                u32x4{wds[0], wds[1], wds[2], wds[3]};
        }
    }

    // The window's other entries, token by token as append_kernel writes
    // them: every one's rows are loaded first, so that their latencies
    // overlap (a call of single tokens, one per sequence, has only these).
    // Entry j is left to this loop when lane 16 + j holds a slot that no
    // complete tile covers.
    const int cov = lane - (s >= 0 ? s % kTile : 0);
    const bool covered = s >= 0 && cov >= 0 && ((starts >> cov) & 1ull);
    const uint32_t todo =
        (uint32_t)(__ballot(lane >= kTile && lane < 2 * kTile && s >= 0 && !covered) >> kTile);
    if (todo == 0)
        return;
    TokenVals<QT, D> x[kTile];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
        const int64_t t = min(kTile * w + j, (int64_t)num_tokens - 1);
        x[j] = load_token<QT, D>(static_cast<const TQ *>(k) + ((size_t)t * num_kv_heads + g) * D,
                                 static_cast<const TQ *>(v) + ((size_t)t * num_kv_heads + g) * D,
                                 lane);
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
        if ((todo >> j) & 1u) {
            const int32_t sj = __builtin_amdgcn_readlane(s, kTile + j);
            put_token<QT, KT, D>(x[j], k_cache, v_cache, sj / bs, sj % bs, tile_shift, g,
                                 num_kv_heads, k_inv, v_inv, lane);
        }
    }
}

// Block copies for copy on write: for each pair (src, dst), the K and V of
// block dst (all KV heads, block_bytes each) become those of block src.
// blockIdx.y picks the pair; the threads of a row of workgroups stride over
// the block 16 bytes at a time.  A pair with an id outside [0, num_blocks)
// is skipped.  No block of a call is both a source and a destination (the
// pool holds a block whose copy is pending), so the order of pairs is free.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char *k_cache, char *v_cache,
                                                          const int32_t *pairs,
                                                          int64_t block_bytes, int32_t num_blocks)
{
    const int32_t src = pairs[2 * blockIdx.y];
    const int32_t dst = pairs[2 * blockIdx.y + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
        return;
    const int64_t step = (int64_t)gridDim.x * blockDim.x * 16;
    for (int64_t off = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes;
         off += step) {
        const u32x4 k = load16(k_cache + src * block_bytes + off);
        const u32x4 v = load16(v_cache + src * block_bytes + off);
        *reinterpret_cast<u32x4 *>(k_cache + dst * block_bytes + off) = k;
        *reinterpret_cast<u32x4 *>(v_cache + dst * block_bytes + off) = v;
    }
}

hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs,
                              int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                              hipStream_t s)
{
    if (num_pairs == 0)
        return hipSuccess;
    const int64_t threads = (block_bytes + 15) / 16;
    const int gx = (int)std::min<int64_t>((threads + 255) / 256, 64);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, num_pairs), dim3(256), 0, s,
                       static_cast<char *>(k_cache), static_cast<char *>(v_cache), pairs,
                       block_bytes, num_blocks);
    return hipGetLastError();
}

// Swap transfers: for each pair (src, dst), block dst of the destination
// caches (K and V, block_bytes each) becomes block src of the source caches.
// One side is device memory, the other the device mapping of pinned host
// memory, so the transfer is a plain load/store stream over the host link;
// blockIdx.y picks the pair.  Ids outside [0, n_src) or [0, n_dst) skip the
// pair.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const char *src_k, const char *src_v,
                                                          char *dst_k, char *dst_v,
                                                          const int32_t *pairs,
                                                          int64_t block_bytes, int32_t n_src,
                                                          int32_t n_dst)
{
    const int32_t src = pairs[2 * blockIdx.y];
    const int32_t dst = pairs[2 * blockIdx.y + 1];
    if (src < 0 || src >= n_src || dst < 0 || dst >= n_dst)
        return;
    const int64_t step = (int64_t)gridDim.x * blockDim.x * 16;
    for (int64_t off = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes;
         off += step) {
        const u32x4 k = load16(src_k + src * block_bytes + off);
        const u32x4 v = load16(src_v + src * block_bytes + off);
        *reinterpret_cast<u32x4 *>(dst_k + dst * block_bytes + off) = k;
        *reinterpret_cast<u32x4 *>(dst_v + dst * block_bytes + off) = v;
    }
}

hipError_t launch_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                              const int32_t *pairs, int32_t num_pairs, int64_t block_bytes,
                              int32_t n_src, int32_t n_dst, hipStream_t s)
{
    if (num_pairs == 0)
        return hipSuccess;
    const int64_t threads = (block_bytes + 15) / 16;
    const int gx = (int)std::min<int64_t>((threads + 255) / 256, 64);
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(gx, num_pairs), dim3(256), 0, s,
                       static_cast<const char *>(src_k), static_cast<const char *>(src_v),
                       static_cast<char *>(dst_k), static_cast<char *>(dst_v), pairs,
                       block_bytes, n_src, n_dst);
    return hipGetLastError();
}

template <int QT, int KT>
hipError_t append_by_dim(const void *k, const void *v, void *kc, void *vc, const int32_t *slots,
                         int32_t T, int32_t H, int32_t NB, int32_t TS, int D, float ki,
                         float vi, hipStream_t s)
{
    if (D != 64 && D != 128)
        return hipErrorInvalidValue;
    // Calls of kTilesFrom tokens or more (prefills) go to the tile kernel,
    // shorter ones (decode steps: one token per sequence, no whole tile) to
    // one wave per (token, KV head).  Measured on MI355X, a step of 256
    // tokens x 8 KV heads: 5.0 us one wave per (token, head), 7.4 us in the
    // tile kernel (128 waves of 16 tokens each).
    constexpr int32_t kTilesFrom = 1024;
    if (T >= kTilesFrom) {
        const int64_t waves = ((int64_t)T + kTile - 1) / kTile * H;
        const int grid = (int)((waves + 3) / 4);
        if (D == 64)
            hipLaunchKernelGGL((append_tiles_kernel<QT, KT, 64>), dim3(grid), dim3(256), 0, s, k,
                               v, kc, vc, slots, T, H, NB, TS, ki, vi);
        else
            hipLaunchKernelGGL((append_tiles_kernel<QT, KT, 128>), dim3(grid), dim3(256), 0, s,
                               k, v, kc, vc, slots, T, H, NB, TS, ki, vi);
        return hipGetLastError();
    }
    const int64_t waves = (int64_t)T * H;
    const int grid = (int)((waves + 3) / 4);
    if (D == 64)
        hipLaunchKernelGGL((append_kernel<QT, KT, 64>), dim3(grid), dim3(256), 0, s, k, v, kc, vc,
                           slots, T, H, NB, TS, ki, vi);
    else
        hipLaunchKernelGGL((append_kernel<QT, KT, 128>), dim3(grid), dim3(256), 0, s, k, v, kc,
                           vc, slots, T, H, NB, TS, ki, vi);
    return hipGetLastError();
}

hipError_t launch_append(const void *k, const void *v, void *kc, void *vc, const int32_t *slots,
                         int32_t T, int32_t H, int32_t NB, int32_t TS, int D, pa_dtype qt,
                         pa_dtype kt, float k_inv, float v_inv, hipStream_t s)
{
    if (qt == PA_F32 && kt == PA_F32)
        return append_by_dim<PA_F32, PA_F32>(k, v, kc, vc, slots, T, H, NB, TS, D, k_inv, v_inv,
                                             s);
    if (qt == PA_F16 && kt == PA_F16)
        return append_by_dim<PA_F16, PA_F16>(k, v, kc, vc, slots, T, H, NB, TS, D, k_inv, v_inv,
                                             s);
    if (qt == PA_BF16 && kt == PA_BF16)
        return append_by_dim<PA_BF16, PA_BF16>(k, v, kc, vc, slots, T, H, NB, TS, D, k_inv,
                                               v_inv, s);
    if (qt == PA_BF16 && kt == PA_FP8_E4M3)
        return append_by_dim<PA_BF16, PA_FP8_E4M3>(k, v, kc, vc, slots, T, H, NB, TS, D, k_inv,
                                                   v_inv, s);
    if (qt == PA_F16 && kt == PA_FP8_E4M3)
        return append_by_dim<PA_F16, PA_FP8_E4M3>(k, v, kc, vc, slots, T, H, NB, TS, D, k_inv,
                                                  v_inv, s);
    return hipErrorInvalidValue;
}

} // namespace pa
