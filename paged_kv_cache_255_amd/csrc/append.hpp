// One token's K row and V column for one KV head, written into its cache slot
// by one wave: the cache append of append_kernel and of the entries of
// append_tiles_kernel outside complete tiles.  (The decode launch that
// appends the step's token itself writes the same bytes from its own
// registers, MfmaWave::store_new_token; the GPU tests compare the caches.)
//
// dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
// PagedAttention Fixes It", §1: every step appends the new token's K and V to
// the cache; §4: the slot is a place inside a physical block; §6 "Enable FP8
// KV Cache": the cache may hold 1-byte FP8 values.  hyperinfer.ai, "KV cache &
// paged attention deep dive", "KV quantization cuts memory in half".
//
// Lane d writes dims d, d + 64, ...  The K row of a slot is contiguous
// ([block][head][token][dim]); V is stored per block and head as 16-token
// tiles ([block][head][token / 16][16 D], element order v_tile_index), so
// the V column of a slot is scattered over the tile.  FP8: the E4M3 code of
// x * inv (inv = 1/scale in fp32), nearest even, saturating.
#pragma once

#include "device.hpp"

namespace pa {

// One token's K row and V column values for one KV head as lane `lane`
// holds them: dims lane, lane + 64, ...
template <int QT, int D>
struct TokenVals {
    typename Store<QT>::T k[D / kWave], v[D / kWave];
};

template <int QT, int D>
__device__ __forceinline__ TokenVals<QT, D> load_token(const typename Store<QT>::T *ks,
                                                       const typename Store<QT>::T *vs, int lane)
{
    TokenVals<QT, D> x;
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) {
        x.k[i] = ks[i * kWave + lane];
        x.v[i] = vs[i * kWave + lane];
    }
    return x;
}

template <int QT, int KT, int D>
__device__ __forceinline__ void put_token(const TokenVals<QT, D> &x, void *k_cache,
                                          void *v_cache, int32_t blk, int32_t off,
                                          int32_t tile_shift, int32_t g, int32_t num_kv_heads,
                                          float k_inv, float v_inv, int lane)
{
    using TK = typename Store<KT>::T;
    // first tile of (blk, g); `off` (0 .. block_size - 1) is in tile off / 16
    const size_t tile0 = ((size_t)blk * num_kv_heads + g) << tile_shift;
    TK *kd = static_cast<TK *>(k_cache) + (tile0 * kTile + off) * D;
    TK *vd = static_cast<TK *>(v_cache) + (tile0 + off / kTile) * D * kTile;
    const int u = off % kTile;
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) {
        const int d = i * kWave + lane;
        const int vi = v_tile_index<Store<KT>::bytes>(u, d);
        if constexpr (KT == PA_FP8_E4M3) {
            kd[d] = f32_to_e4m3(to_f32<QT>(x.k[i]) * k_inv);
            vd[vi] = f32_to_e4m3(to_f32<QT>(x.v[i]) * v_inv);
        } else {
            kd[d] = x.k[i];
            vd[vi] = x.v[i];
        }
    }
}

template <int QT, int KT, int D>
__device__ __forceinline__ void store_token(const typename Store<QT>::T *ks,
                                            const typename Store<QT>::T *vs, void *k_cache,
                                            void *v_cache, int32_t blk, int32_t off,
                                            int32_t tile_shift, int32_t g, int32_t num_kv_heads,
                                            float k_inv, float v_inv, int lane)
{
    put_token<QT, KT, D>(load_token<QT, D>(ks, vs, lane), k_cache, v_cache, blk, off, tile_shift,
                         g, num_kv_heads, k_inv, v_inv, lane);
}

} // namespace pa
