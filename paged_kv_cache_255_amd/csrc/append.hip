// Cache append: scatter each new token's K and V into its slot.
//
// dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
// PagedAttention Fixes It", §1: every step appends the new token's K and V to
// the cache; §4: the slot is a place inside a physical block; §6 "Enable FP8
// KV Cache": the cache may hold 1-byte FP8 values.  hyperinfer.ai, "KV cache &
// paged attention deep dive", "KV quantization cuts memory in half".
//
// One wave per (token, KV head); lane d writes dims d, d + 64, ...  The K row
// of a slot is contiguous ([block][head][token][dim]); the V column is strided
// by the block size ([block][head][dim][token]).
#include "device.hpp"

namespace pa {

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void append_kernel(const void *k, const void *v, void *k_cache,
                                                     void *v_cache, const int32_t *slots,
                                                     int32_t num_tokens, int32_t num_kv_heads,
                                                     int32_t num_blocks, float k_inv, float v_inv)
{
    using TQ = typename Store<QT>::T;
    using TK = typename Store<KT>::T;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= (int64_t)num_tokens * num_kv_heads)
        return;
    const int32_t t = (int32_t)(w / num_kv_heads);
    const int32_t g = (int32_t)(w % num_kv_heads);
    const int32_t slot = slots[t];
    if (slot < 0 || (int64_t)slot >= (int64_t)num_blocks * kBlockSize)
        return;
    const int32_t blk = slot / kBlockSize;
    const int32_t off = slot % kBlockSize;
    const TQ *ks = static_cast<const TQ *>(k) + ((size_t)t * num_kv_heads + g) * D;
    const TQ *vs = static_cast<const TQ *>(v) + ((size_t)t * num_kv_heads + g) * D;
    TK *kd = static_cast<TK *>(k_cache) + (((size_t)blk * num_kv_heads + g) * kBlockSize + off) * D;
    TK *vd = static_cast<TK *>(v_cache) + ((size_t)blk * num_kv_heads + g) * D * kBlockSize + off;
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) {
        const int d = i * kWave + lane;
        if constexpr (KT == PA_FP8_E4M3) {
            kd[d] = f32_to_e4m3(to_f32<QT>(ks[d]) * k_inv);
            vd[(size_t)d * kBlockSize] = f32_to_e4m3(to_f32<QT>(vs[d]) * v_inv);
        } else {
            kd[d] = ks[d];
            vd[(size_t)d * kBlockSize] = vs[d];
        }
    }
}

template <int QT, int KT>
hipError_t append_by_dim(const void *k, const void *v, void *kc, void *vc, const int32_t *slots,
                         int32_t T, int32_t H, int32_t NB, int D, float ki, float vi,
                         hipStream_t s)
{
    const int64_t waves = (int64_t)T * H;
    const int grid = (int)((waves + 3) / 4);
    if (D == 64)
        hipLaunchKernelGGL((append_kernel<QT, KT, 64>), dim3(grid), dim3(256), 0, s, k, v, kc, vc,
                           slots, T, H, NB, ki, vi);
    else if (D == 128)
        hipLaunchKernelGGL((append_kernel<QT, KT, 128>), dim3(grid), dim3(256), 0, s, k, v, kc,
                           vc, slots, T, H, NB, ki, vi);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_append(const void *k, const void *v, void *kc, void *vc, const int32_t *slots,
                         int32_t T, int32_t H, int32_t NB, int D, pa_dtype qt, pa_dtype kt,
                         float k_inv, float v_inv, hipStream_t s)
{
    if (qt == PA_F32 && kt == PA_F32)
        return append_by_dim<PA_F32, PA_F32>(k, v, kc, vc, slots, T, H, NB, D, k_inv, v_inv, s);
    if (qt == PA_F16 && kt == PA_F16)
        return append_by_dim<PA_F16, PA_F16>(k, v, kc, vc, slots, T, H, NB, D, k_inv, v_inv, s);
    if (qt == PA_BF16 && kt == PA_BF16)
        return append_by_dim<PA_BF16, PA_BF16>(k, v, kc, vc, slots, T, H, NB, D, k_inv, v_inv, s);
    if (qt == PA_BF16 && kt == PA_FP8_E4M3)
        return append_by_dim<PA_BF16, PA_FP8_E4M3>(k, v, kc, vc, slots, T, H, NB, D, k_inv, v_inv,
                                                   s);
    if (qt == PA_F16 && kt == PA_FP8_E4M3)
        return append_by_dim<PA_F16, PA_FP8_E4M3>(k, v, kc, vc, slots, T, H, NB, D, k_inv, v_inv,
                                                  s);
    return hipErrorInvalidValue;
}

} // namespace pa
