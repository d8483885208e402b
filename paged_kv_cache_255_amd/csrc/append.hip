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
    const int64_t waves = (int64_t)T * H;
    const int grid = (int)((waves + 3) / 4);
    if (D == 64)
        hipLaunchKernelGGL((append_kernel<QT, KT, 64>), dim3(grid), dim3(256), 0, s, k, v, kc, vc,
                           slots, T, H, NB, TS, ki, vi);
    else if (D == 128)
        hipLaunchKernelGGL((append_kernel<QT, KT, 128>), dim3(grid), dim3(256), 0, s, k, v, kc,
                           vc, slots, T, H, NB, TS, ki, vi);
    else
        return hipErrorInvalidValue;
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
