// Read ceiling of the GPU: the rate one streaming read of a large buffer
// reaches, the practical roof for a kernel whose time is its HBM reads
// (vaibhawkumar.in, "Why LLMs run out of VRAM...", "Why fragmentation matters
// more than bandwidth": decode is bound by how fast the cache can be read).
// The decode kernels are reported against the vendor peak and against this.
//
// Each lane reads 16 bytes per load, N loads in flight: load k of lane t in
// round r reads 16-byte piece t + (r N + k) S of the buffer (S = threads of the
// grid), so one load instruction of a wave covers 1 KiB contiguous.  The
// values are XOR-folded and the fold is written only if it equals a constant
// (in practice never), so every load is needed and nothing else is stored.
#include <map>
#include <mutex>

#include "device.hpp"

namespace pa {

template <int N, bool STREAM>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *buf, int64_t pieces,
                                                          uint32_t *sink)
{
    const int64_t S = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (N - 1) * S < pieces; i += N * S) {
        u32x4 v[N];
#pragma unroll
        for (int k = 0; k < N; ++k)
            v[k] = STREAM ? load16_stream(buf + i + k * S) : load16(buf + i + k * S);
#pragma unroll
        for (int k = 0; k < N; ++k)
            acc ^= v[k];
    }
    for (; i < pieces; i += S)
        acc ^= load16(buf + i);
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u)
        sink[0] = acc.x;
}

// LDS a workgroup asks for so that a CU holds one of them (one wave per SIMD),
// as the balanced decode launch does; 0 if the device cannot grant it.
static int one_per_cu_lds()
{
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end())
        return it->second;
    int per_cu = 0, per_block = 0;
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
        return 0;
    int want = per_cu / 2 + 1024;
    if (want > per_block)
        want = 0;
    cache[dev] = want;
    return want;
}

template <int N>
static hipError_t probe_n(const void *buf, int64_t pieces, int32_t wgs, bool stream,
                          bool one_per_cu, uint32_t *sink, hipStream_t s)
{
    const int lds = one_per_cu ? one_per_cu_lds() : 0;
    const u32x4 *b = static_cast<const u32x4 *>(buf);
    if (stream)
        hipLaunchKernelGGL((read_probe_kernel<N, true>), dim3(wgs), dim3(256), lds, s, b, pieces,
                           sink);
    else
        hipLaunchKernelGGL((read_probe_kernel<N, false>), dim3(wgs), dim3(256), lds, s, b, pieces,
                           sink);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, int64_t pieces, int32_t loads, int32_t wgs,
                             bool stream, bool one_per_cu, uint32_t *sink, hipStream_t s)
{
    switch (loads) {
    case 4: return probe_n<4>(buf, pieces, wgs, stream, one_per_cu, sink, s);
    case 8: return probe_n<8>(buf, pieces, wgs, stream, one_per_cu, sink, s);
    case 16: return probe_n<16>(buf, pieces, wgs, stream, one_per_cu, sink, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace pa
