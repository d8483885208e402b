// Runs the whole-tile cache append (append_tiles_kernel) and the per-token
// one (append_kernel) of the library's device sources on the CPU, each lane a
// thread, on the same tokens, and compares the two caches byte for byte.
// Built with AddressSanitizer, it also shows that every load and store of
// the tile kernel stays inside its buffers.
// Input file: int32 header T H NB tile_shift kv (0: bf16, 1: FP8 E4M3 under
// bf16), then slots[T].  Exit 0 when the caches match.
#include <hip/hip_runtime.h>
thread_local dim3 threadIdx, blockIdx;
// the copy kernels of append.hip read these; the append kernels do not
static const dim3 gridDim(1), blockDim(256);
thread_local SimWave *g_wave;
SimBlock *g_block;
#include "append.hip"
#include <random>
#include <thread>
#include <vector>
using namespace pa;

template <class F> static void run_wave(unsigned block, unsigned wave_in_block, F f)
{
    SimWave w;
    SimBlock blk;
    blk.total = 64;
    g_block = &blk;
    std::vector<std::thread> th;
    for (int l = 0; l < 64; ++l)
        th.emplace_back([&, l] {
            g_wave = &w;
            threadIdx = dim3(wave_in_block * 64 + l);
            blockIdx = dim3(block);
            f();
        });
    for (auto &t : th)
        t.join();
}

template <int KT>
static int run(int T, int H, int NB, int TS, const std::vector<int32_t> &slots)
{
    constexpr int D = 128;
    const int KE = Store<KT>::bytes;
    std::mt19937 rng(1234);
    std::normal_distribution<float> nd(0.f, 1.f);
    std::vector<__bf16> k((size_t)T * H * D), v((size_t)T * H * D);
    for (auto &x : k) x = (__bf16)nd(rng);
    for (auto &x : v) x = (__bf16)nd(rng);
    const size_t cache_bytes = (size_t)NB * H * (16 << TS) * D * KE;
    std::vector<uint8_t> kc_a(cache_bytes, 0xA5), vc_a(cache_bytes, 0xA5);
    std::vector<uint8_t> kc_b(cache_bytes, 0xA5), vc_b(cache_bytes, 0xA5);
    const float ki = 1.0f / 0.75f, vi = 1.0f / 1.25f;
    // per-token reference: one wave per (token, KV head)
    const int64_t waves_a = (int64_t)T * H;
    for (int64_t wv = 0; wv < waves_a; ++wv)
        run_wave((unsigned)(wv / 4), (unsigned)(wv % 4), [&] {
            append_kernel<PA_BF16, KT, D>(k.data(), v.data(), kc_a.data(), vc_a.data(),
                                          slots.data(), T, H, NB, TS, ki, vi);
        });
    // tile kernel: one wave per (16-entry window, KV head)
    const int64_t waves_b = ((int64_t)T + 15) / 16 * H;
    for (int64_t wv = 0; wv < waves_b; ++wv)
        run_wave((unsigned)(wv / 4), (unsigned)(wv % 4), [&] {
            append_tiles_kernel<PA_BF16, KT, D>(k.data(), v.data(), kc_b.data(), vc_b.data(),
                                                slots.data(), T, H, NB, TS, ki, vi);
        });
    size_t dk = 0, dv = 0, first_k = SIZE_MAX, first_v = SIZE_MAX;
    for (size_t i = 0; i < cache_bytes; ++i) {
        if (kc_a[i] != kc_b[i] && dk++ == 0)
            first_k = i;
        if (vc_a[i] != vc_b[i] && dv++ == 0)
            first_v = i;
    }
    const size_t diff = dk + dv;
    printf("bytes %zu, differing %zu (K %zu first %zd, V %zu first %zd)\n", 2 * cache_bytes, diff,
           dk, (ssize_t)first_k, dv, (ssize_t)first_v);
    return diff ? 3 : 0;
}

int main(int argc, char **argv)
{
    if (argc < 2)
        return 2;
    FILE *fp = fopen(argv[1], "rb");
    if (!fp)
        return 2;
    int32_t hdr[5];
    if (fread(hdr, 4, 5, fp) != 5)
        return 2;
    const int T = hdr[0], H = hdr[1], NB = hdr[2], TS = hdr[3], kv = hdr[4];
    std::vector<int32_t> slots(T);
    if (fread(slots.data(), 4, T, fp) != (size_t)T)
        return 2;
    fclose(fp);
    return kv == 0 ? run<PA_BF16>(T, H, NB, TS, slots) : run<PA_FP8_E4M3>(T, H, NB, TS, slots);
}
