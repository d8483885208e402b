// Runs the balanced MFMA decode kernel (with the step's append folded in,
// with and without the shared-block hint) and the segment merge of the
// library's own device sources on the CPU: every lane is a thread, a wave is
// 64 of them, the decode's workgroups run their four waves at once,
// cross-lane operations and barriers are emulated, and the MFMA
// and conversion builtins return placeholders, so the values are not checked
// here, only the indexing.  Built with AddressSanitizer, it shows that every
// load and store stays inside its buffer, that every cross-lane operation is
// reached by all lanes, and that every output element is written.
// Input file: int32 header B maxb NB Hkv G D W max_len, then lens[B],
// tables[B][maxb], slots[B], then a share plan of 2 + 8 B words (pa.h
// layout).  argv: input, mode: 0 no plan, 1 the plan as a cache-policy hint
// only, 2 the plan with prefix rows; optional: LDS bytes per wave that hold
// a run's results until it ends (default: what the launch gives; 0 stores
// them at once).
#include <hip/hip_runtime.h>
thread_local dim3 threadIdx, blockIdx;
thread_local SimWave *g_wave;
SimBlock *g_block;
#include "decode_mfma.hip"
#include "merge.hip"
#include <cmath>
#include <thread>
#include <vector>
using namespace pa;

// All four waves of a workgroup at once (256 threads): __syncthreads waits
// for all of them, so a barrier that some wave of the workgroup misses, or
// reaches a different number of times, stops the run (DEADLOCK) instead of
// passing.
template <class F> static void run_block(unsigned block, F f)
{
    SimWave w[4];
    SimBlock blk;
    blk.total = 256;
    g_block = &blk;
    std::vector<std::thread> th;
    for (int t = 0; t < 256; ++t)
        th.emplace_back([&, t] {
            g_wave = &w[t / 64];
            threadIdx = dim3(t);
            blockIdx = dim3(block);
            f();
        });
    for (auto &x : th)
        x.join();
}

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

int main(int argc, char **argv)
{
    if (argc < 3)
        return 2;
    FILE *fp = fopen(argv[1], "rb");
    if (!fp)
        return 2;
    int32_t hdr[8];
    if (fread(hdr, 4, 8, fp) != 8)
        return 2;
    const int B = hdr[0], maxb = hdr[1], NB = hdr[2], H = hdr[3], G = hdr[4], D = hdr[5],
              W = hdr[6], maxlen = hdr[7];
    std::vector<int32_t> lens(B), tables((size_t)B * maxb), slots(B), plan(2 + 8 * (size_t)B);
    if (fread(lens.data(), 4, B, fp) != (size_t)B ||
        fread(tables.data(), 4, tables.size(), fp) != tables.size() ||
        fread(slots.data(), 4, B, fp) != (size_t)B ||
        fread(plan.data(), 4, plan.size(), fp) != plan.size())
        return 2;
    fclose(fp);
    if (D != 128)
        return 2;
    const int mode = atoi(argv[2]);
    const bool hint = mode > 0;
    // exact-size buffers, so that any access past them is reported
    const size_t cache_elems = (size_t)NB * H * 16 * D;
    std::vector<__bf16> k(cache_elems, (__bf16)0.f), v(cache_elems, (__bf16)0.f);
    const size_t q_elems = (size_t)B * H * G * D;
    std::vector<__bf16> q(q_elems, (__bf16)0.f), out(q_elems);
    std::memset(out.data(), 0xFF, 2 * q_elems);
    std::vector<__bf16> kn((size_t)B * H * D, (__bf16)0.f), vn((size_t)B * H * D, (__bf16)0.f);
    // the library's sizing: W + B Hkv sequence slots, then with prefix rows
    // (W + Hkv B / 2) pieces of 4 x 16 / G member slots
    const int64_t seq_slots = (int64_t)W + (int64_t)B * H;
    const int64_t nslots =
        seq_slots + (mode == 2 ? ((int64_t)W + (int64_t)H * (B / 2)) * prefix_row_seqs(G) : 0);
    // NaN in every slot: a merge that reads a slot no run wrote gives NaN
    std::vector<float> ws((size_t)nslots * G * (2 + D), __builtin_nanf(""));
    // the decode's record of each segment's parts (prefix rows): garbage
    // until written, so a merge that reads an entry no run wrote reads
    // the last slot (NaN) after clamping
    std::vector<int32_t> dir((size_t)B * H * 4, 0x7F7F7F7F);

    DecodeArgs a{};
    a.q = q.data(); a.k_cache = k.data(); a.v_cache = v.data(); a.block_tables = tables.data();
    a.seq_lens = lens.data(); a.seq_starts = nullptr; a.share = hint ? plan.data() : nullptr;
    a.prefix = mode == 2; a.prefix_base = seq_slots; a.seg_dir = mode == 2 ? dir.data() : nullptr;
    a.out = out.data(); a.ws = ws.data(); a.num_seqs = B; a.num_q_heads = H * G;
    a.num_kv_heads = H; a.group = G; a.num_blocks = NB; a.tile_shift = 0;
    a.max_blocks_per_seq = maxb; a.max_seq_len = maxlen; a.partition = kPartitionBalanced;
    a.max_parts = 1; a.waves = W; a.num_slots = nslots; a.score_scale = 0.1f; a.v_scale = 1.f;
    a.append = 1; a.k_new = kn.data(); a.v_new = vn.data(); a.slots = slots.data();
    a.k_inv = a.v_inv = 1.f;
    a.stage_bytes = argc > 3 ? atoi(argv[3]) : (int32_t)sizeof(u32x4) * kStageQuads;
    if (a.stage_bytes < 0 || a.stage_bytes > (int32_t)sizeof(u32x4) * kStageQuads)
        return 2;
    for (int wave = 0; wave < W; wave += 4) {
        if (hint)
            run_block(wave / 4, [&] { decode_mfma_balanced_kernel<PA_BF16, PA_BF16, 128, true>(a, W); });
        else
            run_block(wave / 4, [&] { decode_mfma_balanced_kernel<PA_BF16, PA_BF16, 128, false>(a, W); });
    }
    // prefix-row member slots the decode wrote (their m values)
    size_t row_slots = 0;
    for (int64_t w = seq_slots; w < nslots; ++w)
        row_slots += !std::isnan(ws[(size_t)w * G * 2]);
    for (int seg = 0; seg < B * H; ++seg)
        run_wave(seg, 0, [&] { merge_segment_kernel<PA_BF16, 128>(a); });
    // every element written, and none NaN: with the placeholder arithmetic
    // every real result is finite, and NaN marks an unwritten output (0xFFFF)
    // or a merge that read a slot no run wrote
    size_t unwritten = 0, nan = 0;
    const uint16_t *o16 = reinterpret_cast<const uint16_t *>(out.data());
    for (size_t e = 0; e < q_elems; ++e) {
        unwritten += (o16[e] == 0xFFFF);
        nan += ((o16[e] & 0x7F80) == 0x7F80 && (o16[e] & 0x7F) != 0);
    }
    printf("unwritten %zu of %zu, NaN %zu, row slots %zu\n", unwritten, q_elems, nan, row_slots);
    return (unwritten || nan) ? 3 : 0;
}
