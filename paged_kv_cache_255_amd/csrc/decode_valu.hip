// PagedAttention decode on the vector ALU: one wave per work item (sequence,
// KV head, token range), fp32 arithmetic for every storage dtype.
//
// What it computes: dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation
// and How PagedAttention Fixes It", §1 (attention formula, decode of one new
// query against the cached K/V) and §4 "The PagedAttention CUDA Kernel" (the
// query walks its block table and reads K/V from scattered physical blocks).
// The softmax is evaluated online (running max m, running sum l, rescaled
// accumulator), one 16-token tile at a time, in log2 units.  A cache block of
// 16 << k tokens is 1 << k consecutive tiles of the layout below.
//
// Lane layout inside a wave, per 16-token tile:
//   K tile [16][D]: lane = 4 * token + c; lane c of a quad reads 16-byte
//     chunks c, c+4, c+8, ... of its token's row, so each load instruction
//     covers 64 contiguous bytes of every row.  Partial dot products are
//     summed over the quad.
//   V tile (element order v_tile_index): read 1 KiB per instruction, 16
//     bytes per lane; lane L holds dims 16 j + L % 16 of tokens
//     4 (L / 16) .. 4 (L / 16) + 3 and accumulates them; the four lanes of a
//     dim (L % 16 equal) are combined at the end.
//   The probabilities move from the K layout to the V layout through LDS.
#include "device.hpp"
#include "work.hpp"

namespace pa {

template <int QT, int KT, int D, int G>
struct ValuShape {
    using TQ = typename Store<QT>::T;
    static constexpr int KE = Store<KT>::bytes;
    static constexpr int ROW_BYTES = D * KE;          // one K row
    static constexpr int CHUNKS = ROW_BYTES / 16;     // 16-byte chunks in a K row
    static constexpr int CH_PER_LANE = CHUNKS / 4;
    static constexpr int EPC = 16 / KE;               // elements per chunk
    static constexpr int VP = 4 / KE;                 // dims per 16-byte V piece
    static constexpr int V_INSTR = D / (16 * VP);     // 1 KiB V loads per tile
    static constexpr int VD = D / 16;                 // dims per lane
    static constexpr int TILE_BYTES = kTile * D * KE;
    static_assert(CH_PER_LANE >= 1 && CHUNKS % 4 == 0, "K row too short for quad layout");
    static_assert(V_INSTR >= 1 && D % (16 * VP) == 0, "V tile layout");
};

template <int QT, int KT, int D, int G>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a, int32_t num_items)
{
    using S = ValuShape<QT, KT, D, G>;
    using TQ = typename S::TQ;
    __shared__ float p_lds[4][G][kTile];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t w = blockIdx.x * 4 + wid;
    if (w >= num_items)
        return;
    const Item it = item_of(a, w);
    if (it.valid_len && it.n > 0 && it.t0 >= it.t1)
        return; // part beyond the end of this sequence
    if (it.valid_len && it.n == 0 && it.p > 0)
        return;

    const int tq = lane >> 2;    // token of this lane in the K layout
    const int cq = lane & 3;     // quad lane
    const int vdim = lane & 15;        // V: dims 16 j + vdim
    const int vtok0 = 4 * (lane >> 4); // of tokens vtok0 .. vtok0 + 3

    // q of the G heads, the slice matching this lane's K chunks, in fp32.
    float qv[G][S::CH_PER_LANE][S::EPC];
    {
        const TQ *qp = static_cast<const TQ *>(a.q) +
                       ((size_t)it.b * a.num_q_heads + (size_t)it.g * G) * D;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < S::CH_PER_LANE; ++j)
#pragma unroll
                for (int e = 0; e < S::EPC; ++e)
                    qv[h][j][e] = to_f32<QT>(qp[h * D + (cq + 4 * j) * S::EPC + e]) * a.score_scale;
    }

    float m[G], l[G], acc[G][S::VD];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kMaxStart;
        l[h] = 0.f;
#pragma unroll
        for (int j = 0; j < S::VD; ++j)
            acc[h][j] = 0.f;
    }

    // window start: tokens before it are left out (n = 0 rows are not read)
    const bool windowed = a.seq_starts && it.valid_len && it.n > 0;
    const int32_t w0 = windowed ? __builtin_amdgcn_readfirstlane(a.seq_starts[it.b]) : 0;
    bool bad = !it.valid_len || w0 < 0 || w0 > it.n;
    // Block ids come through scalar loads (the table does not change while
    // the kernel runs), so waiting for one never waits for tile loads.
    using CI32 = __attribute__((address_space(4))) const int32_t;
    const CI32 *table = (const CI32 *)(a.block_tables + (size_t)it.b * a.max_blocks_per_seq);
    const char *kbase = static_cast<const char *>(a.k_cache);
    const char *vbase = static_cast<const char *>(a.v_cache);
    const int32_t sh = a.tile_shift; // a block is 1 << sh tiles
    const int32_t jb0 = uniform(it.t0 / kTile);
    const int32_t jb1 = bad ? jb0 : uniform((it.t1 + kTile - 1) / kTile);

    // One tile as loaded: this lane's K chunks of token tq, and V pieces
    // 64 i + lane (dims 16 (VP i + e) + vdim of tokens vtok0 .., places 4 e ..).
    struct Raw {
        u32x4 k[S::CH_PER_LANE];
        u32x4 v[S::V_INSTR];
    };
    // Block id of tile jb (clamped to the last tile); an id outside the pool
    // is recorded and block 0 read in its place.
    auto id_of = [&](int32_t jb) -> int32_t {
        const int32_t p = uniform(table[uniform(min(jb, jb1 - 1) >> sh)]);
        const bool out = (uint32_t)p >= (uint32_t)a.num_blocks;
        bad |= out;
        return out ? 0 : p;
    };
    // every tile with the streaming (read-once) hint; this kernel does not
    // use the seq_shared hint
    auto load = [&](int32_t jb, int32_t phys, Raw &R) {
        jb = min(jb, jb1 - 1);
        const size_t tile =
            ((((size_t)phys * a.num_kv_heads + it.g) << sh) + (jb & ((1 << sh) - 1))) *
            S::TILE_BYTES;
        const char *kp = kbase + tile + tq * S::ROW_BYTES + cq * 16;
        const char *vp = vbase + tile + lane * 16;
#pragma unroll
        for (int j = 0; j < S::CH_PER_LANE; ++j)
            R.k[j] = load16_stream(kp + 64 * j);
#pragma unroll
        for (int i = 0; i < S::V_INSTR; ++i)
            R.v[i] = load16_stream(vp + i * 1024);
    };
    auto compute = [&](const Raw &R, int32_t jb) {
        const int32_t tok_base = jb * kTile;
        const bool tail = tok_base + kTile > it.t1 || tok_base < w0;
        float kv[S::CH_PER_LANE][S::EPC];
#pragma unroll
        for (int j = 0; j < S::CH_PER_LANE; ++j)
            Chunk<KT>::unpack(R.k[j], kv[j]);
        float vv[S::VD][4];
#pragma unroll
        for (int i = 0; i < S::V_INSTR; ++i) {
            float e[4 * S::VP];
            Chunk<KT>::unpack(R.v[i], e);
#pragma unroll
            for (int x = 0; x < S::VP; ++x)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vv[S::VP * i + x][r] = e[4 * x + r];
        }

        // scores of token tq for the G heads (log2 units)
        const bool tok_ok = tok_base + tq < it.t1 && tok_base + tq >= w0;
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int j = 0; j < S::CH_PER_LANE; ++j)
#pragma unroll
                for (int e = 0; e < S::EPC; ++e)
                    d = fmaf(qv[h][j][e], kv[j][e], d);
            d += shfl_xor(d, 1);
            d += shfl_xor(d, 2);
            s[h] = tok_ok ? d : -INFINITY;
        }
        // online softmax update, tile max over the whole wave
        float pr[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float bm = s[h];
            bm = fmaxf(bm, shfl_xor(bm, 4));
            bm = fmaxf(bm, shfl_xor(bm, 8));
            bm = fmaxf(bm, shfl_xor(bm, 16));
            bm = fmaxf(bm, shfl_xor(bm, 32));
            const float mn = fmaxf(m[h], bm);
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
            m[h] = mn;
            pr[h] = __builtin_amdgcn_exp2f(s[h] - mn);
            l[h] = fmaf(l[h], alpha, pr[h]);
#pragma unroll
            for (int j = 0; j < S::VD; ++j)
                acc[h][j] *= alpha;
        }
        // K layout -> V layout for the probabilities
#pragma unroll
        for (int h = cq; h < G; h += 4)
            p_lds[wid][h][tq] = pr[h];
        wave_lds_sync();
        if (tail) {
#pragma unroll
            for (int j = 0; j < S::VD; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (tok_base + vtok0 + r >= it.t1 || tok_base + vtok0 + r < w0)
                        vv[j][r] = 0.f; // slots outside the range may hold anything
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pv[r] = p_lds[wid][h][vtok0 + r];
#pragma unroll
            for (int j = 0; j < S::VD; ++j) {
                float t = acc[h][j];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    t = fmaf(pv[r], vv[j][r], t);
                acc[h][j] = t;
            }
        }
        wave_lds_sync();
    };

    // A ring of two tiles: the next tile's loads go out before the current
    // tile's math.  The loop handles tiles in pairs and has one exit, at the
    // bottom, and the next load is issued on every path (past the end it
    // re-reads the last tile), so the compiler's wait before the math covers
    // the current tile only.
    if (jb1 > jb0) {
        const int32_t n = jb1 - jb0;
        Raw R[2];
        load(jb0, id_of(jb0), R[0]);
        int32_t id_next = id_of(jb0 + 1);
        int32_t i = 0;
        for (; i + 2 <= n; i = uniform(i + 2)) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int32_t jb = jb0 + i + d;
                const int32_t id_after = id_of(jb + 2);
                load(jb + 1, id_next, R[(d + 1) % 2]);
                compute(R[d], jb);
                id_next = id_after;
            }
        }
        if (i < n)
            compute(R[0], jb0 + i); // the last tile of an odd count
        // no load into these registers is left in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }

    // combine lane partials: l over the 16 token quads, acc over the four
    // lanes of a dim
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] += shfl_xor(l[h], 4);
        l[h] += shfl_xor(l[h], 8);
        l[h] += shfl_xor(l[h], 16);
        l[h] += shfl_xor(l[h], 32);
#pragma unroll
        for (int j = 0; j < S::VD; ++j) {
            acc[h][j] += shfl_xor(acc[h][j], 16);
            acc[h][j] += shfl_xor(acc[h][j], 32);
        }
    }

    const bool writer = lane < 16;
    if (a.partition == 0) {
        TQ *o = static_cast<TQ *>(a.out) + ((size_t)it.b * a.num_q_heads + (size_t)it.g * G) * D;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            // l = 0: no token in the range (n = 0 or an empty window)
            const float inv = (l[h] == 0.f) ? 0.f : a.v_scale / l[h];
#pragma unroll
            for (int j = 0; j < S::VD; ++j) {
                float r = bad ? NAN : acc[h][j] * inv;
                if (writer)
                    o[h * D + 16 * j + vdim] = from_f32<QT>(r);
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (lane == 0) {
                float *ml = ws_ml(a, w, h);
                ml[0] = bad ? NAN : m[h];
                ml[1] = bad ? NAN : l[h];
            }
            float *accp = ws_acc(a, w, h, D);
#pragma unroll
            for (int j = 0; j < S::VD; ++j)
                if (writer)
                    accp[16 * j + vdim] = bad ? NAN : acc[h][j] * a.v_scale;
        }
    }
}

// Host-side launcher, instantiated per supported (q, kv, D, G).
template <int QT, int KT, int D, int G>
hipError_t launch_valu(const DecodeArgs &a, int32_t num_items, hipStream_t stream)
{
    const int grid = (num_items + 3) / 4;
    hipLaunchKernelGGL((decode_valu_kernel<QT, KT, D, G>), dim3(grid), dim3(256), 0, stream, a,
                       num_items);
    return hipGetLastError();
}

// Dispatch on the runtime shape; returns hipErrorInvalidValue if the shape has
// no instantiation.
template <int QT, int KT, int D>
hipError_t valu_by_group(const DecodeArgs &a, int32_t n, hipStream_t s)
{
    switch (a.group) {
    case 1: return launch_valu<QT, KT, D, 1>(a, n, s);
    case 2: return launch_valu<QT, KT, D, 2>(a, n, s);
    case 4: return launch_valu<QT, KT, D, 4>(a, n, s);
    case 8:
        if constexpr (D == 64)
            return launch_valu<QT, KT, D, 8>(a, n, s);
        else
            return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int QT, int KT>
hipError_t valu_by_dim(const DecodeArgs &a, int D, int32_t n, hipStream_t s)
{
    if (D == 64)
        return valu_by_group<QT, KT, 64>(a, n, s);
    if (D == 128)
        return valu_by_group<QT, KT, 128>(a, n, s);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_valu(const DecodeArgs &a, pa_dtype qt, pa_dtype kt, int D,
                              int32_t num_items, hipStream_t s)
{
    if (qt == PA_F32 && kt == PA_F32)
        return valu_by_dim<PA_F32, PA_F32>(a, D, num_items, s);
    if (qt == PA_F16 && kt == PA_F16)
        return valu_by_dim<PA_F16, PA_F16>(a, D, num_items, s);
    if (qt == PA_BF16 && kt == PA_BF16)
        return valu_by_dim<PA_BF16, PA_BF16>(a, D, num_items, s);
    if (qt == PA_BF16 && kt == PA_FP8_E4M3)
        return valu_by_dim<PA_BF16, PA_FP8_E4M3>(a, D, num_items, s);
    if (qt == PA_F16 && kt == PA_FP8_E4M3)
        return valu_by_dim<PA_F16, PA_FP8_E4M3>(a, D, num_items, s);
    return hipErrorInvalidValue;
}

bool valu_supports(pa_dtype qt, pa_dtype kt, int D, int G)
{
    const bool dt = (qt == kt && qt != PA_FP8_E4M3) ||
                    (kt == PA_FP8_E4M3 && (qt == PA_BF16 || qt == PA_F16));
    const bool g = G == 1 || G == 2 || G == 4 || (G == 8 && D == 64);
    return dt && (D == 64 || D == 128) && g;
}

} // namespace pa
