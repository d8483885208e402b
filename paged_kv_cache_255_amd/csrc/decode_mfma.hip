// PagedAttention decode on the matrix cores (gfx950 MFMA).
//
// What it computes: dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation
// and How PagedAttention Fixes It", §1 (attention formula; one new query per
// sequence against the cached K/V) and §4 "The PagedAttention CUDA Kernel"
// (the query walks its block table and reads K/V from scattered physical
// blocks); §2 "Example 2" (query heads of a group share one KV head).
//
// One wave per work item (sequence, KV head, token range).  The G query heads
// of the KV head sit in the 16 columns of the MFMA tiles (G <= 16; unused
// columns carry q = 0 and are discarded), so each K and V tile is read from
// HBM once for the whole group.  Per 16-token block:
//   S^T[16 tokens][16 heads] = K_tile[16][D] * Q^T[D][16]     (D/32 MFMA 16x16x32)
//   online softmax on S^T, 4 tokens x 1 head per lane
//   O^T[D][16 heads] += V^T_tile[D][16] * P^T[16][16 heads]   (D/16 MFMA 16x16x16)
// The MFMA output layout of S^T (lane l: tokens 4*(l/16)+r, head l%16) is the
// B-operand layout of the second product, so P never leaves the registers.
// FP8 tiles are widened to the q type with the hardware converter (exact:
// every E4M3 value is a bf16 and an fp16 value).
#include "device.hpp"
#include "work.hpp"

namespace pa {

template <int QT> struct Mma;
template <> struct Mma<PA_BF16> {
    using A8 = bf16x8;
    using A4 = bf16x4;
    __device__ static f32x4 qk(A8 a, A8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 pv(A4 a, A4 b, f32x4 c)
    {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                          __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
    // two E4M3 (word `hi` of w) -> two bf16, packed
    __device__ static uint32_t fp8x2(uint32_t w, bool hi)
    {
        bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
        return __builtin_bit_cast(uint32_t, r);
    }
    __device__ static uint32_t pack2(float a, float b)
    {
        bf16x2 r = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, r);
    }
};
template <> struct Mma<PA_F16> {
    using A8 = f16x8;
    using A4 = f16x4;
    __device__ static f32x4 qk(A8 a, A8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 pv(A4 a, A4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
    __device__ static uint32_t fp8x2(uint32_t w, bool hi)
    {
        f16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
        return __builtin_bit_cast(uint32_t, r);
    }
    __device__ static uint32_t pack2(float a, float b)
    {
        f16x2 r = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, r);
    }
};

// Static shape of one kernel instance.
template <int QT, int KT, int D>
struct MfmaShape {
    static constexpr int KE = Store<KT>::bytes;              // 2 or 1
    static constexpr int ROW_BYTES = D * KE;                  // one K row
    static constexpr int CHUNKS = ROW_BYTES / 16;             // 16-byte chunks per K row
    static constexpr int CH_PER_LANE = CHUNKS / 4;            // chunks per lane per tile
    static constexpr int QK_MMAS = D / 32;
    static constexpr int PV_TILES = D / 16;
    static constexpr int V_ROW_BYTES = kBlockSize * KE;       // one V^T row (16 tokens)
    static constexpr int TILE_BYTES = kBlockSize * D * KE;
    static_assert(CHUNKS % 4 == 0, "row must split into 4 lane groups");
};

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a, int32_t num_items)
{
    using S = MfmaShape<QT, KT, D>;
    using M = Mma<QT>;
    using TQ = typename Store<QT>::T;
    using A8 = typename M::A8;
    using A4 = typename M::A4;

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t w = blockIdx.x * 4 + wid;
    if (w >= num_items)
        return;
    const Item it = item_of(a, w);
    if (it.valid_len && it.n > 0 && it.t0 >= it.t1)
        return;
    if (it.valid_len && it.n == 0 && it.p > 0)
        return;

    const int col = lane & 15; // MFMA column: query head within the group
    const int grp = lane >> 4; // lane group: 4 tokens of S^T, 4 dims of O^T
    const int G = a.group;

    // q of head `col` as the B operand of the D/32 QK products; chunk
    // mapping identical to the K operand below.
    A8 qop[S::QK_MMAS];
    {
        const TQ *qp = static_cast<const TQ *>(a.q) +
                       ((size_t)it.b * a.num_q_heads + (size_t)it.g * G + col) * D;
#pragma unroll
        for (int m = 0; m < S::QK_MMAS; ++m) {
            int d0;
            if constexpr (S::KE == 2)
                d0 = (grp + 4 * m) * 8;
            else
                d0 = (grp + 4 * (m / 2)) * 16 + 8 * (m % 2);
            A8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = col < G ? qp[d0 + i] : (TQ)0.f;
            qop[m] = v;
        }
    }

    f32x4 acc[S::PV_TILES];
#pragma unroll
    for (int t = 0; t < S::PV_TILES; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY; // running max of head `col` (log2 units)
    float l_run = 0.f;       // this lane's share of the running sum

    bool bad = !it.valid_len;
    const int32_t *table = a.block_tables + (size_t)it.b * a.max_blocks_per_seq;
    const char *kbase = static_cast<const char *>(a.k_cache);
    const char *vbase = static_cast<const char *>(a.v_cache);
    const int32_t jb0 = it.t0 / kBlockSize;
    const int32_t jb1 = bad ? jb0 : (it.t1 + kBlockSize - 1) / kBlockSize;
    const float sc = a.score_scale;

    for (int32_t jb = jb0; jb < jb1; ++jb) {
        const int32_t phys = __builtin_amdgcn_readfirstlane(table[jb]);
        if (phys < 0 || phys >= a.num_blocks) {
            bad = true;
            break;
        }
        const size_t tile = ((size_t)phys * a.num_kv_heads + it.g) * S::TILE_BYTES;
        const int32_t tok_base = jb * kBlockSize;
        const int32_t valid = it.t1 - tok_base; // tokens of this block in range (>= 1)

        // K: token `col`, chunks grp, grp+4, ... (64 contiguous bytes of every
        // row per load instruction)
        u32x4 kr[S::CH_PER_LANE];
#pragma unroll
        for (int j = 0; j < S::CH_PER_LANE; ++j)
            kr[j] = load16(kbase + tile + col * S::ROW_BYTES + (grp + 4 * j) * 16);
        // V^T: dims 16t + col, tokens 4*grp .. 4*grp+3 (512 contiguous bytes
        // per load instruction)
        uint32_t vr[S::PV_TILES][S::KE];
#pragma unroll
        for (int t = 0; t < S::PV_TILES; ++t) {
            const char *p = vbase + tile + (16 * t + col) * S::V_ROW_BYTES + grp * 4 * S::KE;
            if constexpr (S::KE == 2) {
                const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
                vr[t][0] = x.x;
                vr[t][1] = x.y;
            } else {
                vr[t][0] = *reinterpret_cast<const uint32_t *>(p);
            }
        }

        // S^T = K * Q^T
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < S::QK_MMAS; ++m) {
            A8 kop;
            if constexpr (S::KE == 2) {
                kop = __builtin_bit_cast(A8, kr[m]);
            } else {
                const u32x4 c = kr[m / 2];
                const uint32_t w0 = (m % 2) ? c.z : c.x;
                const uint32_t w1 = (m % 2) ? c.w : c.y;
                u32x4 e = {M::fp8x2(w0, false), M::fp8x2(w0, true), M::fp8x2(w1, false),
                           M::fp8x2(w1, true)};
                kop = __builtin_bit_cast(A8, e);
            }
            s = M::qk(kop, qop[m], s);
        }

        // online softmax for head `col`; this lane holds tokens 4*grp + r
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            x[r] = (4 * grp + r < valid) ? s[r] * sc : -INFINITY;
        float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        bm = fmaxf(bm, shfl_xor(bm, 16));
        bm = fmaxf(bm, shfl_xor(bm, 32));
        const float mn = fmaxf(m_run, bm);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            p[r] = __builtin_amdgcn_exp2f(x[r] - mn);
        l_run = fmaf(l_run, alpha, (p[0] + p[1]) + (p[2] + p[3]));
        const u32x2 pp = {M::pack2(p[0], p[1]), M::pack2(p[2], p[3])};
        const A4 pop = __builtin_bit_cast(A4, pp);

        // O^T += V^T * P^T
        const bool tail = valid < kBlockSize;
#pragma unroll
        for (int t = 0; t < S::PV_TILES; ++t) {
            u32x2 vw;
            if constexpr (S::KE == 2) {
                vw = u32x2{vr[t][0], vr[t][1]};
            } else {
                vw = u32x2{M::fp8x2(vr[t][0], false), M::fp8x2(vr[t][0], true)};
            }
            if (tail) {
                // slots past the end may hold anything (NaN included): zero them
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (4 * grp + r >= valid) {
                        const uint32_t keep = (r & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                        if (r < 2)
                            vw.x &= keep;
                        else
                            vw.y &= keep;
                    }
                }
            }
            acc[t] *= alpha;
            acc[t] = M::pv(__builtin_bit_cast(A4, vw), pop, acc[t]);
        }
    }

    // the lane groups hold disjoint tokens: sum their shares of l
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);

    if (col >= G)
        return;
    if (a.partition == 0) {
        TQ *o = static_cast<TQ *>(a.out) +
                ((size_t)it.b * a.num_q_heads + (size_t)it.g * G + col) * D;
        const float inv = bad ? NAN : (it.n > 0 ? a.v_scale / l_run : 0.f);
#pragma unroll
        for (int t = 0; t < S::PV_TILES; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[16 * t + 4 * grp + r] = from_f32<QT>(acc[t][r] * inv);
    } else {
        if (grp == 0) {
            float *ml = ws_ml(a, w, col);
            ml[0] = bad ? NAN : m_run;
            ml[1] = bad ? NAN : l_run;
        }
        float *accp = ws_acc(a, w, col, D);
        const float f = bad ? NAN : a.v_scale;
#pragma unroll
        for (int t = 0; t < S::PV_TILES; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                accp[16 * t + 4 * grp + r] = acc[t][r] * f;
    }
}

template <int QT, int KT, int D>
hipError_t launch_mfma(const DecodeArgs &a, int32_t num_items, hipStream_t stream)
{
    const int grid = (num_items + 3) / 4;
    hipLaunchKernelGGL((decode_mfma_kernel<QT, KT, D>), dim3(grid), dim3(256), 0, stream, a,
                       num_items);
    return hipGetLastError();
}

template <int QT, int KT>
hipError_t mfma_by_dim(const DecodeArgs &a, int D, int32_t n, hipStream_t s)
{
    if (D == 64)
        return launch_mfma<QT, KT, 64>(a, n, s);
    if (D == 128)
        return launch_mfma<QT, KT, 128>(a, n, s);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeArgs &a, pa_dtype qt, pa_dtype kt, int D,
                              int32_t num_items, hipStream_t s)
{
    if (qt == PA_BF16 && kt == PA_BF16)
        return mfma_by_dim<PA_BF16, PA_BF16>(a, D, num_items, s);
    if (qt == PA_F16 && kt == PA_F16)
        return mfma_by_dim<PA_F16, PA_F16>(a, D, num_items, s);
    if (qt == PA_BF16 && kt == PA_FP8_E4M3)
        return mfma_by_dim<PA_BF16, PA_FP8_E4M3>(a, D, num_items, s);
    if (qt == PA_F16 && kt == PA_FP8_E4M3)
        return mfma_by_dim<PA_F16, PA_FP8_E4M3>(a, D, num_items, s);
    return hipErrorInvalidValue;
}

bool mfma_supports(pa_dtype qt, pa_dtype kt, int D, int G)
{
    const bool dt = (qt == PA_BF16 || qt == PA_F16) && (kt == qt || kt == PA_FP8_E4M3);
    return dt && (D == 64 || D == 128) && G >= 1 && G <= 16;
}

} // namespace pa
