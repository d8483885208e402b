// Merge of partial softmax states: the second kernel of the partitioned
// decode.  The work items of a (sequence, KV head) left, per query head, a
// running max m_p (log2 units), a sum l_p and an unnormalised accumulator
// acc_p; the exact softmax over the whole sequence is
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// the same identity the online update inside a work item uses.
#include "device.hpp"
#include "work.hpp"

namespace pa {

// Combines the partial states of one output row (sequence b, query head
// h of group g) held in slots w0 .. w0 + nparts - 1:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// the same identity the online update inside a work item uses.  Parts are
// visited in index order, so the result does not depend on which wave merges.
// A NaN partial (a bad block-table entry) makes the row NaN.
template <int QT, int D>
__device__ __forceinline__ void merge_row(const DecodeArgs &a, int32_t b, int32_t g, int h,
                                          int64_t w0, int64_t nparts, int lane)
{
    using TQ = typename Store<QT>::T;
    constexpr int PER_LANE = D / kWave;
    TQ *o = static_cast<TQ *>(a.out) + ((size_t)b * a.num_q_heads + (size_t)g * a.group + h) * D;
    float M = -INFINITY;
    for (int64_t p = lane; p < nparts; p += kWave)
        M = fmaxf(M, ws_ml(a, w0 + p, h)[0]);
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1)
        M = fmaxf(M, shfl_xor(M, x));

    float L = 0.f;
    float acc[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
        acc[i] = 0.f;
    bool nan_seen = false;
    for (int64_t p = 0; p < nparts; ++p) {
        const float *ml = ws_ml(a, w0 + p, h);
        const float mp = ml[0];
        const float lp = ml[1];
        nan_seen |= (mp != mp);
        const float wgt = __builtin_amdgcn_exp2f(mp - M);
        L = fmaf(lp, wgt, L);
        const float *ap = ws_acc(a, w0 + p, h, D);
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            acc[i] = fmaf(ap[i * kWave + lane], wgt, acc[i]);
    }
    const float inv = nan_seen ? NAN : (L == 0.f ? 0.f : 1.f / L); // L = 0: empty window
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
        o[i * kWave + lane] = from_f32<QT>(acc[i] * inv);
}

// Combines the nparts partial states in slots w0 .. w0 + nparts - 1 of
// segment (b, g) into its G output rows, one wave for the whole segment:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// per query head, the identity the online update inside a work item uses,
// applied here one batch of parts at a time (in slot order: the result does
// not depend on which wave merges).  A part's G x D accumulators are
// contiguous ([h][d]); lane l owns outputs o = 256 s + 4 l + j (s < S = G D /
// 256, j < 4), so every load instruction reads 1 KiB of one part and no
// cross-lane reduction is needed.  A NaN partial (a bad block-table entry)
// makes its rows NaN.
template <int QT, int D, int S>
__device__ __forceinline__ void merge_segment_s(const DecodeArgs &a, int32_t b, int32_t g,
                                                int64_t w0, int64_t nparts, int lane)
{
    using TQ = typename Store<QT>::T;
    constexpr int CH = 16 / S; // parts per batch: 16 x 3 loads in flight per lane
    int hs[S];
    float M[S], L[S];
    f32x4 acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        hs[s] = (256 * s + 4 * lane) / D;
        M[s] = -INFINITY;
        L[s] = 0.f;
        acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool nan_seen = false;
    for (int64_t p0 = 0; p0 < nparts; p0 += CH) {
        float mp[CH][S], lp[CH][S];
        f32x4 ap[CH][S];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = p0 + c < nparts;
            const int64_t w = w0 + p0 + (in ? c : 0);
            const float *base = ws_acc(a, w, 0, D);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float *ml = ws_ml(a, w, hs[s]);
                const float *ac = base + 256 * s + 4 * lane;
                mp[c][s] = in ? ml[0] : -INFINITY;
                lp[c][s] = in ? ml[1] : 0.f;
                ap[c][s] = in ? f32x4{ac[0], ac[1], ac[2], ac[3]}
                              : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            float mb = M[s];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                nan_seen |= mp[c][s] != mp[c][s];
                mb = fmaxf(mb, mp[c][s]);
            }
            // every part holds a finite max (a real score, or the finite start
            // value when all its tokens lie before the window), so mb is finite
            const float alpha = __builtin_amdgcn_exp2f(M[s] - mb); // 0 on the first batch
            L[s] *= alpha;
            acc[s] *= alpha;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const float wgt = __builtin_amdgcn_exp2f(mp[c][s] - mb); // 0 past the end
                L[s] = fmaf(lp[c][s], wgt, L[s]);
                acc[s] += ap[c][s] * wgt;
            }
            M[s] = mb;
        }
    }
    TQ *o = static_cast<TQ *>(a.out) + ((size_t)b * a.num_q_heads + (size_t)g * a.group) * D;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float inv = nan_seen ? NAN : (L[s] == 0.f ? 0.f : 1.f / L[s]); // 0: empty window
        TQ *r = o + 256 * s + 4 * lane; // row hs[s], dims (256 s + 4 lane) % D ..
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = from_f32<QT>(acc[s][j] * inv);
    }
}

// G * D / 256 for the shapes merge_segment handles (0: not handled).
__host__ __device__ __forceinline__ int merge_runs(int G, int D)
{
    const int gd = G * D;
    if (gd % 256 != 0)
        return 0;
    const int s = gd / 256;
    return (s == 1 || s == 2 || s == 4 || s == 8) ? s : 0;
}

template <int QT, int D>
__device__ __forceinline__ void merge_segment(const DecodeArgs &a, int32_t b, int32_t g,
                                              int64_t w0, int64_t nparts, int lane)
{
    switch (merge_runs(a.group, D)) {
    case 1: merge_segment_s<QT, D, 1>(a, b, g, w0, nparts, lane); break;
    case 2: merge_segment_s<QT, D, 2>(a, b, g, w0, nparts, lane); break;
    case 4: merge_segment_s<QT, D, 4>(a, b, g, w0, nparts, lane); break;
    case 8: merge_segment_s<QT, D, 8>(a, b, g, w0, nparts, lane); break;
    default: break;
    }
}


template <int QT, int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a)
{
    using TQ = typename Store<QT>::T;
    constexpr int PER_LANE = D / kWave;
    const int lane = threadIdx.x;
    const int32_t row = blockIdx.x; // b * Hq + hq
    const int32_t b = row / a.num_q_heads;
    const int32_t hq = row % a.num_q_heads;
    const int32_t g = hq / a.group;
    const int h = hq % a.group;
    const int32_t n = a.seq_lens[b];

    const bool valid = len_ok(a, n);
    if (!valid || n == 0) {
        TQ *o = static_cast<TQ *>(a.out) + (size_t)row * D;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            o[i * kWave + lane] = from_f32<QT>(valid ? 0.f : NAN);
        return;
    }
    // slots w0 .. w0 + nparts - 1 hold this segment's partial states
    int64_t w0, nparts;
    if (a.partition == kPartitionBalanced) {
        const TileCounts tc = tile_counts(a, lane, b);
        const int64_t T = tc.total;
        const int32_t R = effective_runs(T, a.waves);
        const int64_t S0 = tc.before + (int64_t)g * tiles_of(n);
        const int64_t S1 = S0 + tiles_of(n);
        const int64_t i0 = run_of_tile(S0, T, R);
        const int64_t i1 = run_of_tile(S1 - 1, T, R);
        if (i0 == i1)
            return; // one run held the whole segment and wrote the row itself
        w0 = i0 + (int64_t)b * a.num_kv_heads + g;
        nparts = i1 - i0 + 1;
    } else {
        w0 = ((int64_t)b * a.num_kv_heads + g) * a.max_parts;
        nparts = (n + a.partition - 1) / a.partition;
    }
    merge_row<QT, D>(a, b, g, h, w0, nparts, lane);
}

// One wave per segment (sequence b, KV head g) for the shapes merge_segment
// handles; one workgroup per output row (merge_row) for the others.
template <int QT, int D>
__global__ __launch_bounds__(64) void merge_segment_kernel(DecodeArgs a)
{
    const int lane = threadIdx.x;
    const int32_t b = blockIdx.x / a.num_kv_heads;
    const int32_t g = blockIdx.x % a.num_kv_heads;
    const int32_t n = a.seq_lens[b];
    const bool valid = len_ok(a, n);
    if (!valid || n == 0) {
        using TQ = typename Store<QT>::T;
        TQ *o = static_cast<TQ *>(a.out) + ((size_t)b * a.num_q_heads + (size_t)g * a.group) * D;
        for (int32_t i = lane; i < a.group * D; i += kWave)
            o[i] = from_f32<QT>(valid ? 0.f : NAN);
        return;
    }
    int64_t w0, nparts;
    if (a.partition == kPartitionBalanced) {
        const TileCounts tc = tile_counts(a, lane, b);
        const int64_t T = tc.total;
        const int32_t R = effective_runs(T, a.waves);
        const int64_t S0 = tc.before + (int64_t)g * tiles_of(n);
        const int64_t i0 = run_of_tile(S0, T, R);
        const int64_t i1 = run_of_tile(S0 + tiles_of(n) - 1, T, R);
        if (i0 == i1)
            return; // one run held the whole segment and wrote the rows itself
        w0 = i0 + (int64_t)b * a.num_kv_heads + g;
        nparts = i1 - i0 + 1;
    } else {
        w0 = ((int64_t)b * a.num_kv_heads + g) * a.max_parts;
        nparts = (n + a.partition - 1) / a.partition;
    }
    merge_segment<QT, D>(a, b, g, w0, nparts, lane);
}

template <int QT, int D>
hipError_t merge_launch(const DecodeArgs &a, hipStream_t s)
{
    if (merge_runs(a.group, D) != 0)
        hipLaunchKernelGGL((merge_segment_kernel<QT, D>), dim3(a.num_seqs * a.num_kv_heads),
                           dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((merge_kernel<QT, D>), dim3(a.num_seqs * a.num_q_heads), dim3(64), 0,
                           s, a);
    return hipGetLastError();
}

template <int QT>
hipError_t merge_by_dim(const DecodeArgs &a, int D, hipStream_t s)
{
    if (D == 64)
        return merge_launch<QT, 64>(a, s);
    if (D == 128)
        return merge_launch<QT, 128>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeArgs &a, pa_dtype qt, int D, hipStream_t s)
{
    switch (qt) {
    case PA_F32: return merge_by_dim<PA_F32>(a, D, s);
    case PA_F16: return merge_by_dim<PA_F16>(a, D, s);
    case PA_BF16: return merge_by_dim<PA_BF16>(a, D, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace pa
