// Merge of partial softmax states: the second kernel of the partitioned
// decode.  Each work item of a (sequence, KV head) left, per query head, its
// running max m_p (log2 units), its sum l_p and its unnormalised accumulator
// acc_p; the exact softmax over the whole sequence is
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// the same identity the online update inside a work item uses.  Parts are
// visited in index order, so the result does not depend on scheduling.
#include "device.hpp"
#include "work.hpp"

namespace pa {

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
    TQ *o = static_cast<TQ *>(a.out) + (size_t)row * D;

    const bool valid = len_ok(a, n);
    if (!valid || n == 0) {
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            o[i * kWave + lane] = from_f32<QT>(valid ? 0.f : NAN);
        return;
    }
    // slots w0 .. w0 + nparts - 1 hold this segment's partial states
    int64_t w0, nparts;
    if (a.partition == kPartitionBalanced) {
        const int64_t T = tiles_before(a, lane, a.num_seqs);
        const int32_t R = effective_runs(T, a.waves);
        const int64_t S0 = tiles_before(a, lane, b) + (int64_t)g * blocks_of(n);
        const int64_t S1 = S0 + blocks_of(n);
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
        nan_seen |= (mp != mp);
        const float wgt = __builtin_amdgcn_exp2f(mp - M);
        L = fmaf(ml[1], wgt, L);
        const float *ap = ws_acc(a, w0 + p, h, D);
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            acc[i] = fmaf(ap[i * kWave + lane], wgt, acc[i]);
    }
    const float inv = nan_seen ? NAN : 1.f / L;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
        o[i * kWave + lane] = from_f32<QT>(acc[i] * inv);
}

template <int QT>
hipError_t merge_by_dim(const DecodeArgs &a, int D, hipStream_t s)
{
    const int grid = a.num_seqs * a.num_q_heads;
    if (D == 64)
        hipLaunchKernelGGL((merge_kernel<QT, 64>), dim3(grid), dim3(64), 0, s, a);
    else if (D == 128)
        hipLaunchKernelGGL((merge_kernel<QT, 128>), dim3(grid), dim3(64), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
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
