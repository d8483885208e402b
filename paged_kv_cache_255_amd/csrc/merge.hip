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

// Merge state of the outputs one lane owns in a segment (sequence b, KV
// head g): a part's G x D accumulators are contiguous ([h][d]), and lane l
// owns outputs o = 256 s + 4 l + j (s < S = G D / 256, j < 4), so every load
// instruction reads 1 KiB of one part and no cross-lane reduction is needed.
// Per chunk s: the running max M and sum L of the lane's query head and four
// unnormalised accumulators.
template <int S>
struct MergeState {
    float M[S], L[S];
    f32x4 acc[S];
    bool nan_seen;

    __device__ __forceinline__ MergeState() : nan_seen(false)
    {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            M[s] = -INFINITY;
            L[s] = 0.f;
            acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
};

// Slots holding parts of a segment: w0 + p stride for p < n.
struct PartList {
    int64_t w0, n, stride;
};

// Folds parts [p_begin, p_end) of the list `first` followed by the list
// `then` (part p < first.n in slot first.w0 + p first.stride, part
// first.n + k in slot then.w0 + k then.stride) into st, CH = 16 / S parts
// per batch (16 x 3 loads in flight per lane), in part order, with the
// online rescale between batches:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// per query head, the identity the online update inside a work item uses.
template <int D, int S>
__device__ __forceinline__ void merge_fold(const DecodeArgs &a, const PartList &first,
                                           const PartList &then, int64_t p_begin,
                                           int64_t p_end, int lane, MergeState<S> &st)
{
    constexpr int CH = 16 / S;
    int hs[S];
#pragma unroll
    for (int s = 0; s < S; ++s)
        hs[s] = (256 * s + 4 * lane) / D;
    for (int64_t p0 = p_begin; p0 < p_end; p0 += CH) {
        float mp[CH][S], lp[CH][S];
        f32x4 ap[CH][S];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = p0 + c < p_end;
            const int64_t p = p0 + (in ? c : 0);
            const int64_t w = p < first.n ? first.w0 + p * first.stride
                                          : then.w0 + (p - first.n) * then.stride;
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
            float mb = st.M[s];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                st.nan_seen |= mp[c][s] != mp[c][s];
                mb = fmaxf(mb, mp[c][s]);
            }
            // every part holds a finite max (a real score, or the finite start
            // value when all its tokens lie before the window), so mb is finite
            const float alpha = __builtin_amdgcn_exp2f(st.M[s] - mb); // 0 on the first batch
            st.L[s] *= alpha;
            st.acc[s] *= alpha;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const float wgt = __builtin_amdgcn_exp2f(mp[c][s] - mb); // 0 past the end
                st.L[s] = fmaf(lp[c][s], wgt, st.L[s]);
                st.acc[s] += ap[c][s] * wgt;
            }
            st.M[s] = mb;
        }
    }
}

// Writes the G output rows of segment (b, g) from a finished state.  A NaN
// partial (a bad block-table entry) makes its rows NaN; L = 0 (every token
// before the window start) gives zeros.
template <int QT, int D, int S>
__device__ __forceinline__ void merge_store(const DecodeArgs &a, int32_t b, int32_t g,
                                            const MergeState<S> &st, int lane)
{
    using TQ = typename Store<QT>::T;
    TQ *o = static_cast<TQ *>(a.out) + ((size_t)b * a.num_q_heads + (size_t)g * a.group) * D;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float inv = st.nan_seen ? NAN : (st.L[s] == 0.f ? 0.f : 1.f / st.L[s]);
        TQ *r = o + 256 * s + 4 * lane; // row (256 s + 4 lane) / D
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = from_f32<QT>(st.acc[s][j] * inv);
    }
}

// Combines the nparts partial states in slots w0 .. w0 + nparts - 1 of
// segment (b, g) into its G output rows, one wave for the whole segment.
// Parts are visited in slot order, so the result does not depend on which
// wave merges.
template <int QT, int D, int S>
__device__ __forceinline__ void merge_segment_s(const DecodeArgs &a, int32_t b, int32_t g,
                                                int64_t w0, int64_t nparts, int lane)
{
    MergeState<S> st;
    merge_fold<D, S>(a, PartList{w0, nparts, 1}, PartList{0, 0, 1}, 0, nparts, lane, st);
    merge_store<QT, D, S>(a, b, g, st, lane);
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

// Slots w0 .. w0 + nparts - 1 that hold the partial states of segment
// (sequence b of length n, KV head g).  False when there is nothing to
// merge: in the balanced split, one run held the whole segment and wrote its
// rows itself.
// The balanced split's run bounds for segment (g, b), whose real tiles (nt
// of them) follow its start charge at g * Th + before: the runs that decode
// some of them.  False when one run holds them all.
__device__ __forceinline__ bool balanced_parts(const DecodeArgs &a, int32_t b, int32_t g,
                                               int64_t Th, int64_t before, int32_t nt,
                                               int64_t &w0, int64_t &nparts)
{
    const int64_t T = Th * a.num_kv_heads;
    const int32_t R = effective_runs(T, a.waves);
    const int64_t S0 = (int64_t)g * Th + before + kSegmentCost; // no prefix rows here
    const int64_t i0 = run_of_tile(S0, T, R);
    const int64_t i1 = run_of_tile(S0 + nt - 1, T, R);
    if (i0 == i1)
        return false;
    w0 = balanced_slot(a, i0, g, b);
    nparts = i1 - i0 + 1;
    return true;
}

// What the merge does with segment (g, b) of a balanced launch over at most
// 64 sequences of lengths below kScan32MaxLen: every length comes in with one
// load per lane, issued before anything else (the segment's own length, the
// tiles before it and the head's total all follow from it).
enum SegAction { kSegFillZero, kSegFillNan, kSegWritten, kSegMerge };

__device__ __forceinline__ SegAction balanced_segment_fast(const DecodeArgs &a, int lane,
                                                           int32_t b, int32_t g, int64_t &w0,
                                                           int64_t &nparts)
{
    const bool in = lane < a.num_seqs;
    const int32_t len = in ? a.seq_lens[lane] : 0;
    const int32_t n = __builtin_amdgcn_readlane(len, b);
    const int32_t tiles = in ? split_tiles(a, len, 0, kSegmentCost) : 0;
    const int32_t incl = wave_incl_scan32(tiles);
    if (!len_ok(a, n))
        return kSegFillNan;
    if (n == 0)
        return kSegFillZero;
    const int32_t Th = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int32_t before = __builtin_amdgcn_readlane(incl - tiles, b);
    return balanced_parts(a, b, g, Th, before, tiles_of(n), w0, nparts) ? kSegMerge
                                                                         : kSegWritten;
}

__device__ __forceinline__ bool segment_parts(const DecodeArgs &a, int lane, int32_t b,
                                              int32_t g, int32_t n, int64_t &w0, int64_t &nparts)
{
    if (a.partition == kPartitionBalanced) {
        // segment (g, b) starts at g * Th + (split_tiles of sequences [0, b))
        const HeadTiles ht = head_tiles(a, lane, b, PrefixHead{false, 0, 0, 0});
        return balanced_parts(a, b, g, ht.per_head, ht.before, tiles_of(n), w0, nparts);
    } else {
        w0 = ((int64_t)b * a.num_kv_heads + g) * a.max_parts;
        nparts = (n + a.partition - 1) / a.partition;
    }
    return true;
}

// The parts of segment (g, b) of a launch with prefix rows, as the decode
// recorded them (SegLists): its own pieces, then its row's.  Slots are
// clamped into the workspace, so an entry the decode did not write (a
// length that changed between the two phases) cannot send the merge outside
// it.  False when one run wrote the rows itself.
__device__ __forceinline__ bool prefix_lists(const DecodeArgs &a, const u32x4 &e, PartList &seq,
                                             PartList &row)
{
    const int64_t S = a.num_slots;
    const int64_t sw = min(max((int64_t)(int32_t)e.x, (int64_t)0), S - 1);
    const int64_t sn = min(max((int64_t)(int32_t)e.y, (int64_t)0), S - sw);
    const int64_t stride = prefix_row_seqs(a.group);
    const int64_t rw = min(max((int64_t)(int32_t)e.z, (int64_t)0), S - 1);
    const int64_t rn = min(max((int64_t)(int32_t)e.w, (int64_t)0), (S - 1 - rw) / stride + 1);
    seq = PartList{sw, sn, 1};
    row = PartList{rw, rn, stride};
    return sn > 0;
}

// Combines the segment's parts, its own pieces first, then its row's.
template <int QT, int D, int S>
__device__ __forceinline__ void merge_lists_s(const DecodeArgs &a, int32_t b, int32_t g,
                                              const PartList &seq, const PartList &row, int lane)
{
    MergeState<S> st;
    merge_fold<D, S>(a, seq, row, 0, seq.n + row.n, lane, st);
    merge_store<QT, D, S>(a, b, g, st, lane);
}

template <int QT, int D>
__device__ __forceinline__ void merge_lists(const DecodeArgs &a, int32_t b, int32_t g,
                                            const PartList &seq, const PartList &row, int lane)
{
    switch (merge_runs(a.group, D)) {
    case 1: merge_lists_s<QT, D, 1>(a, b, g, seq, row, lane); break;
    case 2: merge_lists_s<QT, D, 2>(a, b, g, seq, row, lane); break;
    case 4: merge_lists_s<QT, D, 4>(a, b, g, seq, row, lane); break;
    case 8: merge_lists_s<QT, D, 8>(a, b, g, seq, row, lane); break;
    default: break;
    }
}

// The G rows of a segment whose length is out of range (NaN) or zero (0).
template <int QT, int D>
__device__ __forceinline__ void merge_fill(const DecodeArgs &a, int32_t b, int32_t g, bool valid,
                                           int lane)
{
    using TQ = typename Store<QT>::T;
    TQ *o = static_cast<TQ *>(a.out) + ((size_t)b * a.num_q_heads + (size_t)g * a.group) * D;
    for (int32_t i = lane; i < a.group * D; i += kWave)
        o[i] = from_f32<QT>(valid ? 0.f : NAN);
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
    int64_t w0, nparts;
    if (segment_parts(a, lane, b, g, n, w0, nparts))
        merge_row<QT, D>(a, b, g, h, w0, nparts, lane);
}

// One wave per segment (sequence b, KV head g) for the shapes merge_segment
// handles; one workgroup per output row (merge_row) for the others.
// True when balanced_segment_fast applies to the launch.
__device__ __forceinline__ bool segment_fast_path(const DecodeArgs &a)
{
    return a.partition == kPartitionBalanced && !a.prefix && a.num_seqs <= kWave &&
           a.max_seq_len < kScan32MaxLen;
}

template <int QT, int D>
__global__ __launch_bounds__(64) void merge_segment_kernel(DecodeArgs a)
{
    const int lane = threadIdx.x;
    const int32_t b = blockIdx.x / a.num_kv_heads;
    const int32_t g = blockIdx.x % a.num_kv_heads;
    if (segment_fast_path(a)) {
        int64_t w0 = 0, nparts = 0;
        switch (balanced_segment_fast(a, lane, b, g, w0, nparts)) {
        case kSegFillNan: merge_fill<QT, D>(a, b, g, false, lane); return;
        case kSegFillZero: merge_fill<QT, D>(a, b, g, true, lane); return;
        case kSegWritten: return;
        default: merge_segment<QT, D>(a, b, g, w0, nparts, lane); return;
        }
    }
    const int32_t n = a.seq_lens[b];
    // with prefix rows, the decode's record of the segment's parts comes in
    // with the length
    const u32x4 e = a.prefix ? load16(seg_dir_entry(a, g, b)) : u32x4{0u, 0u, 0u, 0u};
    const bool valid = len_ok(a, n);
    if (!valid || n == 0) {
        merge_fill<QT, D>(a, b, g, valid, lane);
        return;
    }
    if (a.prefix) {
        PartList seq, row;
        if (prefix_lists(a, e, seq, row))
            merge_lists<QT, D>(a, b, g, seq, row, lane);
        return;
    }
    int64_t w0, nparts;
    if (segment_parts(a, lane, b, g, n, w0, nparts))
        merge_segment<QT, D>(a, b, g, w0, nparts, lane);
}

// Waves of the wide merge's workgroup: NW x S x 64 lanes x 24 bytes of LDS
// stays at 48 KiB.
__host__ __device__ constexpr int wide_merge_waves(int S) { return S >= 8 ? 4 : 8; }

// Segments with many parts (long sequences, few segments): one workgroup of
// NW waves per segment.  Wave w folds the contiguous parts
// [w nparts / NW, (w + 1) nparts / NW) like the one-wave merge; wave 0 then
// combines the NW states from LDS in wave order, with the same identity:
//   M = max_w M_w,  out = sum_w 2^(M_w - M) acc_w / sum_w 2^(M_w - M) L_w.
// The grouping is fixed, so the bits do not depend on timing.  A wave with
// no parts holds M = -inf and L = acc = 0, which weigh 0 (some wave has a
// part, and every part's max is finite).
template <int QT, int D, int S>
__global__ __launch_bounds__(64 * wide_merge_waves(S)) void merge_segment_wide_kernel(DecodeArgs a)
{
    constexpr int NW = wide_merge_waves(S);
    __shared__ float s_m[NW][S][kWave];
    __shared__ float s_l[NW][S][kWave];
    __shared__ f32x4 s_acc[NW][S][kWave];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t b = blockIdx.x / a.num_kv_heads;
    const int32_t g = blockIdx.x % a.num_kv_heads;
    int64_t w0 = 0, nparts = 0;
    PartList row{0, 0, 1};
    // b, g and the lengths are the same for every wave, so all waves take the
    // same branch and leave together
    if (segment_fast_path(a)) {
        const SegAction act = balanced_segment_fast(a, lane, b, g, w0, nparts);
        if (act == kSegFillNan || act == kSegFillZero) {
            if (wave == 0)
                merge_fill<QT, D>(a, b, g, act == kSegFillZero, lane);
            return;
        }
        if (act == kSegWritten)
            return;
    } else {
        const int32_t n = a.seq_lens[b];
        const u32x4 e = a.prefix ? load16(seg_dir_entry(a, g, b)) : u32x4{0u, 0u, 0u, 0u};
        const bool valid = len_ok(a, n);
        if (!valid || n == 0) {
            if (wave == 0)
                merge_fill<QT, D>(a, b, g, valid, lane);
            return;
        }
        if (a.prefix) {
            PartList seq;
            if (!prefix_lists(a, e, seq, row))
                return;
            w0 = seq.w0;
            nparts = seq.n;
        } else if (!segment_parts(a, lane, b, g, n, w0, nparts)) {
            return;
        }
    }
    // wave w folds its share of the segment's parts: its own pieces, then
    // its row's
    const int64_t total = nparts + row.n;
    MergeState<S> st;
    merge_fold<D, S>(a, PartList{w0, nparts, 1}, row, wave * total / NW,
                     (wave + 1) * total / NW, lane, st);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        s_m[wave][s][lane] = st.M[s];
        s_l[wave][s][lane] = st.nan_seen ? NAN : st.L[s];
        s_acc[wave][s][lane] = st.acc[s];
    }
    __syncthreads();
    if (wave != 0)
        return;
    MergeState<S> tot;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, s_m[w][s][lane]);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float l = s_l[w][s][lane];
            tot.nan_seen |= l != l;
            const float wgt = __builtin_amdgcn_exp2f(s_m[w][s][lane] - M);
            tot.L[s] = fmaf(l, wgt, tot.L[s]);
            tot.acc[s] += s_acc[w][s][lane] * wgt;
        }
        tot.M[s] = M;
    }
    merge_store<QT, D, S>(a, b, g, tot, lane);
}

// Parts a segment is expected to have: in the balanced split W runs over
// B * Hkv segments, each segment touching about W / (B * Hkv) + 1 of them;
// with fixed partitions at most max_parts.
__host__ __forceinline__ int64_t expected_parts(const DecodeArgs &a)
{
    const int64_t segs = (int64_t)a.num_seqs * a.num_kv_heads;
    if (a.partition == kPartitionBalanced)
        return (a.waves + segs - 1) / segs + 1;
    return a.max_parts;
}

template <int QT, int D>
hipError_t merge_launch(const DecodeArgs &a, hipStream_t s)
{
    const dim3 segs(a.num_seqs * a.num_kv_heads);
    const int S = merge_runs(a.group, D);
    // one wave folds 16 / S parts per batch of loads; beyond one batch a
    // segment gets a workgroup of waves
    if (S != 0 && expected_parts(a) > 16 / S) {
        switch (S) {
        case 1:
            hipLaunchKernelGGL((merge_segment_wide_kernel<QT, D, 1>), segs,
                               dim3(64 * wide_merge_waves(1)), 0, s, a);
            break;
        case 2:
            hipLaunchKernelGGL((merge_segment_wide_kernel<QT, D, 2>), segs,
                               dim3(64 * wide_merge_waves(2)), 0, s, a);
            break;
        case 4:
            hipLaunchKernelGGL((merge_segment_wide_kernel<QT, D, 4>), segs,
                               dim3(64 * wide_merge_waves(4)), 0, s, a);
            break;
        default:
            hipLaunchKernelGGL((merge_segment_wide_kernel<QT, D, 8>), segs,
                               dim3(64 * wide_merge_waves(8)), 0, s, a);
            break;
        }
    } else if (S != 0) {
        hipLaunchKernelGGL((merge_segment_kernel<QT, D>), segs, dim3(64), 0, s, a);
    } else {
        hipLaunchKernelGGL((merge_kernel<QT, D>), dim3(a.num_seqs * a.num_q_heads), dim3(64), 0,
                           s, a);
    }
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
