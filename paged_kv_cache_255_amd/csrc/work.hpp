// How a decode launch splits (sequence, KV head, token range) work across
// waves, and where partial softmax states go.  Shared by the decode kernels
// and the merge kernel.
#pragma once

#include "device.hpp"

namespace pa {

struct DecodeArgs {
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    void *out;
    float *ws;                 // partial states (partitioned modes)
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;             // num_q_heads / num_kv_heads
    int32_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
    int32_t partition;         // tokens per work item; 0 = whole sequence
    int32_t max_parts;         // work items per (sequence, KV head)
    float score_scale;         // scale * k_scale * log2(e): scores in log2 units
    float v_scale;
};

// Work item w covers (sequence b, KV head g, part p) with
//   w = (b * num_kv_heads + g) * max_parts + p
// and tokens [p * partition, min((p + 1) * partition, n)); partition 0 means
// the whole sequence (max_parts = 1).
struct Item {
    int32_t b, g, p, t0, t1, n;
    bool valid_len; // n within [0, max_seq_len] and the table row
};

__device__ __forceinline__ Item item_of(const DecodeArgs &a, int32_t w)
{
    Item it;
    it.p = w % a.max_parts;
    const int32_t s = w / a.max_parts;
    it.b = s / a.num_kv_heads;
    it.g = s % a.num_kv_heads;
    it.n = a.seq_lens[it.b];
    it.valid_len = it.n >= 0 && it.n <= a.max_seq_len &&
                   (int64_t)it.n <= (int64_t)a.max_blocks_per_seq * kBlockSize;
    if (a.partition == 0) {
        it.t0 = 0;
        it.t1 = it.n;
    } else {
        it.t0 = it.p * a.partition;
        it.t1 = min(it.t0 + a.partition, it.n);
    }
    return it;
}

// Partial state layout in the workspace, per work item and query head of its
// group: (m, l) pairs first, then the unnormalised accumulators.
//   ws[(w * G + h) * 2 + {0, 1}]                     m (log2 units), l
//   ws[2 * W * G + (w * G + h) * D + d]              acc
__device__ __forceinline__ float *ws_ml(const DecodeArgs &a, int64_t w, int h)
{
    return a.ws + (w * a.group + h) * 2;
}

__device__ __forceinline__ float *ws_acc(const DecodeArgs &a, int64_t w, int h, int D)
{
    const int64_t W = (int64_t)a.num_seqs * a.num_kv_heads * a.max_parts;
    return a.ws + 2 * W * a.group + (w * a.group + h) * (int64_t)D;
}

} // namespace pa
