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
    const int32_t *seq_starts; // window starts, or null (every window starts at 0)
    const int32_t *seq_shared; // leading table entries shared within the batch
                               // (read with caching loads), or null
    void *out;
    float *ws;                 // partial states (partitioned modes)
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;             // num_q_heads / num_kv_heads
    int32_t num_blocks;
    int32_t tile_shift;        // log2(block_size / 16): a block is 1 << tile_shift tiles
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
    int32_t partition;         // tokens per work item; 0 = whole sequence; -1 = balanced
    int32_t max_parts;         // work items per (sequence, KV head) (fixed partitions)
    int32_t waves;             // W, the number of runs (balanced)
    int64_t num_slots;         // partial-state slots in the workspace
    float score_scale;         // scale * k_scale * log2(e): scores in log2 units
    float v_scale;
    // Appending decode: the step's new token of sequence b (k_new, v_new:
    // [num_seqs][Hkv][D] in the q dtype) goes to slot slots[b], written by
    // the wave whose range holds the sequence's last tile.
    int32_t append;
    const void *k_new;
    const void *v_new;
    const int32_t *slots;
    float k_inv, v_inv;        // FP8 cache: 1 / k_scale, 1 / v_scale
};

constexpr int32_t kPartitionBalanced = -1; // PA_PARTITION_BALANCED

// Starting value of a running max: below every score but finite, so that a
// tile whose tokens all lie before the window start (scores -inf) gives
// weights 2^(-inf - m) = 0 rather than NaN.  A real score replaces it at the
// first rescale, with the same bits as a start from -inf.
constexpr float kMaxStart = -3.0e38f;

__device__ __forceinline__ bool len_ok(const DecodeArgs &a, int32_t n)
{
    return n >= 0 && n <= a.max_seq_len &&
           (int64_t)n <= ((int64_t)a.max_blocks_per_seq << a.tile_shift) * kTile;
}

__device__ __forceinline__ int32_t tiles_of(int32_t n) { return (n + kTile - 1) / kTile; }

// Tiles the balanced split charges a segment for starting, on top of its own:
// a wave that moves on to a new (sequence, KV head) inside its run restarts
// its tile pipeline (the lengths, q and the block ids of the new segment, then
// the first tiles' loads).  Measured on MI355X (Llama-3-8B layer, 32
// sequences): with no charge, runs holding two segments ended 3.9 us after
// the others (a tile takes a wave about 1.2 us); whole decode steps took
// 58.1, 57.5, 57.0, 57.1, 57.3, 57.5 and 58.1 us on average (runs of three,
// two sweeps) with charges of 0, 3, 5, 7, 9, 12 and 16 tiles.  In the
// balanced order a segment is kSegmentCost virtual tiles, then its real
// tiles.
constexpr int32_t kSegmentCost = 5;

// Tiles a sequence contributes to the balanced split (its real tiles plus the
// start charge); an empty sequence or a length out of range contributes none
// (the merge kernel writes that row as 0 or NaN).
__device__ __forceinline__ int32_t split_tiles(const DecodeArgs &a, int32_t n)
{
    return (len_ok(a, n) && n > 0) ? tiles_of(n) + kSegmentCost : 0;
}

__device__ __forceinline__ int64_t wave_sum(int64_t v)
{
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1)
        v += __shfl_xor(v, x, kWave);
    return v;
}

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane)
{
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) {
        const int64_t o = __shfl_up(v, x, kWave);
        if (lane >= x)
            v += o;
    }
    return v;
}

// Inclusive prefix sum of a 32-bit value over the 64 lanes of a wave, with
// DPP moves (row shifts within each 16-lane row, then the row broadcasts of
// lanes 15 and 31): six VALU adds, no LDS-queue round trips.
__device__ __forceinline__ int32_t wave_incl_scan32(int32_t v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31
    return v;
}

// Lengths below this keep every per-wave tile sum of up to 64 sequences
// inside 32 bits (64 * 2^21 tiles), so the split can use wave_incl_scan32.
constexpr int32_t kScan32MaxLen = 1 << 25;

__device__ __forceinline__ int64_t readlane64(int64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The balanced split orders the segments head-major: (KV head g, sequence
// b) for g = 0 .. Hkv-1 and, within a head, b = 0 .. B-1.  Every head has
// the same Th tiles (the sequences' split_tiles summed: real tiles and start
// charges), so T = Hkv * Th and segment (g, b) starts at tile
// g * Th + (split_tiles of sequences [0, b)).

// Tiles of sequences [0, b) and of all sequences (one head's share, Th),
// from one pass over the lengths (each lane sums its own sequences; the two
// sums are wave reductions).
struct HeadTiles {
    int64_t before;   // tiles of sequences [0, b)
    int64_t per_head; // Th
};

__device__ __forceinline__ HeadTiles head_tiles(const DecodeArgs &a, int lane, int32_t b)
{
    int64_t before = 0, total = 0;
    for (int32_t c = 0; c < a.num_seqs; c += kWave) {
        const int32_t s = c + lane;
        const int64_t t = (s < a.num_seqs) ? split_tiles(a, a.seq_lens[s]) : 0;
        total += t;
        before += (s < b) ? t : 0;
    }
    return HeadTiles{wave_sum(before), wave_sum(total)};
}

struct SegPos {
    int32_t g;          // KV head
    int32_t b;          // sequence
    int32_t n;          // its length
    int64_t first_tile; // where the segment starts in the balanced order; its
                        // tile j is at first_tile + kSegmentCost + j
};

// The segment holding tile x (x < T = Hkv * Th): head x / Th, then the
// sequence holding tile x % Th of that head, found one 64-sequence chunk at
// a time with a wave scan and a ballot.
__device__ __forceinline__ SegPos locate_tile(const DecodeArgs &a, int lane, int64_t x,
                                              int64_t Th)
{
    const int32_t g = (int32_t)(x / Th);
    const int64_t y = x - (int64_t)g * Th;
    int64_t carry = 0;
    for (int32_t c = 0; c < a.num_seqs; c += kWave) {
        const int32_t b = c + lane;
        const int64_t tiles = (b < a.num_seqs) ? (int64_t)split_tiles(a, a.seq_lens[b]) : 0;
        const int64_t incl = wave_incl_scan(tiles, lane);
        const uint64_t hit = __ballot(b < a.num_seqs && carry + incl > y);
        if (hit) {
            const int k = __ffsll((unsigned long long)hit) - 1;
            SegPos p;
            p.g = g;
            p.b = c + k;
            p.n = uniform_load(a.seq_lens + p.b);
            p.first_tile = (int64_t)g * Th + carry + readlane64(incl - tiles, k);
            return p;
        }
        carry += readlane64(incl, kWave - 1);
    }
    return SegPos{g, a.num_seqs, 0, (int64_t)g * Th + carry};
}

// Runs the balanced split cuts T tiles into: the launch's W waves, but no
// more than T so that every run holds at least one tile (which may be a start
// charge only: such a run decodes nothing and leaves no partial state).
__device__ __forceinline__ int32_t effective_runs(int64_t T, int32_t W)
{
    return (int32_t)(T < (int64_t)W ? T : (int64_t)W);
}

// XCDs (accelerator complex dies) of an MI355X.  The hardware dispatcher
// hands a launch's workgroups to the XCDs round-robin, so workgroup w runs on
// XCD w mod 8.  That order is how the dispatcher behaves, not something HIP
// promises: the run placement below relies on it for speed only (which L2
// holds which tiles).  If the order differed, every run would still be done
// once by one wave, and the results would not change.
constexpr int32_t kXcds = 8;

// Run of wave v (0..3) of workgroup w among W waves.  Each XCD gets one
// eighth of the runs, in order: with the head-major order and 8 KV heads,
// the tiles of one head, so a prefix that the head's sequences share is read
// through one XCD's L2.  (Falls back to run 4 w + v when W is not a
// multiple of 32.)
__device__ __forceinline__ int32_t balanced_run(int32_t w, int32_t v, int32_t W)
{
    if (W % (4 * kXcds) != 0)
        return 4 * w + v;
    return (w % kXcds) * (W / kXcds) + (w / kXcds) * 4 + v;
}

// Where run i of the balanced split starts: Th, T, the number of runs, the
// run's tiles [x0, x1) and the segment holding x0.  Up to 64 sequences the
// tile count is one load per lane and one reduction; beyond, chunked.
struct RunStart {
    int64_t Th, T;
    int32_t runs;
    int64_t x0, x1;
    SegPos pos;
};

__device__ __forceinline__ RunStart run_start(const DecodeArgs &a, int lane, int32_t i,
                                              int32_t W)
{
    RunStart r;
    if (a.num_seqs <= kWave && a.max_seq_len < kScan32MaxLen) {
        // one length per lane: the scan gives Th and the segment together
        const bool in = lane < a.num_seqs;
        const int32_t n = in ? a.seq_lens[lane] : 0;
        const int32_t tiles = in ? split_tiles(a, n) : 0;
        const int32_t incl = wave_incl_scan32(tiles);
        r.Th = __builtin_amdgcn_readlane(incl, kWave - 1);
        r.T = r.Th * a.num_kv_heads;
        r.runs = effective_runs(r.T, W);
        if (i >= r.runs)
            return r;
        r.x0 = (int64_t)i * r.T / r.runs;
        r.x1 = (int64_t)(i + 1) * r.T / r.runs;
        const int32_t g = (int32_t)(r.x0 / r.Th);
        const int32_t y = (int32_t)(r.x0 - (int64_t)g * r.Th);
        const uint64_t hit = __ballot(in && incl > y);
        const int k = __ffsll((unsigned long long)hit) - 1; // y < Th: some lane hits
        r.pos.g = g;
        r.pos.b = k;
        r.pos.n = __builtin_amdgcn_readlane(n, k);
        r.pos.first_tile = (int64_t)g * r.Th + __builtin_amdgcn_readlane(incl - tiles, k);
        return r;
    }
    if (a.num_seqs <= kWave) {
        // one length per lane: the scan gives Th and the segment together
        const bool in = lane < a.num_seqs;
        const int32_t n = in ? a.seq_lens[lane] : 0;
        const int64_t tiles = in ? (int64_t)split_tiles(a, n) : 0;
        const int64_t incl = wave_incl_scan(tiles, lane);
        r.Th = readlane64(incl, kWave - 1);
        r.T = r.Th * a.num_kv_heads;
        r.runs = effective_runs(r.T, W);
        if (i >= r.runs)
            return r;
        r.x0 = (int64_t)i * r.T / r.runs;
        r.x1 = (int64_t)(i + 1) * r.T / r.runs;
        const int32_t g = (int32_t)(r.x0 / r.Th);
        const int64_t y = r.x0 - (int64_t)g * r.Th;
        const uint64_t hit = __ballot(in && incl > y);
        const int k = __ffsll((unsigned long long)hit) - 1; // y < Th: some lane hits
        r.pos.g = g;
        r.pos.b = k;
        r.pos.n = __builtin_amdgcn_readlane(n, k);
        r.pos.first_tile = (int64_t)g * r.Th + readlane64(incl - tiles, k);
        return r;
    }
    r.Th = head_tiles(a, lane, 0).per_head;
    r.T = r.Th * a.num_kv_heads;
    r.runs = effective_runs(r.T, W);
    if (i >= r.runs)
        return r;
    r.x0 = (int64_t)i * r.T / r.runs;
    r.x1 = (int64_t)(i + 1) * r.T / r.runs;
    r.pos = locate_tile(a, lane, r.x0, r.Th);
    return r;
}

// The segment after p that has tiles: the next sequence of the head with
// tiles, else the first such sequence of the next head.
__device__ __forceinline__ SegPos next_segment(const DecodeArgs &a, SegPos p)
{
    SegPos q;
    q.first_tile = p.first_tile + split_tiles(a, p.n);
    q.g = p.g;
    q.b = p.b + 1;
    for (;;) {
        while (q.b < a.num_seqs && split_tiles(a, uniform_load(a.seq_lens + q.b)) == 0)
            ++q.b;
        if (q.b < a.num_seqs || q.g + 1 >= a.num_kv_heads)
            break;
        ++q.g; // every head has the same sequences with tiles
        q.b = 0;
    }
    q.n = q.b < a.num_seqs ? uniform_load(a.seq_lens + q.b) : 0;
    return q;
}

// Partial-state slot of run i's piece of segment (g, b): i + g * B + b.  The
// runs touching one segment are consecutive, and a run's segments follow
// each other, so no two (run, segment) pairs share a slot.
__device__ __forceinline__ int64_t balanced_slot(const DecodeArgs &a, int64_t i, int32_t g,
                                                 int32_t b)
{
    return i + (int64_t)g * a.num_seqs + b;
}

// Run holding tile x when T tiles are cut into R runs [i*T/R, (i+1)*T/R)
// (R <= T, so runs are never empty and consecutive runs are adjacent).
__device__ __forceinline__ int64_t run_of_tile(int64_t x, int64_t T, int32_t R)
{
    return ((x + 1) * R - 1) / T;
}

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
    it.n = uniform_load(a.seq_lens + it.b);
    it.valid_len = len_ok(a, it.n);
    if (a.partition == 0) {
        it.t0 = 0;
        it.t1 = it.n;
    } else {
        it.t0 = it.p * a.partition;
        it.t1 = min(it.t0 + a.partition, it.n);
    }
    return it;
}

// Partial state layout in the workspace, per slot w (a work item, or in the
// balanced split a (run, segment) pair) and query head h of the group: (m, l)
// pairs first, then the unnormalised accumulators.  S = num_slots.
//   ws[(w * G + h) * 2 + {0, 1}]                     m (log2 units), l
//   ws[2 * S * G + (w * G + h) * D + d]              acc
__device__ __forceinline__ float *ws_ml(const DecodeArgs &a, int64_t w, int h)
{
    return a.ws + (w * a.group + h) * 2;
}

__device__ __forceinline__ float *ws_acc(const DecodeArgs &a, int64_t w, int h, int D)
{
    return a.ws + 2 * a.num_slots * a.group + (w * a.group + h) * (int64_t)D;
}

} // namespace pa
