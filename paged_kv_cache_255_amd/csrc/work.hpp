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
    const int32_t *share;      // the batch's share plan (pa.h), or null
    int32_t prefix;            // balanced launch that may read the plan's groups once
                               // per KV head (the launch decides with prefix_layout)
    int64_t prefix_base;       // first partial-state slot of those reads
    int32_t *seg_dir;          // with prefix: per (KV head, sequence), the slots the
                               // merge folds (SegLists), written by the decode
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
    int32_t stage_bytes;       // balanced launch: LDS bytes per wave that hold a run's
                               // results until it ends (0: stored at once)
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
// two sweeps) with charges of 0, 3, 5, 7, 9, 12 and 16 tiles.  Per-wave
// clocks later put a piece's fixed cost at 3.6 (32 sequences) and 4.2 (256
// sequences sharing a prompt) tiles, and a charge of 4 ran both launches
// 1 - 1.5% faster than 5 (3 gave back most of it).  Once a run's results
// were held in LDS until it ends (launches with a share plan), the 256
// sequences ran about 1.5% faster with a charge of 5 or 6 than with 4, while
// 5 cost the 32-sequence launch (no plan) 1%; so in a launch with prefix rows
// (seq_cost) every segment is charged kSegmentCostShared, and in any other
// kSegmentCost (a plan that only marks shared blocks leaves the split, and so
// every bit, as without it).  In the balanced order a segment is that many
// virtual tiles, then its real tiles.
constexpr int32_t kSegmentCost = 4;
constexpr int32_t kSegmentCostShared = 6;

// XCDs (accelerator complex dies) of an MI355X.  The hardware dispatcher
// hands a launch's workgroups to the XCDs round-robin, so workgroup w runs on
// XCD w mod 8.  That order is how the dispatcher behaves, not something HIP
// promises: the run placement below relies on it for speed only (which L2
// holds which tiles).  If the order differed, every run would still be done
// once by one wave, and the results would not change.
constexpr int32_t kXcds = 8;

// ---- the share plan (layout in pa.h) ---------------------------------------
__device__ __forceinline__ const int32_t *plan_shared(const DecodeArgs &a) { return a.share + 2; }
__device__ __forceinline__ const int32_t *plan_group(const DecodeArgs &a)
{
    return a.share + 2 + a.num_seqs;
}
__device__ __forceinline__ const int32_t *plan_rank(const DecodeArgs &a)
{
    return a.share + 2 + 2 * (size_t)a.num_seqs;
}
__device__ __forceinline__ const int32_t *plan_own(const DecodeArgs &a)
{
    return a.share + 2 + 3 * (size_t)a.num_seqs;
}
__device__ __forceinline__ const int32_t *plan_gcount(const DecodeArgs &a)
{
    return a.share + 2 + 4 * (size_t)a.num_seqs;
}
__device__ __forceinline__ const int32_t *plan_gblocks(const DecodeArgs &a)
{
    return a.share + 2 + 5 * (size_t)a.num_seqs;
}
__device__ __forceinline__ const int32_t *plan_members(const DecodeArgs &a)
{
    return a.share + 2 + 6 * (size_t)a.num_seqs;
}
__device__ __forceinline__ const int32_t *plan_gfirst(const DecodeArgs &a)
{
    return a.share + 2 + 7 * (size_t)a.num_seqs;
}

// Column groups a prefix row keeps (each 16 MFMA columns: 16 / G sequences
// times G query heads), and the sequences of one prefix row.
constexpr int32_t kPrefixColGroups = 4;
__host__ __device__ __forceinline__ int32_t prefix_row_seqs(int32_t G)
{
    return kPrefixColGroups * (16 / G);
}

// What a tile of a prefix row costs in the balanced split, as the fraction
// kRowUnitNum / kRowUnitDen of a sequence tile (one unit).  A row's tiles
// come mostly from L2 (the head's other rows read the same blocks) and feed
// kPrefixColGroups MFMA column groups.  Measured on MI355X (Llama-3-8B layer,
// 256 sequences on a 2048-token prompt, per-wave clocks): 0.78 us per row
// tile against 1.14 us per sequence tile.
constexpr int32_t kRowUnitNum = 11;
constexpr int32_t kRowUnitDen = 16;

// Units a row of nt tiles takes after its start charge: its tile j starts at
// unit floor(j num / den).
__device__ __forceinline__ int32_t row_body(int32_t nt)
{
    return nt > 0 ? (int32_t)((int64_t)(nt - 1) * kRowUnitNum / kRowUnitDen) + 1 : 0;
}

// The first tile of a row that starts at unit u or later (u >= 0).
__device__ __forceinline__ int32_t row_tile_at(int64_t u)
{
    return (int32_t)((u * kRowUnitDen + kRowUnitNum - 1) / kRowUnitNum);
}

// Units a sequence of n tokens contributes to the balanced split: its tiles
// past the own_t its prefix row reads, plus the start charge; none when that
// leaves nothing, or for a length out of range (the merge kernel writes that
// row as 0 or NaN, or from its prefix row's state alone).
__device__ __forceinline__ int32_t split_tiles(const DecodeArgs &a, int32_t n, int32_t own_t,
                                              int32_t cost)
{
    const int32_t t = tiles_of(n) - own_t;
    return (len_ok(a, n) && t > 0) ? t + cost : 0;
}

// The sum over the wave's lanes, returned as a wave-uniform value (through
// readfirstlane, so the compiler keeps what depends on it, such as the
// run's bounds and its walk over segments, in scalar registers and uniform
// branches).
__device__ __forceinline__ int64_t wave_sum(int64_t v)
{
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1)
        v += __shfl_xor(v, x, kWave);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)((hi << 32) | lo);
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

// ---- prefix rows of a share plan -------------------------------------------
// With a plan, every group of sequences that map the same leading blocks
// (gblocks of them, the plan's groups) is cut into rows of
// prefix_row_seqs(G) members in rank order, ceil(gcount / SPR) rows per group,
// and every KV head gets the same rows.  A row's tiles are those leading
// blocks, read once for all its members; the members' own segments then
// cover only their tiles past them.  Groups with no blocks get no rows.
struct PrefixHead {
    bool on;
    int32_t ng;    // groups of the plan
    int32_t rows;  // rows per KV head
    int64_t units; // the rows' units per head, start charges included
};

// The start charge of a sequence segment: kSegmentCostShared in a launch with
// prefix rows (a row always pays it), else kSegmentCost.
__device__ __forceinline__ int32_t seq_cost(const PrefixHead &P)
{
    return P.on ? kSegmentCostShared : kSegmentCost;
}

// Group gi's members, clamped into the batch, and its tiles, clamped into a
// table row.
__device__ __forceinline__ int32_t group_count(const DecodeArgs &a, int32_t gi)
{
    return min(max(plan_gcount(a)[gi], 0), a.num_seqs);
}
__device__ __forceinline__ int32_t group_tiles(const DecodeArgs &a, int32_t gi)
{
    return min(max(plan_gblocks(a)[gi], 0), a.max_blocks_per_seq) << a.tile_shift;
}
__device__ __forceinline__ int32_t group_rows(const DecodeArgs &a, int32_t cnt, int32_t nt)
{
    const int32_t spr = prefix_row_seqs(a.group);
    return nt > 0 ? (cnt + spr - 1) / spr : 0;
}
__device__ __forceinline__ int64_t row_units(int32_t nt)
{
    return nt > 0 ? kSegmentCostShared + row_body(nt) : 0;
}

// The launch's rows, the same in every wave of the decode and of the merge.
// Off without a plan, or when the plan holds more groups or rows than B / 2
// (a plan from pa_export_share_plan never does: every group has two members
// or more).
__device__ __forceinline__ PrefixHead prefix_head(const DecodeArgs &a, int lane)
{
    PrefixHead P{false, 0, 0, 0};
    // rows take whole workgroups of each XCD's runs: 4 or more of W / 8
    if (!a.prefix || a.waves % (4 * kXcds) != 0 || a.waves / kXcds < 8)
        return P;
    const int32_t ng = uniform(a.share[1]);
    if (ng <= 0 || ng > a.num_seqs / 2)
        return P;
    int64_t rows = 0, units = 0;
    for (int32_t c = 0; c < ng; c += kWave) {
        const int32_t gi = c + lane;
        int64_t r = 0, u = 0;
        if (gi < ng) {
            const int32_t nt = group_tiles(a, gi);
            r = group_rows(a, group_count(a, gi), nt);
            u = r * row_units(nt);
        }
        rows += wave_sum(r);
        units += wave_sum(u);
    }
    if (rows == 0 || rows > a.num_seqs / 2)
        return P;
    P.on = true;
    P.ng = ng;
    P.rows = (int32_t)rows;
    P.units = units;
    return P;
}

// Leading tiles of sequence b (of n tokens) that its prefix row reads: none
// without rows, for a sequence in no group, or when they would reach the
// sequence's last token (that tile stays with the sequence, so the step's
// token is appended and every tile the row reads is full).
__device__ __forceinline__ int32_t own_tiles(const DecodeArgs &a, const PrefixHead &P, int32_t b,
                                             int32_t n)
{
    if (!P.on)
        return 0;
    const int32_t t = min(max(plan_own(a)[b], 0), a.max_blocks_per_seq) << a.tile_shift;
    return (int64_t)t * kTile < (int64_t)n ? t : 0;
}

// The same for a wave-uniform b, with a scalar load (see uniform_load).
__device__ __forceinline__ int32_t own_tiles_uniform(const DecodeArgs &a, const PrefixHead &P,
                                                     int32_t b, int32_t n)
{
    if (!P.on)
        return 0;
    const int32_t t = min(max(uniform_load(plan_own(a) + b), 0), a.max_blocks_per_seq)
                      << a.tile_shift;
    return (int64_t)t * kTile < (int64_t)n ? t : 0;
}

// A row of a head: the plan's group gi, rows chunk of it (members
// [chunk SPR, (chunk + 1) SPR) of its rank order), its tiles, its index
// among the head's rows and the units of the head's rows before it.
struct RowPos {
    int32_t gi, chunk, nt, row;
    int64_t before;
};

// The row holding unit y (< P.units) of a head's rows (by_unit), or row
// number y (!by_unit): a scan over the groups, 64 at a time.
__device__ __forceinline__ RowPos locate_row(const DecodeArgs &a, int lane, int64_t y,
                                             bool by_unit, const PrefixHead &P)
{
    int64_t rows_c = 0, units_c = 0;
    for (int32_t c = 0; c < P.ng; c += kWave) {
        const int32_t gi = c + lane;
        int64_t r = 0, u = 0;
        int32_t nt = 0;
        if (gi < P.ng) {
            nt = group_tiles(a, gi);
            r = group_rows(a, group_count(a, gi), nt);
            u = row_units(nt);
        }
        const int64_t ri = wave_incl_scan(r, lane), ui = wave_incl_scan(r * u, lane);
        const uint64_t hit = __ballot(gi < P.ng && (by_unit ? units_c + ui : rows_c + ri) > y);
        if (hit) {
            const int k = __ffsll((unsigned long long)hit) - 1;
            RowPos q;
            q.gi = c + k;
            q.nt = __builtin_amdgcn_readlane(nt, k);
            const int64_t u_k = readlane64(u, k);
            const int64_t rows_b = rows_c + readlane64(ri - r, k);
            const int64_t units_b = units_c + readlane64(ui - r * u, k);
            q.chunk = (int32_t)(by_unit ? (y - units_b) / u_k : y - rows_b);
            q.row = (int32_t)rows_b + q.chunk;
            q.before = units_b + (int64_t)q.chunk * u_k;
            return q;
        }
        rows_c += readlane64(ri, kWave - 1);
        units_c += readlane64(ui, kWave - 1);
    }
    return RowPos{0, 0, 0, P.rows, P.units}; // not reached for y inside the rows
}

// Row `chunk` of group gi: its index among the head's rows and the units
// before it.
__device__ __forceinline__ RowPos row_of_group(const DecodeArgs &a, int lane, int32_t gi,
                                               int32_t chunk, const PrefixHead &P)
{
    int64_t rows_c = 0, units_c = 0;
    for (int32_t c = 0; c < P.ng; c += kWave) {
        const int32_t x = c + lane;
        int64_t r = 0, u = 0;
        if (x < P.ng) {
            const int32_t nt = group_tiles(a, x);
            r = group_rows(a, group_count(a, x), nt);
            u = row_units(nt);
        }
        const int64_t ri = wave_incl_scan(r, lane), ui = wave_incl_scan(r * u, lane);
        if (gi < c + kWave) {
            const int k = gi - c;
            RowPos q;
            q.gi = gi;
            q.chunk = chunk;
            q.nt = group_tiles(a, gi);
            q.row = (int32_t)(rows_c + readlane64(ri - r, k)) + chunk;
            q.before = units_c + readlane64(ui - r * u, k) + (int64_t)chunk * readlane64(u, k);
            return q;
        }
        rows_c += readlane64(ri, kWave - 1);
        units_c += readlane64(ui, kWave - 1);
    }
    return RowPos{gi, chunk, 0, P.rows, P.units}; // gi >= P.ng: not called so
}

// ---- the balanced order ------------------------------------------------------
// The balanced split orders the sequence segments head-major: (KV head g,
// sequence b) for g = 0 .. Hkv-1 and, within a head, b = 0 .. B-1.  Every
// head has the same Th units (the sequences' split_tiles summed: tiles and
// start charges), so T = Hkv * Th and segment (g, b) starts at unit
// g * Th + (split_tiles of sequences [0, b)).  A launch with prefix rows cuts
// the rows (head-major too: head g's rows fill units [g P.units,
// (g + 1) P.units)) in a second balanced split over runs of their own.

// Units of sequences [0, b) (`before`) and of all sequences (one head's
// share, Th), from one pass over the lengths (each lane sums its own
// sequences; the two sums are wave reductions).
struct HeadTiles {
    int64_t before;   // units of sequences [0, b)
    int64_t per_head; // Th
};

__device__ __forceinline__ HeadTiles head_tiles(const DecodeArgs &a, int lane, int32_t b,
                                                const PrefixHead &P)
{
    int64_t before = 0, total = 0;
    for (int32_t c = 0; c < a.num_seqs; c += kWave) {
        const int32_t s = c + lane;
        int64_t t = 0;
        if (s < a.num_seqs) {
            const int32_t n = a.seq_lens[s];
            t = split_tiles(a, n, own_tiles(a, P, s, n), seq_cost(P));
        }
        total += t;
        before += (s < b) ? t : 0;
    }
    return HeadTiles{wave_sum(before), wave_sum(total)};
}

// A segment of a balanced split: a sequence (row < 0) or a prefix row.
struct SegPos {
    int32_t g;          // KV head
    int32_t b;          // sequence (B past the last one)
    int32_t n;          // its length; for a row, the row's tiles
    int32_t own;        // the sequence's leading tiles its prefix row reads
    int32_t row;        // -1, or the row's index among the head's rows
    int32_t gi, chunk;  // a row's group and chunk
    int64_t first_tile; // where the segment starts in its split; its first
                        // tile (a sequence's tile own, a row's tile 0) is at
                        // first_tile + its start charge
};

__device__ __forceinline__ SegPos seq_segment(int32_t g, int32_t b, int32_t n, int32_t own,
                                              int64_t first)
{
    return SegPos{g, b, n, own, -1, 0, 0, first};
}

__device__ __forceinline__ SegPos row_segment(int32_t g, const RowPos &r, int64_t head0)
{
    return SegPos{g, 0, r.nt, 0, r.row, r.gi, r.chunk, head0 + r.before};
}

// The sequence segment holding unit x (x < T = Hkv * Th): head x / Th, then
// the sequence holding unit x % Th of that head, found one 64-sequence chunk
// at a time with a wave scan and a ballot.
__device__ __forceinline__ SegPos locate_tile(const DecodeArgs &a, int lane, int64_t x,
                                              int64_t Th, const PrefixHead &P)
{
    const int32_t g = (int32_t)(x / Th);
    const int64_t y = x - (int64_t)g * Th;
    int64_t carry = 0;
    for (int32_t c = 0; c < a.num_seqs; c += kWave) {
        const int32_t b = c + lane;
        int32_t n = 0, own = 0;
        int64_t tiles = 0;
        if (b < a.num_seqs) {
            n = a.seq_lens[b];
            own = own_tiles(a, P, b, n);
            tiles = split_tiles(a, n, own, seq_cost(P));
        }
        const int64_t incl = wave_incl_scan(tiles, lane);
        const uint64_t hit = __ballot(b < a.num_seqs && carry + incl > y);
        if (hit) {
            const int k = __ffsll((unsigned long long)hit) - 1;
            return seq_segment(g, c + k, __builtin_amdgcn_readlane(n, k),
                               __builtin_amdgcn_readlane(own, k),
                               (int64_t)g * Th + carry + readlane64(incl - tiles, k));
        }
        carry += readlane64(incl, kWave - 1);
    }
    return seq_segment(g, a.num_seqs, 0, 0, (int64_t)g * Th + carry);
}

// Runs the balanced split cuts T tiles into: the launch's W waves, but no
// more than T so that every run holds at least one tile (which may be a start
// charge only: such a run decodes nothing and leaves no partial state).
__device__ __forceinline__ int32_t effective_runs(int64_t T, int32_t W)
{
    return (int32_t)(T < (int64_t)W ? T : (int64_t)W);
}

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

// Where run i of a balanced split starts: Th, T, the number of runs, the
// run's units [x0, x1) and the segment holding x0.
struct RunStart {
    int64_t Th, T;
    int32_t runs;
    int64_t x0, x1;
    SegPos pos;
};

// Run i of W over the sequence segments.  Up to 64 sequences the unit count
// is one load per lane (two with prefix rows) and one reduction; beyond,
// chunked.
__device__ __forceinline__ RunStart run_start(const DecodeArgs &a, int lane, int32_t i,
                                              int32_t W, const PrefixHead &P)
{
    RunStart r;
    if (a.num_seqs <= kWave && a.max_seq_len < kScan32MaxLen) {
        // one length per lane: the scan gives Th and the segment together
        const bool in = lane < a.num_seqs;
        const int32_t n = in ? a.seq_lens[lane] : 0;
        const int32_t own = in ? own_tiles(a, P, lane, n) : 0;
        const int32_t tiles = in ? split_tiles(a, n, own, seq_cost(P)) : 0;
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
        r.pos = seq_segment(g, k, __builtin_amdgcn_readlane(n, k),
                            __builtin_amdgcn_readlane(own, k),
                            (int64_t)g * r.Th + __builtin_amdgcn_readlane(incl - tiles, k));
        return r;
    }
    if (a.num_seqs <= kWave) {
        // one length per lane: the scan gives Th and the segment together
        const bool in = lane < a.num_seqs;
        const int32_t n = in ? a.seq_lens[lane] : 0;
        const int32_t own = in ? own_tiles(a, P, lane, n) : 0;
        const int64_t tiles = in ? (int64_t)split_tiles(a, n, own, seq_cost(P)) : 0;
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
        r.pos = seq_segment(g, k, __builtin_amdgcn_readlane(n, k),
                            __builtin_amdgcn_readlane(own, k),
                            (int64_t)g * r.Th + readlane64(incl - tiles, k));
        return r;
    }
    r.Th = head_tiles(a, lane, 0, P).per_head;
    r.T = r.Th * a.num_kv_heads;
    r.runs = effective_runs(r.T, W);
    if (i >= r.runs)
        return r;
    r.x0 = (int64_t)i * r.T / r.runs;
    r.x1 = (int64_t)(i + 1) * r.T / r.runs;
    r.pos = locate_tile(a, lane, r.x0, r.Th, P);
    return r;
}

// The sequence segment after p that has tiles: the next sequence of the
// head with tiles, else the first such sequence of the next head.
// (b and g pass through uniform() so that the compiler keeps the walk in
// scalar registers: as a divergent loop it would wait for the wave's
// outstanding vector stores at its head.)
__device__ __forceinline__ SegPos next_segment(const DecodeArgs &a, const SegPos &p,
                                               const PrefixHead &P)
{
    const int64_t first = p.first_tile + split_tiles(a, p.n, p.own, seq_cost(P));
    int32_t g = uniform(p.g), b = uniform(p.b + 1);
    for (;;) {
        while (b < a.num_seqs) {
            const int32_t n = uniform_load(a.seq_lens + b);
            const int32_t own = own_tiles_uniform(a, P, b, n);
            if (split_tiles(a, n, own, seq_cost(P)) > 0)
                return seq_segment(g, b, n, own, first);
            b = uniform(b + 1);
        }
        if (g + 1 >= a.num_kv_heads)
            return seq_segment(g, b, 0, 0, first);
        g = uniform(g + 1); // every head has the same sequences with tiles
        b = 0;
    }
}

// ---- one round of loads for a launch with prefix rows -----------------------
// A launch with a plan splits on every sequence's length and shared tiles and
// on every group's size; read in loops, those take a round trip per 64
// entries and per lookup.  For up to kRegChunks x 64 sequences and 64
// groups, LaunchRegs loads them all in one round, one entry per lane and
// chunk, and answers the split's lookups from registers (the same answers as
// head_tiles, locate_tile, prefix_head, locate_row and row_of_group).
constexpr int32_t kRegChunks = 4;

struct LaunchRegs {
    bool ok; // the batch and the plan fit (else use the loops)
    PrefixHead P;
    int32_t n[kRegChunks], own[kRegChunks], units[kRegChunks], incl[kRegChunks];
    int32_t carry[kRegChunks]; // units of the chunks before (wave-uniform)
    int32_t Th;                // units of all sequences (wave-uniform)
    int32_t g_nt, g_rows, g_unit; // group `lane`: tiles, rows, units a row
    int32_t g_count;              // group `lane`: members (as group_count)
    int32_t g_rows_incl;          // rows of groups 0 .. lane
    int64_t g_units_incl;         // units of groups 0 .. lane

    // units of sequences [0, b)
    __device__ __forceinline__ int64_t before(int32_t b) const
    {
        int64_t v = 0;
#pragma unroll
        for (int c = 0; c < kRegChunks; ++c)
            if (b >= c * kWave && b < (c + 1) * kWave) {
                const int k = b - c * kWave;
                v = carry[c] + (k > 0 ? __builtin_amdgcn_readlane(incl[c], k - 1) : 0);
            }
        return uniform((int32_t)v);
    }

    // the sequence segment holding unit x of the sequences' split
    __device__ __forceinline__ SegPos locate_seq(int64_t x) const
    {
        const int32_t g = (int32_t)(x / Th);
        const int32_t y = (int32_t)(x - (int64_t)g * Th);
        SegPos p{g, 0, 0, 0, -1, 0, 0, 0};
        bool found = false;
#pragma unroll
        for (int c = 0; c < kRegChunks; ++c) {
            const uint64_t hit = __ballot(carry[c] + incl[c] > y && units[c] > 0);
            if (!found && hit) {
                const int k = __ffsll((unsigned long long)hit) - 1;
                p = SegPos{g, c * kWave + k, __builtin_amdgcn_readlane(n[c], k),
                           __builtin_amdgcn_readlane(own[c], k), -1, 0, 0,
                           (int64_t)g * Th + carry[c] +
                               __builtin_amdgcn_readlane(incl[c] - units[c], k)};
                found = true;
            }
        }
        return p; // y < Th: some chunk hits
    }

    // the row holding unit y of a head's rows (by_unit), or row number y
    __device__ __forceinline__ RowPos locate_row(int64_t y, bool by_unit) const
    {
        const uint64_t hit = __ballot(g_rows > 0 &&
                                      (by_unit ? g_units_incl > y : (int64_t)g_rows_incl > y));
        const int k = __ffsll((unsigned long long)hit) - 1; // y inside the rows: some group hits
        const int32_t unit = __builtin_amdgcn_readlane(g_unit, k);
        const int32_t rows_b = __builtin_amdgcn_readlane(g_rows_incl - g_rows, k);
        const int64_t units_b = readlane64(g_units_incl - (int64_t)g_rows * g_unit, k);
        RowPos q;
        q.gi = k;
        q.nt = __builtin_amdgcn_readlane(g_nt, k);
        q.chunk = (int32_t)(by_unit ? (y - units_b) / unit : y - rows_b);
        q.row = rows_b + q.chunk;
        q.before = units_b + (int64_t)q.chunk * unit;
        return q;
    }

    // row `chunk` of group gi (gi < P.ng)
    __device__ __forceinline__ RowPos row_of_group(int32_t gi, int32_t chunk) const
    {
        RowPos q;
        q.gi = gi;
        q.chunk = chunk;
        q.nt = __builtin_amdgcn_readlane(g_nt, gi);
        q.row = __builtin_amdgcn_readlane(g_rows_incl - g_rows, gi) + chunk;
        q.before = readlane64(g_units_incl - (int64_t)g_rows * g_unit, gi) +
                   (int64_t)chunk * __builtin_amdgcn_readlane(g_unit, gi);
        return q;
    }
};

__device__ __forceinline__ LaunchRegs launch_regs(const DecodeArgs &a, int lane)
{
    LaunchRegs R;
    R.P = PrefixHead{false, 0, 0, 0};
    R.ok = a.prefix && a.num_seqs <= kRegChunks * kWave && a.max_seq_len < kScan32MaxLen &&
           a.waves % (4 * kXcds) == 0 && a.waves / kXcds >= 8;
    if (!R.ok)
        return R;
    // every load first, then the arithmetic
    const int32_t ng = uniform_load(a.share + 1);
    int32_t raw_own[kRegChunks];
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
        const int32_t b = c * kWave + lane;
        R.n[c] = b < a.num_seqs ? a.seq_lens[b] : 0;
        raw_own[c] = b < a.num_seqs ? plan_own(a)[b] : 0;
    }
    const bool gin = lane < a.num_seqs;
    const int32_t gcnt = gin ? plan_gcount(a)[lane] : 0;
    const int32_t gblk = gin ? plan_gblocks(a)[lane] : 0;
    if (ng <= 0 || ng > a.num_seqs / 2 || ng > kWave) {
        R.ok = ng <= 0 || ng > a.num_seqs / 2; // no rows (P off) is fine; too many groups: loops
        R.P = PrefixHead{false, 0, 0, 0};
        R.g_nt = R.g_rows = R.g_unit = R.g_rows_incl = R.g_count = 0;
        R.g_units_incl = 0;
    } else {
        const bool in = lane < ng;
        R.g_nt = in ? min(max(gblk, 0), a.max_blocks_per_seq) << a.tile_shift : 0;
        R.g_count = in ? min(max(gcnt, 0), a.num_seqs) : 0;
        R.g_rows = in ? group_rows(a, R.g_count, R.g_nt) : 0;
        R.g_unit = (int32_t)row_units(R.g_nt);
        R.g_rows_incl = wave_incl_scan32(R.g_rows);
        R.g_units_incl = wave_incl_scan((int64_t)R.g_rows * R.g_unit, lane);
        const int32_t rows = __builtin_amdgcn_readlane(R.g_rows_incl, kWave - 1);
        if (rows > 0 && rows <= a.num_seqs / 2)
            R.P = PrefixHead{true, ng, rows, readlane64(R.g_units_incl, kWave - 1)};
    }
    int32_t carry = 0;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
        const int32_t b = c * kWave + lane;
        int32_t t = 0;
        if (R.P.on && b < a.num_seqs) {
            t = min(max(raw_own[c], 0), a.max_blocks_per_seq) << a.tile_shift;
            t = (int64_t)t * kTile < (int64_t)R.n[c] ? t : 0;
        }
        R.own[c] = t;
        R.units[c] = b < a.num_seqs ? split_tiles(a, R.n[c], t, seq_cost(R.P)) : 0;
        R.incl[c] = wave_incl_scan32(R.units[c]);
        R.carry[c] = carry;
        carry += __builtin_amdgcn_readlane(R.incl[c], kWave - 1);
    }
    R.Th = uniform(carry);
    return R;
}

// run_start from the registers (the sequences' split, W runs)
__device__ __forceinline__ RunStart run_start_regs(const DecodeArgs &a, const LaunchRegs &R,
                                                   int32_t i, int32_t W)
{
    RunStart r;
    r.Th = R.Th;
    r.T = r.Th * a.num_kv_heads;
    r.runs = effective_runs(r.T, W);
    if (i >= r.runs)
        return r;
    r.x0 = (int64_t)i * r.T / r.runs;
    r.x1 = (int64_t)(i + 1) * r.T / r.runs;
    r.pos = R.locate_seq(r.x0);
    return r;
}

// ---- the rows' split -----------------------------------------------------------
// With prefix rows, each XCD's block of W / 8 runs gives its first R (a
// multiple of 4: whole workgroups) to the rows and the others to the
// sequences, so that no CU runs both (a CU serves its waves' loads in order,
// and a row's L2 hits would wait behind the sequences' HBM reads).  R is the
// multiple of 4 that best evens the units per run of the two splits; run r
// of the rows' split (r < Wr = 8 R) and run s of the sequences' (s < W - Wr)
// take XCD x's share when r / R == x, s / (W / 8 - R) == x.
__device__ __forceinline__ int32_t row_runs(const DecodeArgs &a, const PrefixHead &P, int64_t Th,
                                            int32_t W)
{
    const int32_t per = W / kXcds;
    const double ur = (double)P.units * a.num_kv_heads, us = (double)Th * a.num_kv_heads;
    const double ideal = per * ur / (ur + us);
    int32_t lo = (int32_t)(ideal / 4) * 4;
    lo = max(4, min(lo, per - 4));
    const int32_t hi = min(lo + 4, per - 4);
    auto cost = [&](int32_t R) { return fmax(ur / (kXcds * R), us / (W - kXcds * R)); };
    return kXcds * (cost(hi) < cost(lo) ? hi : lo);
}

// Run r of Wr over the rows: units [x0, x1) of T = Hkv * P.units and the row
// holding x0.
// (R: the launch's registers when R.ok, else the loops look the rows up)
__device__ __forceinline__ RunStart row_run_start(const DecodeArgs &a, int lane, int32_t r,
                                                  int32_t Wr, const PrefixHead &P,
                                                  const LaunchRegs &R)
{
    RunStart s;
    s.Th = P.units;
    s.T = P.units * a.num_kv_heads;
    s.runs = effective_runs(s.T, Wr);
    if (r >= s.runs)
        return s;
    s.x0 = (int64_t)r * s.T / s.runs;
    s.x1 = (int64_t)(r + 1) * s.T / s.runs;
    const int32_t g = (int32_t)(s.x0 / s.Th);
    const int64_t y = s.x0 - (int64_t)g * s.Th;
    s.pos = row_segment(g, R.ok ? R.locate_row(y, true) : locate_row(a, lane, y, true, P),
                        (int64_t)g * s.Th);
    return s;
}

// The row after p: the head's next row, else the next head's first.
__device__ __forceinline__ SegPos next_row(const DecodeArgs &a, int lane, const SegPos &p,
                                           const PrefixHead &P, const LaunchRegs &R)
{
    const int64_t first = p.first_tile + row_units(p.n);
    const bool wrap = p.row + 1 >= P.rows;
    const int32_t g = wrap ? p.g + 1 : p.g;
    const int32_t y = wrap ? 0 : p.row + 1;
    const RowPos r = R.ok ? R.locate_row(y, false) : locate_row(a, lane, y, false, P);
    return SegPos{g, 0, r.nt, 0, r.row, r.gi, r.chunk, first};
}

// Partial-state slot of run i's piece of sequence segment (g, b):
// i + g * B + b.  The runs touching one segment are consecutive, and a run's
// segments follow each other, so no two (run, segment) pairs share a slot.
__device__ __forceinline__ int64_t balanced_slot(const DecodeArgs &a, int64_t i, int32_t g,
                                                 int32_t b)
{
    return i + (int64_t)g * a.num_seqs + b;
}

// First slot of row run r's piece of row `row` of head g: prefix_base +
// (r + g rows + row) SPR, then one slot per member of the row (by the same
// argument, over the rows, no two pieces share one).
__device__ __forceinline__ int64_t row_slot(const DecodeArgs &a, int64_t r, int32_t g,
                                            int32_t row, const PrefixHead &P)
{
    return a.prefix_base + (r + (int64_t)g * P.rows + row) * prefix_row_seqs(a.group);
}

// Run holding tile x when T tiles are cut into R runs [i*T/R, (i+1)*T/R)
// (R <= T, so runs are never empty and consecutive runs are adjacent).
__device__ __forceinline__ int64_t run_of_tile(int64_t x, int64_t T, int32_t R)
{
    // x < T: with T R below 2^32 the quotient is a 32-bit division (a 64-bit
    // one is a long emulated sequence)
    if (T * R < ((int64_t)1 << 32))
        return (int64_t)(((uint32_t)(x + 1) * (uint32_t)R - 1u) / (uint32_t)T);
    return ((x + 1) * R - 1) / T;
}

// The partial states of segment (sequence b of n tokens, KV head g) of a
// balanced launch with prefix rows, in the order the merge folds them: the
// pieces of its own tiles in the sequences' split, slots seq_w0 .. seq_w0 +
// seq_n - 1, then, when its prefix row reads its leading tiles, one slot per
// piece of that row at the member's place in it, row_w0 + k SPR for k <
// row_n.  seq_n = 0 when one run held all the sequence's tiles, no row read
// any, and that run wrote the rows itself.  The run that decodes the
// segment's first own tile (unit S0 of the sequences' split of T units over
// R runs) writes them to seg_dir for the merge.
struct SegLists {
    int32_t seq_w0, seq_n, row_w0, row_n;
};

__device__ __forceinline__ int32_t *seg_dir_entry(const DecodeArgs &a, int32_t g, int32_t b)
{
    return a.seg_dir + 4 * ((int64_t)g * a.num_seqs + b);
}

// (grp_raw, rank_raw: plan_group(a)[b] and plan_rank(a)[b] as loaded, so
// that the caller can issue those loads early)
__device__ __forceinline__ SegLists segment_lists(const DecodeArgs &a, int lane, int32_t b,
                                                  int32_t g, int32_t n, int32_t own, int64_t S0,
                                                  int64_t T, int32_t R, int32_t Wr,
                                                  const PrefixHead &P, const LaunchRegs &L,
                                                  int32_t grp_raw, int32_t rank_raw)
{
    SegLists e{0, 0, 0, 0};
    const int32_t nt = tiles_of(n) - own; // >= 1: a member's own tiles hold its last token
    const int64_t i0 = run_of_tile(S0, T, R);
    const int64_t i1 = run_of_tile(S0 + nt - 1, T, R);
    e.seq_w0 = (int32_t)balanced_slot(a, i0, g, b);
    e.seq_n = own == 0 && i0 == i1 ? 0 : (int32_t)(i1 - i0 + 1);
    if (own > 0 && P.on) {
        const int32_t spr = prefix_row_seqs(a.group);
        const int32_t gi = uniform(min(max(grp_raw, 0), P.ng - 1));
        const int32_t count =
            uniform(L.ok ? __builtin_amdgcn_readlane(L.g_count, gi) : group_count(a, gi));
        const int32_t rank = uniform(min(max(rank_raw, 0), max(count - 1, 0)));
        const RowPos r = L.ok ? L.row_of_group(gi, rank / spr)
                              : row_of_group(a, lane, gi, rank / spr, P);
        if (count > 0 && r.nt > 0) {
            // the rows' own split: Hkv * P.units units over Wr runs
            const int64_t Tr = P.units * a.num_kv_heads;
            const int32_t Rr = effective_runs(Tr, Wr);
            const int64_t S0r = (int64_t)g * P.units + r.before + kSegmentCostShared;
            const int64_t j0 = run_of_tile(S0r, Tr, Rr);
            const int64_t j1 = run_of_tile(S0r + row_body(r.nt) - 1, Tr, Rr);
            e.row_w0 = (int32_t)(row_slot(a, j0, g, r.row, P) + rank % spr);
            e.row_n = (int32_t)(j1 - j0 + 1);
        }
    }
    return e;
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
