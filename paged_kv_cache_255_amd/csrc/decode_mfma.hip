// PagedAttention decode on the matrix cores (gfx950 MFMA).
//
// What it computes: dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation
// and How PagedAttention Fixes It", §1 (attention formula; one new query per
// sequence against the cached K/V) and §4 "The PagedAttention CUDA Kernel"
// (the query walks its block table and reads K/V from scattered physical
// blocks); §2 "Example 2" (query heads of a group share one KV head).
//
// A wave processes a run of 16-token tiles of one (sequence, KV head); a cache
// block of 16, 32, ... 256 tokens is 1, 2, ... 16 consecutive tiles.  The G
// query heads of the KV head sit in the 16 columns of the MFMA tiles (G <= 16;
// unused columns carry q = 0 and are discarded), so each K and V tile is read
// from HBM once for the whole group.  Per tile:
//   S^T[16 tokens][16 heads] = K_tile[16][D] * Q^T[D][16]     (D/32 MFMA 16x16x32)
//   online softmax on S^T, 4 tokens x 1 head per lane
//   O^T[D][16 heads] += V^T_tile[D][16] * P^T[16][16 heads]   (D/16 MFMA 16x16x16)
// The output layout of S^T (lane l: tokens 4*(l/16)+r, head l%16) is the
// B-operand layout of the second product, so P never leaves the registers.
// FP8 tiles are widened to the q type with the hardware converter (exact:
// every E4M3 value is a bf16 and an fp16 value).
//
// A wave keeps a ring of DEPTH tiles (2 at 16-bit KV, 4 at FP8): the loads of
// the next DEPTH - 1 tiles are in flight while the current tile's math runs,
// and each block-table entry is read with a scalar load one tile before the
// loads that use it.
//
// Work split (DecodeArgs::partition):
//   0   one wave per (sequence, KV head), output written directly;
//   > 0 one wave per (sequence, KV head, partition of that many tokens),
//       partial states merged by merge.hip;
//   balanced: the tiles of all (KV head, sequence) segments, head-major,
//       are cut into W equal runs, one per wave (W = the waves the GPU holds
//       at once), each XCD taking one eighth of them in order; a run that
//       covers a whole segment writes the output, the others leave partial
//       states that merge.hip combines.
#include <map>
#include <mutex>
#include <type_traits>

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

// Largest gap (log2 units) between a tile's scores and the reference max
// before the accumulators are rescaled: weights stay <= 2^8, exact in bf16/fp16
// range and harmless to fp32 sums.
constexpr float kLazyRescale = 8.0f;

// One wave's state and per-tile work for one (sequence, KV head).
template <int QT, int KT, int D>
struct MfmaWave {
    using M = Mma<QT>;
    using TQ = typename Store<QT>::T;
    using A8 = typename M::A8;
    using A4 = typename M::A4;
    static constexpr int KE = Store<KT>::bytes;        // 2 or 1
    static constexpr int ROW_BYTES = D * KE;            // one K row
    static constexpr int CHUNKS = ROW_BYTES / 16;       // 16-byte chunks per K row
    static constexpr int CH_PER_LANE = CHUNKS / 4;      // chunks per lane per tile
    static constexpr int QK_MMAS = D / 32;
    static constexpr int PV_TILES = D / 16;
    static constexpr int TILE_BYTES = kTile * D * KE;
    // Tiles in flight per wave: an FP8 tile is half the bytes of a 16-bit
    // one, so twice as many keep the same bytes in flight.
    static constexpr int DEPTH = KE == 1 ? 4 : 2;
    static_assert(CHUNKS % 4 == 0, "row must split into 4 lane groups");

    struct Tile {
        u32x4 k[CH_PER_LANE];
        uint32_t v[PV_TILES][KE];
    };

    // The step's new token (pa_decode_append), in the cache's storage format
    // and in tile layout: the K chunks a lane would hold if its column were
    // the token's row, and the V value of dim 16 t + col.  It replaces the
    // token's slot in the registers of the last tile, so that tile's loads
    // need not wait for the token's own store.
    struct NewToken {
        u32x4 k[CH_PER_LANE];
        uint32_t v[PV_TILES];
        int tok; // the token's offset inside its tile
    };

    int col; // MFMA column: query head within the group
    int grp; // lane group: 4 tokens of S^T, 4 dims of O^T
    A8 qop[QK_MMAS];
    f32x4 acc[PV_TILES];
    float m_run; // running max of head `col` (log2 units)
    float l_run; // this lane's share of the running sum

    __device__ MfmaWave(int lane) : col(lane & 15), grp(lane >> 4) {}

    // q of head `col` as the B operand of the QK products; the dim mapping
    // matches the K operand loaded by load_tile.
    __device__ void start(const DecodeArgs &a, int32_t b, int32_t g)
    {
        const TQ *qp = static_cast<const TQ *>(a.q) +
                       ((size_t)b * a.num_q_heads + (size_t)g * a.group + col) * D;
        const bool real = col < a.group;
#pragma unroll
        for (int m = 0; m < QK_MMAS; ++m) {
            int d0;
            if constexpr (KE == 2)
                d0 = (grp + 4 * m) * 8;
            else
                d0 = (grp + 4 * (m / 2)) * 16 + 8 * (m % 2);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (real)
                v = load16(qp + d0); // 8 consecutive q values, 16-byte aligned
            qop[m] = __builtin_bit_cast(A8, v);
        }
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t)
            acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = kMaxStart;
        l_run = 0.f;
    }

    // Row (b, g) of k_new / v_new as loaded (q dtype), in tile layout: the
    // K chunks of the token's row that lane (col, grp) would hold (16-bit
    // KV: chunk grp + 4 j, 8 dims; FP8: chunk grp + 4 j, 16 dims, as two
    // 16-byte halves) and the V value of dim 16 t + col.
    struct RawToken {
        u32x4 k[KE == 2 ? CH_PER_LANE : 2 * CH_PER_LANE];
        TQ v[PV_TILES];
    };

    __device__ void load_token_raw(const DecodeArgs &a, int32_t b, int32_t g, RawToken &rt) const
    {
        const size_t row = ((size_t)b * a.num_kv_heads + g) * D;
        const TQ *kr = static_cast<const TQ *>(a.k_new) + row;
        const TQ *vr = static_cast<const TQ *>(a.v_new) + row;
#pragma unroll
        for (int j = 0; j < CH_PER_LANE; ++j) {
            const int c = grp + 4 * j; // chunk of the K row this lane holds
            if constexpr (KE == 2) {
                rt.k[j] = load16(kr + c * 8);
            } else {
                rt.k[2 * j] = load16(kr + c * 16);
                rt.k[2 * j + 1] = load16(kr + c * 16 + 8);
            }
        }
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t)
            rt.v[t] = vr[16 * t + col];
    }

    // The raw token in the cache's storage format, converted as the append
    // does (FP8: e4m3 of x * inv, nearest even, saturating).
    __device__ void finish_token(const DecodeArgs &a, const RawToken &rt, int tok,
                                 NewToken &nt) const
    {
        nt.tok = tok;
#pragma unroll
        for (int j = 0; j < CH_PER_LANE; ++j) {
            if constexpr (KE == 2) {
                nt.k[j] = rt.k[j];
            } else {
                const u32x4 lo = rt.k[2 * j], hi = rt.k[2 * j + 1];
                const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                auto half = [](uint32_t x, bool high) {
                    return to_f32<QT>(__builtin_bit_cast(TQ, (uint16_t)(high ? x >> 16 : x & 0xFFFFu)));
                };
                uint32_t q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    q[i] = e4m3x4(half(w[2 * i], false) * a.k_inv, half(w[2 * i], true) * a.k_inv,
                                  half(w[2 * i + 1], false) * a.k_inv,
                                  half(w[2 * i + 1], true) * a.k_inv);
                nt.k[j] = u32x4{q[0], q[1], q[2], q[3]};
            }
        }
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t) {
            if constexpr (KE == 2)
                nt.v[t] = __builtin_bit_cast(uint16_t, rt.v[t]);
            else
                nt.v[t] = f32_to_e4m3(to_f32<QT>(rt.v[t]) * a.v_inv);
        }
    }

    // Stores the token from its tile-layout registers into cache slot
    // (block blk, offset off): the lanes of column 0 write the K row (chunk
    // grp + 4 j each), the lanes of group 0 the V values of dims 16 t + col.
    // The same bytes as store_token writes for the append kernel.
    __device__ void store_new_token(const DecodeArgs &a, const NewToken &nt, int32_t blk,
                                    int32_t off, int32_t sh, int32_t g) const
    {
        using TK = typename Store<KT>::T;
        const size_t tile0 = ((size_t)blk * a.num_kv_heads + g) << sh;
        if (col == 0) {
            char *kd = reinterpret_cast<char *>(static_cast<TK *>(const_cast<void *>(a.k_cache)) +
                                                (tile0 * kTile + off) * D);
#pragma unroll
            for (int j = 0; j < CH_PER_LANE; ++j)
                *reinterpret_cast<u32x4 *>(kd + (grp + 4 * j) * 16) = nt.k[j];
        }
        if (grp == 0) {
            TK *vd = static_cast<TK *>(const_cast<void *>(a.v_cache)) +
                     (tile0 + off / kTile) * D * kTile;
            const int u = off % kTile;
#pragma unroll
            for (int t = 0; t < PV_TILES; ++t) {
                const int vi = v_tile_index<KE>(u, 16 * t + col);
                if constexpr (KE == 2)
                    reinterpret_cast<uint16_t *>(vd)[vi] = (uint16_t)nt.v[t];
                else
                    reinterpret_cast<uint8_t *>(vd)[vi] = (uint8_t)nt.v[t];
            }
        }
    }

    // Puts the new token into tile T (the sequence's last tile).
    __device__ void apply_new_token(Tile &T, const NewToken &nt) const
    {
#pragma unroll
        for (int j = 0; j < CH_PER_LANE; ++j)
            if (col == nt.tok)
                T.k[j] = nt.k[j];
        if (grp != nt.tok / 4)
            return;
        const int r = nt.tok % 4; // the token's place among this lane's 4
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t) {
            if constexpr (KE == 2) {
                const int w = r / 2, sh = 16 * (r % 2);
                const uint32_t keep = ~(0xFFFFu << sh);
                if (w == 0)
                    T.v[t][0] = (T.v[t][0] & keep) | (nt.v[t] << sh);
                else
                    T.v[t][1] = (T.v[t][1] & keep) | (nt.v[t] << sh);
            } else {
                const int sh = 8 * r;
                T.v[t][0] = (T.v[t][0] & ~(0xFFu << sh)) | (nt.v[t] << sh);
            }
        }
    }

    // K: token `col`, chunks grp, grp+4, ... (64 contiguous bytes of every row
    // per load instruction).  V^T: dims 16t + col, tokens 4*grp .. 4*grp+3
    // (1 KiB contiguous per load instruction, see v_tile_index).  kt and vt
    // are wave-uniform.  STREAM: loads for data read once (the nontemporal
    // hint); otherwise loads that keep the tile in the caches, for blocks
    // other sequences also read.
    template <bool STREAM>
    __device__ static u32x4 load16_policy(const char *p)
    {
        if constexpr (STREAM)
            return load16_stream(p);
        else
            return load16(p);
    }

    template <bool STREAM>
    __device__ static void load_tile(const char *kt, const char *vt, int col, int grp, Tile &T)
    {
#pragma unroll
        for (int j = 0; j < CH_PER_LANE; ++j)
            T.k[j] = load16_policy<STREAM>(kt + col * ROW_BYTES + (grp + 4 * j) * 16);
        // lane L = col + 16 grp takes 16-byte piece 64 q + L of the V tile:
        // V^T rows 16 t + col, tokens 4 grp .. 4 grp + 3, for the 16 / (4 KE)
        // values of t that piece holds (v_tile_index)
        const int L = col + 16 * grp;
#pragma unroll
        for (int q = 0; q < PV_TILES * 4 * KE / 16; ++q) {
            const u32x4 x = load16_policy<STREAM>(vt + q * 1024 + 16 * L);
            if constexpr (KE == 2) {
                T.v[2 * q][0] = x.x;
                T.v[2 * q][1] = x.y;
                T.v[2 * q + 1][0] = x.z;
                T.v[2 * q + 1][1] = x.w;
            } else {
                T.v[4 * q][0] = x.x;
                T.v[4 * q + 1][0] = x.y;
                T.v[4 * q + 2][0] = x.z;
                T.v[4 * q + 3][0] = x.w;
            }
        }
    }

    // K operand of QK product m: 8 dims of the lane's token row (FP8 widened
    // to the q type).
    __device__ static A8 k_operand(const Tile &T, int m)
    {
        if constexpr (KE == 2) {
            return __builtin_bit_cast(A8, T.k[m]);
        } else {
            const u32x4 c = T.k[m / 2];
            const uint32_t w0 = (m % 2) ? c.z : c.x;
            const uint32_t w1 = (m % 2) ? c.w : c.y;
            u32x4 e = {M::fp8x2(w0, false), M::fp8x2(w0, true), M::fp8x2(w1, false),
                       M::fp8x2(w1, true)};
            return __builtin_bit_cast(A8, e);
        }
    }

    // V^T operand of PV product t: the lane's 4 tokens of dim 16 t + col.
    __device__ static u32x2 v_operand(const Tile &T, int t)
    {
        if constexpr (KE == 2)
            return u32x2{T.v[t][0], T.v[t][1]};
        else
            return u32x2{M::fp8x2(T.v[t][0], false), M::fp8x2(T.v[t][0], true)};
    }

    // Scaled scores of S^T (tokens lo .. valid - 1 of the tile, -inf for the
    // others) and the tile's max over them, per query head.
    __device__ float scores(const f32x4 &s, int lo, int valid, float sc, float (&x)[4]) const
    {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            x[r] = (4 * grp + r < valid && 4 * grp + r >= lo) ? s[r] * sc : -INFINITY;
        const float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        return max_xor32(max_xor16(bm));
    }

    // The reference max m_run moves only when a tile's max exceeds it by
    // more than kLazyRescale (log2 units); until then the weights
    // 2^(s - m_run) stay below 2^kLazyRescale and acc, l need no rescale.
    // Any reference gives the same softmax: acc and l share it.
    __device__ void rescale_if(float bm)
    {
        if (__any(bm > m_run + kLazyRescale)) {
            const float mn = fmaxf(m_run, bm);
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
            m_run = mn;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < PV_TILES; ++t)
                acc[t] *= alpha;
        }
    }

    // The tile's softmax weights 2^(x - m_run), added to l, as the B operand
    // of the PV products.
    __device__ A4 weights(const float (&x)[4])
    {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            p[r] = __builtin_amdgcn_exp2f(x[r] - m_run);
        l_run += (p[0] + p[1]) + (p[2] + p[3]);
        const u32x2 pp = {M::pack2(p[0], p[1]), M::pack2(p[2], p[3])};
        return __builtin_bit_cast(A4, pp);
    }

    // One tile: its tokens lo .. valid - 1 (0 <= lo, valid <= 16) belong to
    // the range; lo > 0 only in a tile that holds the window start.
    __device__ void compute(const Tile &T, int lo, int valid, float sc)
    {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < QK_MMAS; ++m)
            s = M::qk(k_operand(T, m), qop[m], s);
        float x[4];
        rescale_if(scores(s, lo, valid, sc, x));
        const A4 pop = weights(x);
        // Slots past the end or before the window start may hold anything
        // (NaN included): their V values are zeroed, without a branch, so
        // 0 * garbage never reaches acc.  This lane's tokens r = 0..3 are in
        // the range when khi > r >= klo.
        const int khi = valid - 4 * grp, klo = lo - 4 * grp;
        const uint32_t keep_x = (klo <= 0 && khi > 0 ? 0x0000FFFFu : 0u) |
                                (klo <= 1 && khi > 1 ? 0xFFFF0000u : 0u);
        const uint32_t keep_y = (klo <= 2 && khi > 2 ? 0x0000FFFFu : 0u) |
                                (klo <= 3 && khi > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t) {
            u32x2 vw = v_operand(T, t);
            vw.x &= keep_x;
            vw.y &= keep_y;
            acc[t] = M::pv(__builtin_bit_cast(A4, vw), pop, acc[t]);
        }
    }

    // A whole tile (all 16 tokens in range) for CG states at once, each
    // with the arithmetic of compute(T, 0, 16, sc): the K and V operands are
    // formed once, and the groups' products and softmax steps are issued
    // side by side instead of one group after another.
    template <int CG>
    __device__ static void compute_groups(MfmaWave (&w)[CG], const Tile &T, float sc)
    {
        f32x4 s[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c)
            s[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < QK_MMAS; ++m) {
            const A8 kop = k_operand(T, m);
#pragma unroll
            for (int c = 0; c < CG; ++c)
                s[c] = M::qk(kop, w[c].qop[m], s[c]);
        }
        float x[CG][4], bm[CG];
        bool move = false;
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            bm[c] = w[c].scores(s[c], 0, kTile, sc, x[c]);
            move |= bm[c] > w[c].m_run + kLazyRescale;
        }
        if (__any(move)) {
#pragma unroll
            for (int c = 0; c < CG; ++c)
                w[c].rescale_if(bm[c]);
        }
        A4 pop[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c)
            pop[c] = w[c].weights(x[c]);
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t) {
            const A4 vop = __builtin_bit_cast(A4, v_operand(T, t));
#pragma unroll
            for (int c = 0; c < CG; ++c)
                w[c].acc[t] = M::pv(vop, pop[c], w[c].acc[t]);
        }
    }

    // The step's token as run() leaves it (pa_decode_append): in the cache's
    // storage format, bound for offset `off` of block `blk`; put is false
    // when the range does not end the sequence or the slot is refused.
    struct PendingToken {
        bool put;
        NewToken nt;
        int32_t blk, off;
    };

    // Tokens [t0, t1) of (b, g), of a sequence of n tokens; t0 is a multiple
    // of 16.  Tokens before the window start (seq_starts[b]) are left out.
    // Returns false if a block-table entry is outside the pool (that block is
    // not read), if the window start is outside [0, n], or if the step's
    // token is to be appended here (a.append and t1 == n) and its slot is not
    // the cache slot of position n - 1.
    // HINT: a.share is set (the launch reads its hint once per range and
    // picks the cache policy per tile); without it every tile streams.
    // The appended token is not stored here: it comes back in `tok` for the
    // caller to store (store_pending) or hold.
    template <bool HINT>
    __device__ bool run(const DecodeArgs &a, int32_t b, int32_t g, int32_t t0, int32_t t1,
                        int32_t n_seq, PendingToken &tok)
    {
        // The block table does not change while the kernel runs: its entries
        // are read with scalar loads (one wave-uniform id per tile, fetched
        // one tile before its loads), which keeps them out of the vector-load
        // queue the tiles stream through.
        using CI32 = __attribute__((address_space(4))) const int32_t;
        b = uniform(b);
        g = uniform(g);
        // A block of 16 << sh tokens is 1 << sh tiles: tile jb of the
        // sequence is tile jb & mask of block table[jb >> sh].
        const CI32 *table = (const CI32 *)(a.block_tables + (size_t)b * a.max_blocks_per_seq);
        const int32_t sh = a.tile_shift;
        const int32_t mask = (1 << sh) - 1;
        const char *kbase = static_cast<const char *>(a.k_cache) + ((size_t)g << sh) * TILE_BYTES;
        const char *vbase = static_cast<const char *>(a.v_cache) + ((size_t)g << sh) * TILE_BYTES;
        const size_t bstride = ((size_t)a.num_kv_heads << sh) * TILE_BYTES;
        const int32_t jb0 = uniform(t0 / kTile);
        const int32_t last = uniform((t1 + kTile - 1) / kTile) - 1;
        t1 = uniform(t1);
        const float sc = a.score_scale;
        const uint32_t nblocks = (uint32_t)a.num_blocks;

        auto id_of = [&](int32_t jb) -> int32_t {
            return uniform(table[uniform(min(jb, last) >> sh)]);
        };
        auto valid_of = [&](int32_t jb) { return min(kTile, t1 - jb * kTile); };
        const int32_t w0 = a.seq_starts ? uniform(((const CI32 *)a.seq_starts)[b]) : 0;
        auto lo_of = [&](int32_t jb) { return min(kTile, max(0, w0 - jb * kTile)); };
        const bool append_here = a.append && t1 == uniform(n_seq);

        // A ring of DEPTH tiles over tiles [s0, s1] (s0 <= s1), all read with
        // one cache policy: while one is computed, the next DEPTH - 1 are in
        // flight.  The loop runs over groups of DEPTH tiles and has one exit,
        // at the bottom; the next load is issued on every path (past s1 it
        // re-reads tile s1, an L2 hit).  A load issued on one path only, or an
        // exit that shares a block with the back edge, would make the
        // compiler's wait counts assume a shorter queue and wait for the next
        // tile before the current one is done; so would a branch between the
        // two policies inside the loop.  An entry outside the pool is
        // recorded and block 0 read in its place (the caller turns the result
        // into NaN), so no early exit is needed either.
        bool bad = w0 < 0 || w0 > n_seq;
        auto checked = [&](int32_t id) {
            const bool out = (uint32_t)id >= nblocks;
            bad |= out;
            return out ? 0 : id;
        };
        // The step's token (position t1 - 1) when this range ends the
        // sequence.  Its row is loaded before any tile (the addresses need
        // nothing but b and g).  The slot is checked and the token converted
        // (prepare_token): for FP8, whose ring holds three tiles in flight,
        // once those are issued (keeping the raw FP8 row live through the
        // ring would spill); for 16-bit KV, whose ring holds one, just
        // before the last tile is computed (a wait after the first tile's
        // loads would hold back the second's).  The token replaces its slot
        // in the last tile's registers, and once every tile is in, it is
        // stored to the cache: no store precedes a tile's loads (the vector
        // memory counter covers stores too, so the wait for that tile would
        // wait for the store's acknowledgement as well).
        constexpr bool kPrepareEarly = KE == 1;
        bool put = false;
        NewToken nt;
        RawToken rt;
        // The token's slot and the block id of the last tile come in with
        // vector loads: scalar loads may complete out of order, so the
        // first tile's block id (a scalar load) would wait for these too,
        // and the slots are cold at launch.
        int32_t slot_v = -1, id_last_v = 0, slot = -1, id_last = 0;
        const int32_t off_last = (t1 - 1) & ((kTile << sh) - 1); // in its block
        if (append_here) {
            using GI32 = __attribute__((address_space(1))) const int32_t;
            slot_v = __builtin_nontemporal_load((GI32 *)(a.slots + b));
            id_last_v = __builtin_nontemporal_load(
                (GI32 *)(a.block_tables + (size_t)b * a.max_blocks_per_seq + (last >> sh)));
            load_token_raw(a, b, g, rt);
        }
        auto prepare_token = [&]() {
            slot = uniform(slot_v);
            id_last = uniform(id_last_v);
            if (slot < 0)
                return;
            if ((uint32_t)id_last >= nblocks || slot != (id_last << sh) * kTile + off_last) {
                bad = true;
                return;
            }
            put = true;
            finish_token(a, rt, (t1 - 1) % kTile, nt);
        };
        // With the hint, the block ids of the first DEPTH tiles are fetched
        // before the split below is known (every range starts with a ring at
        // jb0), so that reading the hint adds no step to the chain before
        // the first tile loads.
        int32_t id0[DEPTH];
        if constexpr (HINT) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d)
                id0[d] = id_of(jb0 + d);
        }
        auto ring = [&](auto stream, int32_t s0, int32_t s1, bool first, bool hook) {
            constexpr bool STREAM = decltype(stream)::value;
            auto id_at = [&](int32_t jb) -> int32_t {
                return uniform(table[uniform(min(jb, s1) >> sh)]);
            };
            auto load = [&](int32_t phys, int32_t jb, Tile &T) {
                jb = min(jb, s1);
                const size_t o = (size_t)phys * bstride + (size_t)(jb & mask) * TILE_BYTES;
                load_tile<STREAM>(kbase + o, vbase + o, col, grp, T);
            };
            Tile T[DEPTH];
            const int32_t n = s1 - s0 + 1;
            // tile s0 + k lives in T[k % DEPTH]
            // (with `first`, s0 = jb0 and the ids past s1 are those of tiles
            // of the range past s1: valid blocks, read and not used)
#pragma unroll
            for (int d = 0; d + 1 < DEPTH; ++d)
                load(checked(HINT && first ? id0[d] : id_at(s0 + d)), s0 + d, T[d]);
            // block id of the next tile to load
            int32_t id_next = HINT && first ? id0[DEPTH - 1] : id_at(s0 + DEPTH - 1);
            if (kPrepareEarly && append_here && hook)
                prepare_token();
            int32_t i = 0;
            for (; i + DEPTH <= n; i = uniform(i + DEPTH)) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    const int32_t jb = s0 + i + d;
                    const int32_t id_after = id_at(jb + DEPTH); // one tile ahead of use
                    load(checked(id_next), jb + DEPTH - 1, T[(d + DEPTH - 1) % DEPTH]);
                    __builtin_amdgcn_sched_barrier(0); // that load goes out before T[d] is waited for
                    if (append_here && jb == last) {
                        if (!kPrepareEarly)
                            prepare_token();
                        if (put)
                            apply_new_token(T[d], nt);
                    }
                    compute(T[d], lo_of(jb), valid_of(jb), sc);
                    id_next = id_after;
                }
            }
            // the last n - i (< DEPTH) tiles, already in T[0 ..]
#pragma unroll
            for (int d = 0; d + 1 < DEPTH; ++d) {
                if (i + d < n) {
                    const int32_t jb = s0 + i + d;
                    if (append_here && jb == last) {
                        if (!kPrepareEarly)
                            prepare_token();
                        if (put)
                            apply_new_token(T[d], nt);
                    }
                    compute(T[d], lo_of(jb), valid_of(jb), sc);
                }
            }
            // Drain the re-reads issued past s1, so no load into these
            // registers is in flight when the next ring starts.
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        };
        // The first `shared` blocks of the table are also read by other
        // sequences of the batch: their tiles go through a ring of caching
        // loads, the rest through a ring of streaming loads.
        if constexpr (HINT) {
            int32_t shared = uniform(((const CI32 *)plan_shared(a))[b]);
            shared = min(max(shared, 0), a.max_blocks_per_seq);
            const int32_t split = uniform(min(max(shared << sh, jb0), last + 1));
            if (split > jb0)
                ring(std::integral_constant<bool, false>{}, jb0, split - 1, true, true);
            if (split <= last)
                ring(std::integral_constant<bool, true>{}, split, last, split == jb0,
                     split == jb0);
        } else {
            ring(std::integral_constant<bool, true>{}, jb0, last, false, true);
        }
        tok.put = put;
        tok.nt = nt;
        tok.blk = id_last;
        tok.off = off_last;
        return !bad;
    }

    __device__ void store_pending(const DecodeArgs &a, const PendingToken &tok, int32_t g) const
    {
        if (tok.put)
            store_new_token(a, tok.nt, tok.blk, tok.off, a.tile_shift, g);
    }

    // The bytes store_new_token writes, as two images: the K row (ROW_BYTES,
    // contiguous at k_row) and the V values in dim order (D * KE bytes,
    // scattered over the V tile at v_tile, token u: Stage::image_v).
    __device__ static char *token_k_row(const DecodeArgs &a, const PendingToken &tok, int32_t g)
    {
        const size_t tile0 = ((size_t)tok.blk * a.num_kv_heads + g) << a.tile_shift;
        return static_cast<char *>(const_cast<void *>(a.k_cache)) +
               (tile0 * kTile + tok.off) * ROW_BYTES;
    }

    __device__ static char *token_v_tile(const DecodeArgs &a, const PendingToken &tok, int32_t g)
    {
        const size_t tile0 = ((size_t)tok.blk * a.num_kv_heads + g) << a.tile_shift;
        return static_cast<char *>(const_cast<void *>(a.v_cache)) +
               (tile0 + tok.off / kTile) * TILE_BYTES;
    }

    __device__ void put_token_k(char *img, const NewToken &nt) const
    {
        if (col != 0)
            return;
#pragma unroll
        for (int j = 0; j < CH_PER_LANE; ++j)
            *reinterpret_cast<u32x4 *>(img + (grp + 4 * j) * 16) = nt.k[j];
    }

    __device__ void put_token_v(char *img, const NewToken &nt) const
    {
        if (grp != 0)
            return;
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t) {
            if constexpr (KE == 2)
                reinterpret_cast<uint16_t *>(img)[16 * t + col] = (uint16_t)nt.v[t];
            else
                reinterpret_cast<uint8_t *>(img)[16 * t + col] = (uint8_t)nt.v[t];
        }
    }

    // The lane groups hold disjoint tokens: sum their shares of l.
    __device__ void finish() { l_run = sum_xor32(sum_xor16(l_run)); }

    // Output rows G g .. G g + G - 1 of sequence b (G = group): [G][D].
    __device__ static TQ *out_rows(const DecodeArgs &a, int32_t b, int32_t g)
    {
        return static_cast<TQ *>(a.out) + ((size_t)b * a.num_q_heads + (size_t)g * a.group) * D;
    }

    // The G output rows from o: the output tensor's, or an LDS image of them.
    __device__ void put_out(TQ *o, const DecodeArgs &a, bool ok) const
    {
        if (col >= a.group)
            return;
        o += col * D;
        // l = 0: no token in the range (n = 0 or an empty window)
        const float inv = !ok ? NAN : (l_run == 0.f ? 0.f : a.v_scale / l_run);
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[16 * t + 4 * grp + r] = from_f32<QT>(acc[t][r] * inv);
    }

    // A partial state in the workspace layout: m, l of the G heads ([G][2])
    // from ml, acc ([G][D]) from accp (the workspace's, or LDS images).
    __device__ void put_ml(float *ml, const DecodeArgs &a, bool ok) const
    {
        if (col >= a.group || grp != 0)
            return;
        ml[2 * col] = ok ? m_run : NAN;
        ml[2 * col + 1] = ok ? l_run : NAN;
    }

    __device__ void put_acc(float *accp, const DecodeArgs &a, bool ok) const
    {
        if (col >= a.group)
            return;
        accp += col * D;
        const float f = ok ? a.v_scale : NAN;
#pragma unroll
        for (int t = 0; t < PV_TILES; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                accp[16 * t + 4 * grp + r] = acc[t][r] * f;
    }

    __device__ void write_out(const DecodeArgs &a, int32_t b, int32_t g, int32_t n, bool ok)
    {
        put_out(out_rows(a, b, g), a, ok);
    }

    __device__ void write_partial(const DecodeArgs &a, int64_t slot, bool ok)
    {
        put_ml(ws_ml(a, slot, 0), a, ok);
        put_acc(ws_acc(a, slot, 0, D), a, ok);
    }
};

// A run's results (outputs, partial states, the merge's records of
// segments, appended tokens), held in the wave's LDS area and stored when
// the run ends.  The
// tile loads and the stores count in one in-order counter, so the wait for
// a tile loaded after a store also waits for that store's acknowledgement;
// held to the run's end, the stores keep no tile waiting.  Each record is an
// image of its destination's bytes (a multiple of 8), or, for a token's V
// values, of the values to scatter over their tile; one that does not fit
// beside those held stores them first, and one larger than the whole area
// (or an area of no bytes) is stored directly by the caller.  Headers (the
// destination, bytes, image offset) take the area's first kRecs quads.
// `used` and `nrec` are the same in every lane.
struct Stage {
    static constexpr int kRecs = 16;
    u32x4 *area;
    int32_t cap; // image bytes
    int32_t used, nrec;

    __device__ Stage(u32x4 *q, int32_t bytes)
        : area(q), cap(max(0, (bytes & ~15) - kRecs * 16)), used(0), nrec(0)
    {
    }

    // Whether a record of `bytes` (or two, of `bytes` and `bytes2`) can be
    // held, storing those held if it needs their room.  Then image() /
    // image_v() give the LDS images, in that order.
    __device__ bool fits(int lane, int32_t bytes, int32_t bytes2 = -1)
    {
        const int32_t need = ((bytes + 15) & ~15) + (bytes2 < 0 ? 0 : (bytes2 + 15) & ~15);
        const int32_t recs = bytes2 < 0 ? 1 : 2;
        if (need > cap)
            return false;
        if (used + need > cap || nrec + recs > kRecs)
            flush(lane);
        return true;
    }

    __device__ char *image(int lane, const void *dst, int32_t bytes)
    {
        return take(lane, dst, (uint32_t)bytes, bytes);
    }

    // One token's V values in dim order (ke bytes each), bound for its V
    // tile at vt: stored one value per 16-byte piece, at v_tile_index(u, d),
    // not copied.
    __device__ char *image_v(int lane, const void *vt, int ke, int u, int32_t bytes)
    {
        return take(lane, vt, kScatter | (uint32_t)ke << 24 | (uint32_t)u << 16 | (uint32_t)bytes,
                    bytes);
    }

    static constexpr uint32_t kScatter = 0x80000000u; // header kind bit (bytes < 2^16)

    __device__ char *take(int lane, const void *dst, uint32_t word, int32_t bytes)
    {
        char *img = reinterpret_cast<char *>(area + kRecs) + used;
        if (lane == 0) {
            const uint64_t d = reinterpret_cast<uint64_t>(dst);
            area[nrec] = u32x4{(uint32_t)d, (uint32_t)(d >> 32), word, (uint32_t)used};
        }
        used += (bytes + 15) & ~15;
        nrec += 1;
        return img;
    }

    // Records from here on are stored directly by the caller.
    __device__ void close() { cap = 0; }

    // Stores every record held: 16 bytes per lane and instruction when the
    // destination and size allow, else 8.
    __device__ void flush(int lane)
    {
        if (nrec == 0)
            return;
        using GU4 = __attribute__((address_space(1))) u32x4;
        using GU2 = __attribute__((address_space(1))) u32x2;
        wave_lds_sync();
        for (int32_t r = 0; r < nrec; ++r) {
            const u32x4 h = area[r];
            const uint64_t d = ((uint64_t)(uint32_t)uniform((int32_t)h.y) << 32) |
                               (uint32_t)uniform((int32_t)h.x);
            const uint32_t word = (uint32_t)uniform((int32_t)h.z);
            const int32_t bytes = (int32_t)(word & 0xFFFFu);
            const char *src = reinterpret_cast<const char *>(area + kRecs) + uniform((int32_t)h.w);
            if (word & kScatter) {
                using GU16 = __attribute__((address_space(1))) uint16_t;
                using GU8 = __attribute__((address_space(1))) uint8_t;
                const int ke = (int)(word >> 24) & 0x7F, u = (int)(word >> 16) & 0xFF;
                for (int32_t dd = lane; dd * ke < bytes; dd += kWave) {
                    if (ke == 2)
                        *reinterpret_cast<GU16 *>(d + 2 * v_tile_index<2>(u, dd)) =
                            reinterpret_cast<const uint16_t *>(src)[dd];
                    else
                        *reinterpret_cast<GU8 *>(d + v_tile_index<1>(u, dd)) =
                            reinterpret_cast<const uint8_t *>(src)[dd];
                }
            } else if (((bytes | (int32_t)d) & 15) == 0) {
                for (int32_t o = 16 * lane; o < bytes; o += 16 * kWave)
                    *reinterpret_cast<GU4 *>(d + o) = *reinterpret_cast<const u32x4 *>(src + o);
            } else {
                for (int32_t o = 8 * lane; o < bytes; o += 8 * kWave)
                    *reinterpret_cast<GU2 *>(d + o) = *reinterpret_cast<const u32x2 *>(src + o);
            }
        }
        wave_lds_sync();
        used = 0;
        nrec = 0;
    }
};

// LDS quads of one wave's Stage area (16 KiB).
constexpr int kStageQuads = 1024;

// partition == 0 or > 0: one wave per work item (see work.hpp).  HINT:
// a.share is set; each kernel is built with and without it, so the
// launches without the hint run the same code as before it existed.
template <int QT, int KT, int D, bool HINT>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a, int32_t num_items)
{
    const int lane = threadIdx.x & 63;
    const int32_t w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= num_items)
        return;
    const Item it = item_of(a, w);
    if (it.valid_len && it.n > 0 && it.t0 >= it.t1)
        return;
    if ((!it.valid_len || it.n == 0) && it.p > 0)
        return; // the merge writes such rows without reading partial states
    MfmaWave<QT, KT, D> wv(lane);
    wv.start(a, it.b, it.g);
    bool ok = it.valid_len;
    if (ok && it.t1 > it.t0) {
        typename MfmaWave<QT, KT, D>::PendingToken tok;
        ok = wv.template run<HINT>(a, it.b, it.g, it.t0, it.t1, it.n, tok);
        wv.store_pending(a, tok, it.g);
    }
    wv.finish();
    if (a.partition == 0)
        wv.write_out(a, it.b, it.g, it.n, ok);
    else
        wv.write_partial(a, w, ok);
}

// Tiles [j, je) of prefix row `pos` (head pos.g; members [chunk SPR,
// (chunk + 1) SPR) of group pos.gi in rank order, SPR = kPrefixColGroups *
// 16 / G).  The group's shared tiles are read once, through its first
// member's table, with loads that keep them in the caches (the head's other
// rows read the same tiles), and applied to kPrefixColGroups column groups
// of 16 MFMA columns: 16 / G members times G query heads each, so one tile
// load serves SPR sequences.  Per member and query head, the partial state
// (m, l, acc) goes to slot slot0 + (rank - chunk SPR); the merge folds it with
// the member's other parts.  A block id outside the pool makes the piece's
// states NaN.
template <int QT, int KT, int D>
__device__ void prefix_piece(const DecodeArgs &a, int lane, const SegPos &pos, int32_t j,
                             int32_t je, int64_t slot0)
{
    using Wv = MfmaWave<QT, KT, D>;
    using Tile = typename Wv::Tile;
    using A8 = typename Wv::A8;
    using TQ = typename Store<QT>::T;
    using CI32 = __attribute__((address_space(4))) const int32_t;
    constexpr int CG = kPrefixColGroups;
    // One more tile in flight than a sequence's ring: a row tile comes from
    // L2 and its loads must land while the tile before is computed for
    // every column group.
    constexpr int DEPTH = Wv::DEPTH + 1;
    static_assert(CG == 4, "four column groups");
    const int32_t G = a.group, spc = 16 / G;
    const int32_t gi = uniform(pos.gi), g = uniform(pos.g);
    const int32_t count = uniform(group_count(a, gi));
    const int32_t first = uniform(min(max(plan_gfirst(a)[gi], 0), a.num_seqs - count));
    const int32_t lead = uniform(min(max(plan_members(a)[first], 0), a.num_seqs - 1));
    const int32_t rank0 = uniform(pos.chunk * prefix_row_seqs(G));

    // column col of group cg: member rank0 + cg spc + col / G, query head col % G
    const int col = lane & 15, grp = lane >> 4;
    const int32_t mcol = col / G, h = col % G;
    Wv wv[CG] = {Wv(lane), Wv(lane), Wv(lane), Wv(lane)};
    bool real[CG];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
        const int32_t k = cg * spc + mcol;
        real[cg] = mcol < spc && rank0 + k < count;
        const int32_t b =
            real[cg] ? min(max(plan_members(a)[first + rank0 + k], 0), a.num_seqs - 1) : 0;
        const TQ *qp = static_cast<const TQ *>(a.q) +
                       ((size_t)b * a.num_q_heads + (size_t)g * G + h) * D;
#pragma unroll
        for (int m = 0; m < Wv::QK_MMAS; ++m) {
            int d0;
            if constexpr (Store<KT>::bytes == 2)
                d0 = (grp + 4 * m) * 8;
            else
                d0 = (grp + 4 * (m / 2)) * 16 + 8 * (m % 2);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (real[cg])
                v = load16(qp + d0);
            wv[cg].qop[m] = __builtin_bit_cast(A8, v);
        }
#pragma unroll
        for (int t = 0; t < Wv::PV_TILES; ++t)
            wv[cg].acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        wv[cg].m_run = kMaxStart;
        wv[cg].l_run = 0.f;
    }

    // tiles [j, je) of the lead's table, DEPTH - 1 in flight while one is
    // computed
    const int32_t sh = a.tile_shift;
    const int32_t mask = (1 << sh) - 1;
    const CI32 *table = (const CI32 *)(a.block_tables + (size_t)lead * a.max_blocks_per_seq);
    const char *kbase = static_cast<const char *>(a.k_cache) + ((size_t)g << sh) * Wv::TILE_BYTES;
    const char *vbase = static_cast<const char *>(a.v_cache) + ((size_t)g << sh) * Wv::TILE_BYTES;
    const size_t bstride = ((size_t)a.num_kv_heads << sh) * Wv::TILE_BYTES;
    const uint32_t nblocks = (uint32_t)a.num_blocks;
    const float sc = a.score_scale;
    const int32_t s0 = uniform(j), s1 = uniform(je - 1);
    bool bad = false;
    auto id_at = [&](int32_t jb) -> int32_t { return uniform(table[uniform(min(jb, s1) >> sh)]); };
    auto load = [&](int32_t id, int32_t jb, Tile &T) {
        const bool out = (uint32_t)id >= nblocks;
        bad |= out;
        jb = min(jb, s1);
        const size_t o = (size_t)(out ? 0 : id) * bstride + (size_t)(jb & mask) * Wv::TILE_BYTES;
        Wv::template load_tile<false>(kbase + o, vbase + o, col, grp, T);
    };
    Tile T[DEPTH];
    const int32_t n = s1 - s0 + 1;
#pragma unroll
    for (int d = 0; d + 1 < DEPTH; ++d)
        load(id_at(s0 + d), s0 + d, T[d]);
    int32_t id_next = id_at(s0 + DEPTH - 1);
    int32_t i = 0;
    for (; i + DEPTH <= n; i = uniform(i + DEPTH)) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int32_t jb = s0 + i + d;
            const int32_t id_after = id_at(jb + DEPTH);
            load(id_next, jb + DEPTH - 1, T[(d + DEPTH - 1) % DEPTH]);
            __builtin_amdgcn_sched_barrier(0);
            Wv::compute_groups(wv, T[d], sc);
            id_next = id_after;
        }
    }
#pragma unroll
    for (int d = 0; d + 1 < DEPTH; ++d) {
        if (i + d < n)
            Wv::compute_groups(wv, T[d], sc);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
        wv[cg].finish();
        if (!real[cg])
            continue;
        const int64_t slot = slot0 + cg * spc + mcol;
        if (grp == 0) {
            float *ml = ws_ml(a, slot, h);
            ml[0] = bad ? NAN : wv[cg].m_run;
            ml[1] = bad ? NAN : wv[cg].l_run;
        }
        float *accp = ws_acc(a, slot, h, D);
        const float f = bad ? NAN : a.v_scale;
#pragma unroll
        for (int t = 0; t < Wv::PV_TILES; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                accp[16 * t + 4 * grp + q] = wv[cg].acc[t][q] * f;
    }
}

// Run r of Wr in the rows' split: the row pieces its units [x0, x1) meet.
template <int QT, int KT, int D>
__device__ void decode_rows(const DecodeArgs &a, int lane, int32_t r, int32_t Wr,
                            const PrefixHead &P, const LaunchRegs &R)
{
    const RunStart rs = row_run_start(a, lane, r, Wr, P, R);
    if (r >= rs.runs)
        return;
    SegPos pos = rs.pos;
    int64_t x = rs.x0;
    while (x < rs.x1) {
        const int64_t r0 = pos.first_tile + kSegmentCostShared; // the row's tile 0
        const int64_t end = r0 + row_body(pos.n);
        const int64_t lo = max(x, r0), hi = min(rs.x1, end);
        if (hi > lo) {
            const int32_t j = row_tile_at(lo - r0), je = min(pos.n, row_tile_at(hi - r0));
            if (je > j)
                prefix_piece<QT, KT, D>(a, lane, pos, j, je, row_slot(a, r, pos.g, pos.row, P));
        }
        x = end;
        if (x < rs.x1)
            pos = next_row(a, lane, pos, P, R);
    }
}

// Bytes of the block tables each wave touches at launch (two 1 KiB loads):
// the waves of one XCD together cover the first W/8 * 2 KiB of the tables.
constexpr int kTablePrefetchLoads = 2;

// Balanced split: run i of W takes tiles [i*T/W, (i+1)*T/W) of the list of
// all tiles in head-major order ((KV head, sequence, 16-token tile), each
// segment preceded by its start charge, see work.hpp), T tiles in total;
// balanced_run places each XCD's runs on that XCD's workgroups.  HINT as for
// decode_mfma_kernel.
template <int QT, int KT, int D, bool HINT>
__global__ __launch_bounds__(256)
void decode_mfma_balanced_kernel(DecodeArgs a, int32_t W)
{
    __shared__ u32x4 table_sink[4][kWave]; // receives the prefetch, never read
    // the waves' Stage areas: launches with a share plan only (their runs
    // hold several pieces; without one, a run rarely ends a piece before its
    // last, and the area cost config 2's step 0.4 us)
    __shared__ u32x4 stage_lds[4][HINT ? kStageQuads : 1];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t i0 = balanced_run(blockIdx.x, wave, W);
    if (i0 >= W)
        return;

    // A decode step's tables are cold (the host wrote them for this step),
    // and the scalar loads of each run's first block ids would wait a full
    // HBM round trip after the lengths have been read.  So while the lengths
    // load, the waves of each XCD touch the tables, 1 KiB per wave and load,
    // and those block-id loads find them in the XCD's L2.  (Wave k of an XCD
    // covers bytes [1 KiB (k + r W / 8), +1 KiB); placement as balanced_run.)
    {
        const int64_t tbytes = (int64_t)a.num_seqs * a.max_blocks_per_seq * 4;
        const int32_t per_xcd = W % (4 * kXcds) == 0 ? W / kXcds : W;
        const int32_t k = W % (4 * kXcds) == 0 ? (blockIdx.x / kXcds) * 4 + wave : i0;
        const char *tb = reinterpret_cast<const char *>(a.block_tables);
        // (a hint only: skipped for a table that is not 16-byte aligned)
        const int64_t tbytes_in = (reinterpret_cast<uintptr_t>(tb) & 15) == 0 ? tbytes : 0;
#pragma unroll
        for (int r = 0; r < kTablePrefetchLoads; ++r) {
            const int64_t off = ((int64_t)k + (int64_t)r * per_xcd) * 1024 + 16 * lane;
            if (uniform((int32_t)(((int64_t)k + (int64_t)r * per_xcd) * 1024 < tbytes_in)) &&
                off + 16 <= tbytes_in)
                load16_to_lds(tb + off, &table_sink[wave][0]);
        }
    }

    // Prefix rows only come with a share plan, which also turns on HINT: the
    // launches without one run the code they ran before rows existed.
    PrefixHead P{false, 0, 0, 0};
    LaunchRegs R;
    R.ok = false;
    if constexpr (HINT) {
        R = launch_regs(a, lane);
        P = R.ok ? R.P : prefix_head(a, lane);
    }
    int32_t i = i0, Wseq = W, Wr = 0;
    if (HINT && P.on) {
        // this wave's run in the rows' split or in the sequences'
        const int64_t Th = R.ok ? (int64_t)R.Th : head_tiles(a, lane, 0, P).per_head;
        Wr = row_runs(a, P, Th, W);
        const int32_t per = W / kXcds, rx = Wr / kXcds;
        const int32_t x = i0 / per, loc = i0 - x * per;
        if (loc < rx) {
            decode_rows<QT, KT, D>(a, lane, x * rx + loc, Wr, P, R);
            return;
        }
        i = x * (per - rx) + (loc - rx);
        Wseq = W - Wr;
    }

    // T, the number of runs (never more than units), and the segment holding
    // this wave's first unit
    const RunStart rs = HINT && R.ok ? run_start_regs(a, R, i, Wseq) : run_start(a, lane, i, Wseq, P);
    if (i >= rs.runs)
        return;
    const int64_t x1 = rs.x1;
    SegPos pos = rs.pos;

    // The run's units [x0, x1) meet each segment's start charge and tiles in
    // turn; a piece of tiles is a range to decode (a run may begin or end
    // inside a start charge, which holds nothing to read).
    using Wv = MfmaWave<QT, KT, D>;
    Wv wv(lane);
    Stage st(&stage_lds[wave][0], a.stage_bytes);
    int64_t x = rs.x0;
    while (x < x1) {
        // the sequence's tiles past the ones its prefix row reads
        const int32_t nb = tiles_of(pos.n) - pos.own;
        const int64_t r0 = pos.first_tile + seq_cost(P); // tile pos.own
        const int64_t lo = max(x, r0), hi = min(x1, r0 + nb);
        if (hi > lo) {
            const int32_t j = (int32_t)(lo - r0) + pos.own;
            const int32_t je = (int32_t)(hi - r0) + pos.own;
            // with prefix rows, the run holding the segment's first own tile
            // records where the merge finds all its parts; the plan entries
            // that takes load here, while the piece's tiles do
            const bool record = HINT && a.prefix && j == pos.own;
            int32_t grp_raw = 0, rank_raw = 0;
            if (record && pos.own > 0) {
                grp_raw = uniform_load(plan_group(a) + pos.b);
                rank_raw = uniform_load(plan_rank(a) + pos.b);
            }
            wv.start(a, pos.b, pos.g);
            typename Wv::PendingToken tok;
            const bool ok = wv.template run<HINT>(a, pos.b, pos.g, j * kTile,
                                                  min(je * kTile, pos.n), pos.n, tok);
            // The results of every piece but the run's last go to the run's
            // Stage when they fit (no tile comes after the last piece to wait
            // for its stores); the branches keep every pointer's address
            // space known.
            if (HINT && r0 + nb >= x1)
                st.close();
            if (HINT && tok.put && st.fits(lane, Wv::ROW_BYTES, D * Wv::KE)) {
                wv.put_token_k(st.image(lane, Wv::token_k_row(a, tok, pos.g), Wv::ROW_BYTES),
                               tok.nt);
                wv.put_token_v(st.image_v(lane, Wv::token_v_tile(a, tok, pos.g), Wv::KE,
                                          tok.off % kTile, D * Wv::KE),
                               tok.nt);
            } else {
                wv.store_pending(a, tok, pos.g);
            }
            wv.finish();
            if (j == 0 && je == tiles_of(pos.n)) {
                typename Wv::TQ *o = Wv::out_rows(a, pos.b, pos.g);
                const int32_t bytes = a.group * D * (int32_t)sizeof(typename Wv::TQ);
                if (HINT && st.fits(lane, bytes))
                    wv.put_out(reinterpret_cast<typename Wv::TQ *>(st.image(lane, o, bytes)), a, ok);
                else
                    wv.put_out(o, a, ok);
            } else {
                const int64_t slot = balanced_slot(a, i, pos.g, pos.b);
                float *ml = ws_ml(a, slot, 0), *accp = ws_acc(a, slot, 0, D);
                if (HINT && st.fits(lane, 8 * a.group))
                    wv.put_ml(reinterpret_cast<float *>(st.image(lane, ml, 8 * a.group)), a, ok);
                else
                    wv.put_ml(ml, a, ok);
                if (HINT && st.fits(lane, 4 * D * a.group))
                    wv.put_acc(reinterpret_cast<float *>(st.image(lane, accp, 4 * D * a.group)), a,
                               ok);
                else
                    wv.put_acc(accp, a, ok);
            }
            if (record) {
                const SegLists e = segment_lists(a, lane, pos.b, pos.g, pos.n, pos.own, r0,
                                                 rs.T, rs.runs, Wr, P, R, grp_raw, rank_raw);
                const u32x4 ev = {(uint32_t)e.seq_w0, (uint32_t)e.seq_n, (uint32_t)e.row_w0,
                                  (uint32_t)e.row_n};
                int32_t *dst = seg_dir_entry(a, pos.g, pos.b);
                if (HINT && st.fits(lane, 16)) {
                    u32x4 *img = reinterpret_cast<u32x4 *>(st.image(lane, dst, 16));
                    if (lane == 0)
                        *img = ev;
                } else if (lane == 0) {
                    *reinterpret_cast<u32x4 *>(dst) = ev;
                }
            }
        }
        x = r0 + nb;
        if (x < x1)
            pos = next_segment(a, pos, P);
    }
    if constexpr (HINT)
        st.flush(lane);
}

// Static LDS of the balanced kernel: the table prefetch's sink and, with a
// share plan, the four waves' Stage areas.
constexpr int balanced_static_lds(bool hint)
{
    return (int)sizeof(u32x4) * 4 * (kWave + (hint ? kStageQuads : 1));
}

// LDS bytes the balanced kernel's launch asks for beyond its static arrays,
// and never uses: enough that the workgroup holds just over half of a CU's
// LDS, so that a CU holds one 256-thread workgroup, one wave per SIMD (0 if
// the device cannot grant that much to one workgroup).
// Measured on MI355X: a CU's memory requests are served oldest wave first, so
// a second or third wave per SIMD adds no bandwidth; it only waits, then
// runs as a later generation, which lengthens the tail and cuts the tiles
// into more runs (more partial states to merge).  With one wave per SIMD the
// config-2 step went from 72.0 to 69.9 us, the config-5 one from 236.7 to
// 219.1 us.
static int balanced_lds_bytes(bool hint)
{
    static std::mutex mu;
    static std::map<int, int> cache[2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache[hint].find(dev);
    if (it != cache[hint].end())
        return it->second;
    int per_cu = 0, per_block = 0;
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
        return 0;
    int want = per_cu / 2 + 1024;
    want = want > per_block ? 0 : max(0, want - balanced_static_lds(hint));
    cache[hint][dev] = want;
    return want;
}

template <int QT, int KT, int D>
hipError_t launch_mfma(const DecodeArgs &a, int32_t num_items, hipStream_t stream)
{
    const int grid = (num_items + 3) / 4;
    const bool hint = a.share != nullptr;
    if (a.partition == kPartitionBalanced) {
        auto kern = hint ? &decode_mfma_balanced_kernel<QT, KT, D, true>
                         : &decode_mfma_balanced_kernel<QT, KT, D, false>;
        DecodeArgs b = a;
        b.stage_bytes = hint ? (int32_t)sizeof(u32x4) * kStageQuads : 0;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), balanced_lds_bytes(hint), stream, b,
                           num_items);
    } else {
        auto kern =
            hint ? &decode_mfma_kernel<QT, KT, D, true> : &decode_mfma_kernel<QT, KT, D, false>;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, a, num_items);
    }
    return hipGetLastError();
}

// Waves of the balanced kernel one CU holds at once (with its LDS request).
template <int QT, int KT, int D>
int mfma_balanced_waves_per_cu()
{
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks,
            reinterpret_cast<const void *>(&decode_mfma_balanced_kernel<QT, KT, D, false>), 256,
            balanced_lds_bytes(false)) != hipSuccess)
        return 0;
    return blocks * 4;
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

int mfma_waves_per_cu(pa_dtype qt, pa_dtype kt, int D)
{
#define PA_W(Q, K)                                                                                 \
    if (qt == Q && kt == K)                                                                        \
        return D == 64 ? mfma_balanced_waves_per_cu<Q, K, 64>()                                    \
                       : mfma_balanced_waves_per_cu<Q, K, 128>();
    PA_W(PA_BF16, PA_BF16)
    PA_W(PA_F16, PA_F16)
    PA_W(PA_BF16, PA_FP8_E4M3)
    PA_W(PA_F16, PA_FP8_E4M3)
#undef PA_W
    return 0;
}

bool mfma_supports(pa_dtype qt, pa_dtype kt, int D, int G)
{
    const bool dt = (qt == PA_BF16 || qt == PA_F16) && (kt == qt || kt == PA_FP8_E4M3);
    return dt && (D == 64 || D == 128) && G >= 1 && G <= 16;
}

} // namespace pa
