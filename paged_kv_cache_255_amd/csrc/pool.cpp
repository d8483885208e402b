// Host-side block pool: free list, per-sequence block tables, reference
// counts.  Pure C++17, no HIP; it is what a serving scheduler calls once per
// decode step to get each new token's slot (pa.h documents every call).
//
// [devto] dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
//         PagedAttention Fixes It", §4 (block pool, block tables, on-demand
//         allocation) and §5 (shared blocks with reference counts; a
//         branch's first write goes to a private block: copy on write).
// [hi]    hyperinfer.ai, "KV cache & paged attention deep dive" (free pool,
//         eviction frees a sequence's blocks).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.hpp"

// Identity of a cached full block ([devto] §5 "Automatic Prefix Caching":
// a table of physical blocks looked up by their tokens): the cached block
// that holds the block_size tokens before it (-1 for a sequence's first
// block) and its own block_size token ids.  Chaining by the parent's physical
// id makes equal keys mean equal whole prefixes, and equality is exact (no
// lossy hash).
struct BlockKey {
    int32_t parent;
    std::vector<int32_t> tokens;
    bool operator==(const BlockKey &o) const { return parent == o.parent && tokens == o.tokens; }
};

struct BlockKeyHash {
    size_t operator()(const BlockKey &k) const
    {
        uint64_t h = 0x243F6A8885A308D3ull ^ (uint32_t)k.parent;
        for (int32_t t : k.tokens) {
            h ^= (uint32_t)t;
            h *= 0x9E3779B97F4A7C15ull;
            h ^= h >> 29;
        }
        return (size_t)h;
    }
};

struct pa_pool {
    pa_pool_config cfg{};
    std::vector<int32_t> free_list; // taken from and returned to the back
    std::vector<int32_t> refcount;  // per physical block
    // Export scratch: per block, how many of the exported tables hold it
    // (all zero between calls).
    mutable std::vector<int32_t> batch_count;
    struct Seq {
        bool live = false;
        bool swapped = false; // blocks holds host block ids
        int32_t len = 0;      // positions appended so far
        int32_t start = 0;    // first position of the window
        int32_t dropped = 0;  // leading blocks the window released; blocks[0] is
                              // logical block `dropped`
        std::vector<int32_t> blocks;
    };
    std::vector<Seq> seqs; // index = sequence id
    // Copy on write: (src, dst) block copies made by appends and not yet
    // handed out (pa_pool_take_copies), in the order they were made; and
    // blocks whose last reference went while a pending copy still reads them
    // (they join the free list when the copies are handed out).
    std::vector<std::pair<int32_t, int32_t>> copies;
    std::vector<int32_t> held;
    // Prefix cache: key -> block, and per cached block its key, when it was
    // last registered or matched, and how many cached keys name it as parent.
    // The cache holds one reference on each of its blocks.
    struct Cached {
        BlockKey key;
        uint64_t last_use;
        int32_t children;
    };
    std::unordered_map<BlockKey, int32_t, BlockKeyHash> prefix;
    std::unordered_map<int32_t, Cached> cached;
    uint64_t tick = 0;
    // Host swap space: free host block ids, taken from and returned to the back.
    std::vector<int32_t> host_free;
};

namespace {

// splitmix64 (Steele, Lea, Flood, OOPSLA 2014).
struct SplitMix64 {
    uint64_t s;
    uint64_t next()
    {
        s += 0x9E3779B97F4A7C15ull;
        uint64_t z = s;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

pa_pool::Seq *live_seq(pa_pool *p, int32_t id)
{
    if (!p || id < 0 || (size_t)id >= p->seqs.size() || !p->seqs[id].live)
        return nullptr;
    return &p->seqs[id];
}

const pa_pool::Seq *live_seq(const pa_pool *p, int32_t id)
{
    return live_seq(const_cast<pa_pool *>(p), id);
}

// A live sequence whose blocks are on the device (not swapped out).
pa_pool::Seq *resident_seq(pa_pool *p, int32_t id)
{
    pa_pool::Seq *s = live_seq(p, id);
    return (s && !s->swapped) ? s : nullptr;
}

const pa_pool::Seq *resident_seq(const pa_pool *p, int32_t id)
{
    return resident_seq(const_cast<pa_pool *>(p), id);
}

// Whether an append of ntok tokens to `s` writes into a partly filled last
// block that another table also maps ([devto] §5 "Zero-Copy Forking": a
// branch's first new token goes to a private block; copy on write).
bool needs_copy(const pa_pool *p, const pa_pool::Seq &s, int32_t ntok)
{
    return ntok > 0 && s.len % p->cfg.block_size != 0 && p->refcount[s.blocks.back()] > 1;
}

// New blocks `s` needs for ntok more tokens (a private copy of a shared last
// block counts as one).
pa_status check_append(const pa_pool *p, const pa_pool::Seq &s, int32_t ntok, int32_t *need)
{
    const int32_t bs = p->cfg.block_size;
    int64_t total = (int64_t)s.len + ntok;
    if (total > INT32_MAX)
        return pa::fail(PA_ERR_INVALID_ARG, "sequence length overflows int32");
    *need = blocks_for(total, bs) - s.dropped - (int32_t)s.blocks.size() +
            (needs_copy(p, s, ntok) ? 1 : 0);
    return PA_OK;
}

// Drops one reference to block b; at zero it goes back to the free list, or
// is held while a pending copy still reads it.  A pending copy into b is
// dropped (nothing maps b any more).
void release_block(pa_pool *p, int32_t b)
{
    if (--p->refcount[b] != 0)
        return;
    auto &c = p->copies;
    c.erase(std::remove_if(c.begin(), c.end(), [b](const std::pair<int32_t, int32_t> &e) {
                return e.second == b;
            }),
            c.end());
    for (const auto &e : c)
        if (e.first == b) {
            p->held.push_back(b);
            return;
        }
    p->free_list.push_back(b);
}

void do_append(pa_pool *p, pa_pool::Seq &s, int32_t ntok, int32_t *slots)
{
    const int32_t bs = p->cfg.block_size;
    if (needs_copy(p, s, ntok)) {
        // the private copy is taken first: pop, map it in place of the
        // shared block, remember the copy the device must make
        const int32_t shared = s.blocks.back();
        const int32_t mine = p->free_list.back();
        p->free_list.pop_back();
        p->refcount[mine] = 1;
        s.blocks.back() = mine;
        p->copies.emplace_back(shared, mine);
        release_block(p, shared); // refcount > 1: never reaches zero here
    }
    const int32_t need =
        blocks_for((int64_t)s.len + ntok, bs) - s.dropped - (int32_t)s.blocks.size();
    for (int32_t i = 0; i < need; ++i) {
        int32_t b = p->free_list.back();
        p->free_list.pop_back();
        p->refcount[b] = 1;
        s.blocks.push_back(b);
    }
    for (int32_t i = 0; i < ntok; ++i) {
        int32_t pos = s.len + i;
        if (slots)
            slots[i] = s.blocks[pos / bs - s.dropped] * bs + pos % bs;
    }
    s.len += ntok;
}

} // namespace

extern "C" {

pa_status pa_block_pool_init(const pa_pool_config *cfg, pa_pool **out)
{
    if (!cfg || !out)
        return pa::fail(PA_ERR_INVALID_ARG, "null argument");
    *out = nullptr;
    if (cfg->num_blocks <= 0 || cfg->block_size <= 0 || cfg->num_layers <= 0 ||
        cfg->num_kv_heads <= 0 || cfg->head_dim <= 0 || cfg->num_host_blocks < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "pool sizes must be positive");
    if (pa::dtype_bytes(cfg->kv_dtype) == 0)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown kv dtype");
    if (cfg->block_size != 16 && cfg->block_size != 32 && cfg->block_size != 64 &&
        cfg->block_size != 128 && cfg->block_size != 256)
        return pa::fail(PA_ERR_UNSUPPORTED, "block_size must be 16, 32, 64, 128 or 256");
    if ((int64_t)cfg->num_blocks * cfg->block_size > INT32_MAX)
        return pa::fail(PA_ERR_INVALID_ARG, "num_blocks * block_size overflows int32 slots");
    pa_pool *p = new (std::nothrow) pa_pool();
    if (!p)
        return pa::fail(PA_ERR_INVALID_ARG, "out of host memory");
    p->cfg = *cfg;
    p->free_list.resize(cfg->num_blocks);
    for (int32_t i = 0; i < cfg->num_blocks; ++i)
        p->free_list[i] = i;
    if (cfg->shuffle_seed != 0) {
        SplitMix64 rng{cfg->shuffle_seed};
        for (int64_t i = cfg->num_blocks - 1; i > 0; --i) {
            uint64_t j = rng.next() % (uint64_t)(i + 1);
            std::swap(p->free_list[i], p->free_list[j]);
        }
    }
    p->refcount.assign(cfg->num_blocks, 0);
    p->host_free.resize(cfg->num_host_blocks);
    for (int32_t i = 0; i < cfg->num_host_blocks; ++i)
        p->host_free[i] = i;
    *out = p;
    return PA_OK;
}

void pa_block_pool_destroy(pa_pool *pool) { delete pool; }

uint64_t pa_kv_bytes_per_token(const pa_pool *p)
{
    if (!p)
        return 0;
    return 2ull * (uint64_t)p->cfg.num_layers * (uint64_t)p->cfg.num_kv_heads *
           (uint64_t)p->cfg.head_dim * (uint64_t)pa::dtype_bytes(p->cfg.kv_dtype);
}

uint64_t pa_block_bytes(const pa_pool *p)
{
    if (!p)
        return 0;
    return (uint64_t)p->cfg.block_size * (uint64_t)p->cfg.num_kv_heads *
           (uint64_t)p->cfg.head_dim * (uint64_t)pa::dtype_bytes(p->cfg.kv_dtype);
}

pa_status pa_seq_create(pa_pool *p, int32_t *seq_out)
{
    if (!p || !seq_out)
        return pa::fail(PA_ERR_INVALID_ARG, "null argument");
    if (p->seqs.size() >= (size_t)INT32_MAX)
        return pa::fail(PA_ERR_CAPACITY, "sequence ids exhausted");
    p->seqs.emplace_back();
    p->seqs.back().live = true;
    *seq_out = (int32_t)(p->seqs.size() - 1);
    return PA_OK;
}

pa_status pa_seq_append_slots(pa_pool *p, int32_t seq, int32_t ntok, int32_t *slots_out)
{
    pa_pool::Seq *s = resident_seq(p, seq);
    if (!s)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown, freed or swapped-out sequence id");
    if (ntok < 0 || (ntok > 0 && !slots_out))
        return pa::fail(PA_ERR_INVALID_ARG, "bad token count or null slots_out");
    int32_t need = 0;
    pa_status st = check_append(p, *s, ntok, &need);
    if (st != PA_OK)
        return st;
    if ((size_t)need > p->free_list.size())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "block pool exhausted");
    do_append(p, *s, ntok, slots_out);
    return PA_OK;
}

pa_status pa_seq_append_slots_batch(pa_pool *p, const int32_t *seqs, int32_t nseq, int32_t ntok,
                                    int32_t *slots_out)
{
    if (!p || nseq < 0 || ntok < 0 || (nseq > 0 && !seqs) || (nseq > 0 && ntok > 0 && !slots_out))
        return pa::fail(PA_ERR_INVALID_ARG, "bad batch arguments");
    std::vector<int32_t> sorted(seqs, seqs + nseq);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
        return pa::fail(PA_ERR_INVALID_ARG, "sequence repeated in batch");
    int64_t total = 0;
    for (int32_t i = 0; i < nseq; ++i) {
        pa_pool::Seq *s = resident_seq(p, seqs[i]);
        if (!s)
            return pa::fail(PA_ERR_INVALID_ARG,
                            "unknown, freed or swapped-out sequence id in batch");
        int32_t need = 0;
        pa_status st = check_append(p, *s, ntok, &need);
        if (st != PA_OK)
            return st;
        total += need;
    }
    if ((size_t)total > p->free_list.size())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "block pool exhausted");
    for (int32_t i = 0; i < nseq; ++i)
        do_append(p, p->seqs[seqs[i]], ntok, slots_out ? slots_out + (size_t)i * ntok : nullptr);
    return PA_OK;
}

pa_status pa_seq_fork(pa_pool *p, int32_t parent, int32_t *child_out)
{
    if (!child_out || !resident_seq(p, parent))
        return pa::fail(PA_ERR_INVALID_ARG, "unknown or swapped-out parent, or null child_out");
    int32_t child;
    pa_status st = pa_seq_create(p, &child);
    if (st != PA_OK)
        return st;
    pa_pool::Seq &par = p->seqs[parent];
    pa_pool::Seq &c = p->seqs[child];
    c.blocks = par.blocks;
    c.len = par.len;
    c.start = par.start;
    c.dropped = par.dropped;
    for (int32_t b : c.blocks)
        ++p->refcount[b];
    *child_out = child;
    return PA_OK;
}

pa_status pa_seq_free(pa_pool *p, int32_t seq)
{
    pa_pool::Seq *s = live_seq(p, seq);
    if (!s)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown or already freed sequence id");
    if (s->swapped) {
        for (int32_t h : s->blocks)
            p->host_free.push_back(h);
    } else {
        for (int32_t b : s->blocks)
            release_block(p, b);
    }
    s->blocks.clear();
    s->blocks.shrink_to_fit();
    s->len = s->start = s->dropped = 0;
    s->swapped = false;
    s->live = false;
    return PA_OK;
}

pa_status pa_seq_slide_window(pa_pool *p, int32_t seq, int32_t window, int32_t *released_out)
{
    pa_pool::Seq *s = resident_seq(p, seq);
    if (!s || window < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown or swapped-out sequence, or window < 0");
    const int32_t bs = p->cfg.block_size;
    s->start = std::max(s->start, s->len - window);
    int32_t released = 0;
    size_t k = 0; // leading blocks wholly before the start
    while (k < s->blocks.size() && (int64_t)s->start - (int64_t)(s->dropped + k) * bs >= bs)
        ++k;
    for (size_t i = 0; i < k; ++i) {
        release_block(p, s->blocks[i]);
        ++released;
    }
    s->blocks.erase(s->blocks.begin(), s->blocks.begin() + k);
    s->dropped += (int32_t)k;
    if (released_out)
        *released_out = released;
    return PA_OK;
}

pa_status pa_seq_swap_out(pa_pool *p, int32_t seq, int32_t *pairs_out, int32_t max_pairs,
                          int32_t *count_out)
{
    pa_pool::Seq *s = resident_seq(p, seq);
    if (!s || !count_out || max_pairs < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown or swapped-out sequence, or bad arguments");
    if (!p->copies.empty())
        return pa::fail(PA_ERR_INVALID_ARG,
                        "copy-on-write copies are pending: take and make them first");
    const size_t n = s->blocks.size();
    *count_out = (int32_t)n;
    if (n > p->host_free.size())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "host swap space exhausted");
    if (n > 0 && (!pairs_out || (size_t)max_pairs < n))
        return pa::fail(PA_ERR_CAPACITY, "more blocks than max_pairs");
    std::vector<int32_t> host(n);
    for (size_t i = 0; i < n; ++i) {
        host[i] = p->host_free.back();
        p->host_free.pop_back();
        pairs_out[2 * i] = s->blocks[i];
        pairs_out[2 * i + 1] = host[i];
    }
    for (int32_t b : s->blocks)
        release_block(p, b);
    s->blocks = std::move(host);
    s->swapped = true;
    return PA_OK;
}

pa_status pa_seq_swap_in(pa_pool *p, int32_t seq, int32_t *pairs_out, int32_t max_pairs,
                         int32_t *count_out)
{
    pa_pool::Seq *s = live_seq(p, seq);
    if (!s || !s->swapped || !count_out || max_pairs < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "sequence not swapped out, or bad arguments");
    const size_t n = s->blocks.size();
    *count_out = (int32_t)n;
    if (n > p->free_list.size())
        return pa::fail(PA_ERR_OUT_OF_BLOCKS, "block pool exhausted");
    if (n > 0 && (!pairs_out || (size_t)max_pairs < n))
        return pa::fail(PA_ERR_CAPACITY, "more blocks than max_pairs");
    std::vector<int32_t> dev(n);
    for (size_t i = 0; i < n; ++i) {
        dev[i] = p->free_list.back();
        p->free_list.pop_back();
        p->refcount[dev[i]] = 1;
        pairs_out[2 * i] = s->blocks[i];
        pairs_out[2 * i + 1] = dev[i];
    }
    for (int32_t h : s->blocks)
        p->host_free.push_back(h);
    s->blocks = std::move(dev);
    s->swapped = false;
    return PA_OK;
}

pa_status pa_seq_length(const pa_pool *p, int32_t seq, int32_t *len_out)
{
    const pa_pool::Seq *s = live_seq(p, seq);
    if (!s || !len_out)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown sequence or null len_out");
    *len_out = s->len;
    return PA_OK;
}

pa_status pa_block_refcount(const pa_pool *p, int32_t block, int32_t *refcount_out)
{
    if (!p || !refcount_out || block < 0 || block >= p->cfg.num_blocks)
        return pa::fail(PA_ERR_INVALID_ARG, "bad block id or null output");
    *refcount_out = p->refcount[block];
    return PA_OK;
}

pa_status pa_export_block_tables(const pa_pool *p, const int32_t *seqs, int32_t nseq,
                                 int32_t max_blocks, int32_t *tables_out, int32_t *lens_out,
                                 int32_t *starts_out, int32_t *shared_out)
{
    if (!p || nseq < 0 || max_blocks < 0 || (nseq > 0 && !seqs))
        return pa::fail(PA_ERR_INVALID_ARG, "bad export arguments");
    for (int32_t i = 0; i < nseq; ++i) {
        const pa_pool::Seq *s = resident_seq(p, seqs[i]);
        if (!s)
            return pa::fail(PA_ERR_INVALID_ARG, "unknown or swapped-out sequence id in export");
        if (tables_out && s->blocks.size() > (size_t)max_blocks)
            return pa::fail(PA_ERR_CAPACITY, "block table longer than max_blocks");
    }
    for (int32_t i = 0; i < nseq; ++i) {
        const pa_pool::Seq &s = p->seqs[seqs[i]];
        if (tables_out) {
            int32_t *row = tables_out + (size_t)i * max_blocks;
            const size_t n = s.blocks.size();
            if (n)
                std::memcpy(row, s.blocks.data(), n * sizeof(int32_t));
            std::fill(row + n, row + max_blocks, -1);
        }
        const int32_t base = s.dropped * p->cfg.block_size; // first kept position
        if (lens_out)
            lens_out[i] = s.len - base;
        if (starts_out)
            starts_out[i] = s.start - base;
    }
    if (shared_out) {
        // leading table entries whose block another exported table also holds
        std::vector<int32_t> &cnt = p->batch_count;
        if (cnt.size() != (size_t)p->cfg.num_blocks)
            cnt.assign(p->cfg.num_blocks, 0);
        for (int32_t i = 0; i < nseq; ++i)
            for (int32_t b : p->seqs[seqs[i]].blocks)
                ++cnt[b];
        for (int32_t i = 0; i < nseq; ++i) {
            const std::vector<int32_t> &bl = p->seqs[seqs[i]].blocks;
            size_t k = 0;
            while (k < bl.size() && cnt[bl[k]] > 1)
                ++k;
            shared_out[i] = (int32_t)k;
        }
        for (int32_t i = 0; i < nseq; ++i)
            for (int32_t b : p->seqs[seqs[i]].blocks)
                cnt[b] = 0;
    }
    return PA_OK;
}

pa_status pa_export_share_plan(const pa_pool *p, const int32_t *seqs, int32_t nseq,
                               int32_t *plan_out)
{
    if (!p || nseq < 0 || (nseq > 0 && (!seqs || !plan_out)))
        return pa::fail(PA_ERR_INVALID_ARG, "bad share-plan arguments");
    for (int32_t i = 0; i < nseq; ++i)
        if (!resident_seq(p, seqs[i]))
            return pa::fail(PA_ERR_INVALID_ARG, "unknown or swapped-out sequence id in export");
    if (nseq == 0)
        return PA_OK;
    const int32_t B = nseq;
    const int32_t bs = p->cfg.block_size;
    int32_t *shared = plan_out + 2;
    int32_t *group_of = plan_out + 2 + B;
    int32_t *rank = plan_out + 2 + 2 * B;
    int32_t *own = plan_out + 2 + 3 * B;
    int32_t *gcount = plan_out + 2 + 4 * B;
    int32_t *gblocks = plan_out + 2 + 5 * B;
    int32_t *members = plan_out + 2 + 6 * B;
    int32_t *gfirst = plan_out + 2 + 7 * B;
    std::fill(plan_out, plan_out + PA_SHARE_PLAN_WORDS(B), 0);
    plan_out[0] = PA_SHARE_PLAN_MAGIC;
    // the hint: leading entries whose block another exported table holds
    pa_status st = pa_export_block_tables(p, seqs, nseq, 0, nullptr, nullptr, nullptr, shared);
    if (st != PA_OK)
        return st;
    std::fill(group_of, group_of + B, -1);
    // candidates: no window, first entry shared; keyed by the first block,
    // in order of their first member
    std::vector<int32_t> first_of_key(p->cfg.num_blocks, -1);
    std::vector<std::vector<int32_t>> sets;
    for (int32_t i = 0; i < B; ++i) {
        const pa_pool::Seq &q = p->seqs[seqs[i]];
        if (q.dropped != 0 || q.start != 0 || q.blocks.empty() || shared[i] < 1 || q.len <= bs)
            continue;
        const int32_t key = q.blocks[0];
        if (first_of_key[key] < 0) {
            first_of_key[key] = (int32_t)sets.size();
            sets.emplace_back();
        }
        sets[first_of_key[key]].push_back(i);
    }
    int32_t ngroups = 0, placed = 0;
    for (const std::vector<int32_t> &m : sets) {
        if (m.size() < 2)
            continue;
        // the longest run of leading entries every member holds alike, all
        // before each member's last token (its block stays its own)
        size_t k = SIZE_MAX;
        for (int32_t i : m)
            k = std::min(k, (size_t)((p->seqs[seqs[i]].len - 1) / bs));
        const std::vector<int32_t> &lead = p->seqs[seqs[m[0]]].blocks;
        size_t j = 0;
        for (; j < k; ++j) {
            bool same = true;
            for (int32_t i : m)
                same = same && p->seqs[seqs[i]].blocks[j] == lead[j];
            if (!same)
                break;
        }
        if (j == 0)
            continue;
        gcount[ngroups] = (int32_t)m.size();
        gblocks[ngroups] = (int32_t)j;
        gfirst[ngroups] = placed;
        for (size_t r = 0; r < m.size(); ++r) {
            group_of[m[r]] = ngroups;
            rank[m[r]] = (int32_t)r;
            own[m[r]] = (int32_t)j;
            members[placed++] = m[r];
        }
        ++ngroups;
    }
    plan_out[1] = ngroups;
    return PA_OK;
}

pa_status pa_pool_take_copies(pa_pool *p, int32_t *pairs_out, int32_t max_pairs,
                              int32_t *count_out)
{
    if (!p || !count_out || max_pairs < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "bad arguments");
    const size_t n = p->copies.size();
    *count_out = (int32_t)n;
    if (n == 0)
        return PA_OK;
    if (!pairs_out || (size_t)max_pairs < n)
        return pa::fail(PA_ERR_CAPACITY, "more pending copies than max_pairs");
    for (size_t i = 0; i < n; ++i) {
        pairs_out[2 * i] = p->copies[i].first;
        pairs_out[2 * i + 1] = p->copies[i].second;
    }
    p->copies.clear();
    for (int32_t b : p->held)
        p->free_list.push_back(b);
    p->held.clear();
    return PA_OK;
}

pa_status pa_prefix_register(pa_pool *p, int32_t seq, const int32_t *tokens, int32_t ntok,
                             int32_t *added_out)
{
    pa_pool::Seq *s = resident_seq(p, seq);
    if (!s)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown, freed or swapped-out sequence id");
    if (ntok < 0 || ntok > s->len || (ntok > 0 && !tokens))
        return pa::fail(PA_ERR_INVALID_ARG, "ntok must be in [0, sequence length]");
    if (s->start != 0 || s->dropped != 0)
        return pa::fail(PA_ERR_INVALID_ARG, "the sequence's window has moved: no prefix left");
    const int32_t bs = p->cfg.block_size;
    int32_t added = 0, prev = -1;
    for (int32_t i = 0; i < ntok / bs; ++i) {
        BlockKey key;
        key.parent = prev;
        key.tokens.assign(tokens + (size_t)i * bs, tokens + (size_t)(i + 1) * bs);
        auto it = p->prefix.find(key);
        if (it != p->prefix.end()) {
            prev = it->second;
            p->cached[prev].last_use = ++p->tick;
            continue;
        }
        const int32_t b = s->blocks[i];
        if (p->cached.count(b))
            break; // cached under other tokens: not this prefix's block
        p->prefix.emplace(key, b);
        p->cached[b] = pa_pool::Cached{key, ++p->tick, 0};
        ++p->refcount[b];
        if (prev >= 0)
            ++p->cached[prev].children;
        prev = b;
        ++added;
    }
    if (added_out)
        *added_out = added;
    return PA_OK;
}

pa_status pa_prefix_match(pa_pool *p, int32_t seq, const int32_t *tokens, int32_t ntok,
                          int32_t *matched_out)
{
    pa_pool::Seq *s = resident_seq(p, seq);
    if (!s || !matched_out)
        return pa::fail(PA_ERR_INVALID_ARG, "unknown sequence or null matched_out");
    if (s->len != 0)
        return pa::fail(PA_ERR_INVALID_ARG, "prefix matching needs an empty sequence");
    if (ntok < 0 || (ntok > 0 && !tokens))
        return pa::fail(PA_ERR_INVALID_ARG, "bad tokens");
    const int32_t bs = p->cfg.block_size;
    int32_t prev = -1, n = 0;
    for (int32_t i = 0; i < ntok / bs; ++i) {
        BlockKey key;
        key.parent = prev;
        key.tokens.assign(tokens + (size_t)i * bs, tokens + (size_t)(i + 1) * bs);
        auto it = p->prefix.find(key);
        if (it == p->prefix.end())
            break;
        prev = it->second;
        p->cached[prev].last_use = ++p->tick;
        ++p->refcount[prev];
        s->blocks.push_back(prev);
        ++n;
    }
    s->len = n * bs;
    *matched_out = n * bs;
    return PA_OK;
}

pa_status pa_prefix_evict(pa_pool *p, int32_t max_blocks, int32_t *evicted_out)
{
    if (!p || max_blocks < 0)
        return pa::fail(PA_ERR_INVALID_ARG, "bad arguments");
    int32_t n = 0;
    while (n < max_blocks) {
        // the least recently used cached block that only the cache maps and
        // that no cached key names as parent (ties: lower block id)
        int32_t best = -1;
        uint64_t best_use = 0;
        for (const auto &e : p->cached) {
            if (p->refcount[e.first] != 1 || e.second.children != 0)
                continue;
            if (best < 0 || e.second.last_use < best_use ||
                (e.second.last_use == best_use && e.first < best)) {
                best = e.first;
                best_use = e.second.last_use;
            }
        }
        if (best < 0)
            break;
        const BlockKey key = p->cached[best].key;
        p->prefix.erase(key);
        if (key.parent >= 0)
            --p->cached[key.parent].children;
        p->cached.erase(best);
        release_block(p, best);
        ++n;
    }
    if (evicted_out)
        *evicted_out = n;
    return PA_OK;
}

pa_status pa_pool_get_stats(const pa_pool *p, pa_pool_stats *out)
{
    if (!p || !out)
        return pa::fail(PA_ERR_INVALID_ARG, "null argument");
    pa_pool_stats st{};
    st.num_blocks = p->cfg.num_blocks;
    st.free_blocks = (int32_t)p->free_list.size();
    st.used_blocks = st.num_blocks - st.free_blocks;
    for (int32_t r : p->refcount)
        st.shared_blocks += (r > 1);
    st.cached_blocks = (int32_t)p->cached.size();
    st.free_host_blocks = (int32_t)p->host_free.size();
    for (const auto &s : p->seqs) {
        if (!s.live)
            continue;
        ++st.live_seqs;
        st.logical_tokens += s.len - s.start;
        if (s.swapped) {
            ++st.swapped_seqs;
            continue;
        }
        st.mapped_blocks += (int64_t)s.blocks.size();
        st.tail_slack_tokens +=
            ((int64_t)s.dropped + (int64_t)s.blocks.size()) * p->cfg.block_size - s.len;
    }
    *out = st;
    return PA_OK;
}

} // extern "C"
