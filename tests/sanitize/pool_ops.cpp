// Seeded random operation streams through the host block pool's C API, for a
// build of pool.cpp under AddressSanitizer and UndefinedBehaviorSanitizer.
// Every call of the pool API is made, including the error paths, and after
// each operation the pool's counts are checked against what its own exports
// say:
//   used + free = num_blocks, where used counts the blocks with references
//   and, while copies are queued, the blocks they still read,
//   sum of refcounts = blocks mapped by resident tables + blocks cached,
//   each exported table holds ceil(len / block_size) ids, all in range,
//   a block a table maps has a reference count of at least its mappings.
// Exit status 0 when every check holds; the sanitizers abort on a fault.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa.h"

namespace {

uint64_t g_state;
uint32_t rnd(uint32_t n)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33) % (n ? n : 1);
}

int g_fail = 0;
void check(bool ok, const char *what, int step)
{
    if (!ok && g_fail < 20) {
        std::fprintf(stderr, "step %d: %s\n", step, what);
        ++g_fail;
    }
}

struct Seq {
    int32_t id;
    bool swapped;
    bool windowed;
};

void run(int32_t NB, int32_t bs, int32_t host_blocks, uint64_t seed, int steps)
{
    g_state = seed;
    pa_pool_config cfg{NB, bs, 2, 4, 64, PA_BF16, seed, host_blocks};
    pa_pool *pool = nullptr;
    if (pa_block_pool_init(&cfg, &pool) != PA_OK) {
        check(false, "pool init", 0);
        return;
    }
    std::vector<Seq> seqs;
    std::vector<int32_t> buf(1 << 16), buf2(1 << 16);
    std::vector<int32_t> tokens(4096);
    for (auto &t : tokens)
        t = (int32_t)rnd(5); // few distinct ids: prefixes repeat
    for (int step = 0; step < steps; ++step) {
        const uint32_t op = rnd(13);
        const int ns = (int)seqs.size();
        Seq *s = ns ? &seqs[rnd(ns)] : nullptr;
        int32_t n = 0, id = 0;
        switch (op) {
        case 0:
            if (pa_seq_create(pool, &id) == PA_OK)
                seqs.push_back({id, false, false});
            break;
        case 1:
        case 2:
            if (s && !s->swapped)
                (void)pa_seq_append_slots(pool, s->id, (int32_t)rnd(3 * bs), buf.data());
            break;
        case 3: {
            std::vector<int32_t> batch;
            for (auto &x : seqs)
                if (!x.swapped && rnd(2))
                    batch.push_back(x.id);
            if (!batch.empty())
                (void)pa_seq_append_slots_batch(pool, batch.data(), (int32_t)batch.size(),
                                                1 + (int32_t)rnd(2), buf.data());
            break;
        }
        case 4:
            if (s && !s->swapped && pa_seq_fork(pool, s->id, &id) == PA_OK)
                seqs.push_back({id, false, s->windowed});
            break;
        case 5:
            if (s) {
                check(pa_seq_free(pool, s->id) == PA_OK, "free", step);
                seqs.erase(seqs.begin() + (s - seqs.data()));
            }
            break;
        case 6:
            if (s && !s->swapped) {
                if (pa_seq_slide_window(pool, s->id, 1 + (int32_t)rnd(4 * bs), &n) == PA_OK)
                    s->windowed = true;
            }
            break;
        case 7:
            (void)pa_pool_take_copies(pool, buf.data(), (int32_t)buf.size() / 2, &n);
            break;
        case 8:
            if (s && host_blocks > 0) {
                (void)pa_pool_take_copies(pool, buf.data(), (int32_t)buf.size() / 2, &n);
                if (!s->swapped) {
                    // asks for the count; it succeeds, and swaps, for an empty table
                    if (pa_seq_swap_out(pool, s->id, nullptr, 0, &n) == PA_OK ||
                        pa_seq_swap_out(pool, s->id, buf.data(), (int32_t)buf.size() / 2, &n) ==
                            PA_OK)
                        s->swapped = true;
                } else if (pa_seq_swap_in(pool, s->id, buf.data(), (int32_t)buf.size() / 2,
                                          &n) == PA_OK) {
                    s->swapped = false;
                }
            }
            break;
        case 9:
            if (s && !s->swapped && !s->windowed) {
                int32_t len = 0;
                (void)pa_seq_length(pool, s->id, &len);
                if (len <= (int32_t)tokens.size())
                    (void)pa_prefix_register(pool, s->id, tokens.data(), len, &n);
            }
            break;
        case 10:
            if (pa_seq_create(pool, &id) == PA_OK) {
                seqs.push_back({id, false, false});
                (void)pa_prefix_match(pool, id, tokens.data(), (int32_t)rnd(8 * bs), &n);
            }
            break;
        case 11:
            (void)pa_prefix_evict(pool, (int32_t)rnd(8), &n);
            break;
        default: {
            // invalid arguments: every call must refuse them without a fault
            (void)pa_seq_append_slots(pool, 1 << 30, 1, buf.data());
            (void)pa_seq_free(pool, -5);
            (void)pa_block_refcount(pool, NB, &n);
            (void)pa_block_refcount(pool, -1, &n);
            (void)pa_seq_fork(pool, 1 << 20, &id);
            (void)pa_export_block_tables(pool, nullptr, 0, 4, nullptr, nullptr, nullptr,
                                         nullptr);
            (void)pa_last_error();
            break;
        }
        }

        // invariants
        pa_pool_stats st{};
        check(pa_pool_get_stats(pool, &st) == PA_OK, "stats", step);
        std::vector<int32_t> res;
        for (auto &x : seqs)
            if (!x.swapped)
                res.push_back(x.id);
        int32_t maxb = 0;
        for (int32_t sid : res) {
            int32_t len = 0;
            check(pa_seq_length(pool, sid, &len) == PA_OK, "length", step);
            maxb = std::max(maxb, (len + bs - 1) / bs);
        }
        maxb = std::max(maxb, 1);
        const int nr = (int)res.size();
        std::vector<int32_t> tables((size_t)std::max(nr, 1) * maxb), lens(std::max(nr, 1)),
            starts(std::max(nr, 1)), shared(std::max(nr, 1));
        if (nr) {
            check(pa_export_block_tables(pool, res.data(), nr, maxb, tables.data(), lens.data(),
                                         starts.data(), shared.data()) == PA_OK,
                  pa_last_error(), step);
        }
        std::vector<int64_t> mapped(NB, 0);
        int64_t mapped_total = 0;
        for (int r = 0; r < nr; ++r) {
            const int32_t nb = (lens[r] + bs - 1) / bs;
            check(starts[r] >= 0 && starts[r] <= lens[r], "window start", step);
            check(shared[r] >= 0 && shared[r] <= nb, "shared count", step);
            for (int32_t j = 0; j < maxb; ++j) {
                const int32_t b = tables[(size_t)r * maxb + j];
                if (j < nb) {
                    check(b >= 0 && b < NB, "table entry in range", step);
                    if (b >= 0 && b < NB)
                        ++mapped[b];
                    ++mapped_total;
                } else {
                    check(b == -1, "padding entry", step);
                }
            }
        }
        check(mapped_total == st.mapped_blocks, "mapped blocks", step);
        int64_t refs = 0;
        int32_t used = 0;
        for (int32_t b = 0; b < NB; ++b) {
            int32_t rc = 0;
            check(pa_block_refcount(pool, b, &rc) == PA_OK, "refcount", step);
            check(rc >= mapped[b], "refcount covers mappings", step);
            refs += rc;
            used += rc > 0;
        }
        // blocks a queued copy still reads count as used until the copies go
        check(used <= st.used_blocks, "used blocks", step);
        check(st.used_blocks + st.free_blocks == NB, "used + free", step);
        check(refs == st.mapped_blocks + st.cached_blocks, "references", step);
        int32_t q = 0;
        if (pa_pool_take_copies(pool, nullptr, 0, &q) == PA_OK && q == 0)
            check(used == st.used_blocks, "used blocks with no copies queued", step);
    }
    pa_block_pool_destroy(pool);
}

} // namespace

int main()
{
    const int32_t sizes[] = {16, 32, 64, 256};
    for (int i = 0; i < 4; ++i)
        for (uint64_t seed = 1; seed <= 3; ++seed)
            run(24 + 17 * i, sizes[i], i % 2 ? 40 : 0, seed * 977 + i, 3000);
    std::printf("pool ops: %d failed checks\n", g_fail);
    return g_fail ? 1 : 0;
}
