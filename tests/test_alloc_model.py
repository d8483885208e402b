"""Pins of the allocator model (oracle/alloc_model.py) against the pages'
worked examples, published generator outputs and policy-free invariants."""
import json
import os

import numpy as np

from oracle import alloc_model as am

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_splitmix64_published_outputs():
    g = _golden("splitmix64_vectors.json")
    for vec in g["vectors"]:
        r = am.SplitMix64(vec["seed"])
        for want in vec["first_outputs"]:
            assert r.next() == int(want, 0)


def test_shuffled_free_list_is_a_permutation():
    for seed in [0, 1, 77, 2**63 + 5]:
        p = am.PoolModel(1000, 16, seed)
        assert sorted(p.free) == list(range(1000))
    assert am.PoolModel(50, 16, 0).free == list(range(50))
    assert am.PoolModel(50, 16, 3).free != list(range(50))


def test_on_demand_allocation_at_multiples_of_block_size():
    """dev.to §4 'On-Demand Allocation': one block at the start, tokens
    1..15 write into it, token 16 takes the next block."""
    p = am.PoolModel(10, 16, 0)
    s = p.seq_create()
    used = []
    for t in range(40):
        st, _ = p.append_slots(s, 1)
        assert st == am.OK
        used.append(p.stats()["used_blocks"])
    assert used[0] == 1 and used[15] == 1 and used[16] == 2 and used[31] == 2 and used[32] == 3


def test_page_addressing_example():
    """dev.to §4 figure: logical blocks 0/1/2 -> physical 84/12/903."""
    ex = _golden("devto_block_table_example.json")
    phys = [e["physical"] for e in ex["logical_blocks"]]
    p = am.PoolModel(1000, ex["block_size"], 0)
    p.free = [b for b in range(1000) if b not in phys] + phys[::-1]  # pops 84, 12, 903
    s = p.seq_create()
    st, slots = p.append_slots(s, 48)
    assert st == am.OK
    assert p.tables[s] == phys
    for e in ex["logical_blocks"]:
        for t in range(e["first_token"], e["last_token"] + 1):
            assert slots[t] == e["physical"] * 16 + (t - e["first_token"])
    assert slots[20] == 196 and slots[47] == 14463


def test_fork_example_and_sharing_saving():
    """dev.to §5: two prompt blocks mapped by both branches (refcount 2),
    each branch's first new token goes to its own private block."""
    ex = _golden("devto_fork_example.json")
    p = am.PoolModel(200, 16, 0)
    prompt_blocks = ex["prompt_physical_blocks"]
    priv = [b["private_block"] for b in ex["branches"]]
    order = prompt_blocks + priv  # pop order
    p.free = [b for b in range(200) if b not in order] + order[::-1]
    root = p.seq_create()
    assert p.append_slots(root, 32)[0] == am.OK
    st, a = p.fork(root)
    assert st == am.OK
    st, b = p.fork(root)
    p.free_seq(root)
    assert all(p.refcount[x] == ex["sharers_in_example"] for x in prompt_blocks)
    st, sa = p.append_slots(a, 16)
    st, sb = p.append_slots(b, 16)
    assert p.tables[a] == prompt_blocks + [priv[0]]
    assert p.tables[b] == prompt_blocks + [priv[1]]
    assert sa[0] == priv[0] * 16 and sb[-1] == priv[1] * 16 + 15
    # k sharers of a prompt use 1/k of the duplicated memory: 75% saved at k = 4
    k = ex["samples_sharing_prompt"]
    q = am.PoolModel(100, 16, 9)
    r = q.seq_create()
    q.append_slots(r, 32)
    kids = [q.fork(r)[1] for _ in range(k)]
    q.free_seq(r)
    st = q.stats()
    assert 1 - st["used_blocks"] / st["mapped_blocks"] == ex["prompt_memory_saving_with_4_sharers"]
    assert len(kids) == k


def test_out_of_blocks_changes_nothing():
    p = am.PoolModel(5, 16, 4)
    s = p.seq_create()
    assert p.append_slots(s, 60)[0] == am.OK  # 4 blocks
    before = (list(p.free), dict(p.lens), {k: list(v) for k, v in p.tables.items()})
    assert p.append_slots(s, 40)[0] == am.ERR_OUT_OF_BLOCKS  # needs 3 more
    t = p.seq_create()
    assert p.append_slots_batch([s, t], 20)[0] == am.ERR_OUT_OF_BLOCKS
    assert p.free == before[0] and p.lens[s] == before[1][s] and p.tables[s] == before[2][s]
    assert p.lens[t] == 0


def test_copy_on_write_of_a_shared_partial_block():
    """dev.to §5: a branch's first new token goes to a private block.  With a
    20-token prompt the second block is partly filled and shared after the
    fork, so the first branch to write gets a private block that starts as a
    copy of it; the last table still mapping it then writes in place."""
    p = am.PoolModel(8, 16, 0)  # pops 7, 6, 5, ...
    s = p.seq_create()
    assert p.append_slots(s, 20) == (am.OK, list(range(7 * 16, 7 * 16 + 16))
                                     + list(range(6 * 16, 6 * 16 + 4)))
    _, c = p.fork(s)
    assert p.refcount[6] == 2 and p.refcount[7] == 2
    assert p.append_slots(s, 1) == (am.OK, [5 * 16 + 4])     # private block 5
    assert p.tables[s] == [7, 5] and p.tables[c] == [7, 6]
    assert p.refcount[6] == 1 and p.refcount[5] == 1
    assert p.append_slots(c, 1) == (am.OK, [6 * 16 + 4])     # in place: only c maps 6
    assert p.take_copies() == [(6, 5)]
    assert p.take_copies() == []


def test_copy_on_write_holds_a_freed_source_and_drops_a_freed_destination():
    p = am.PoolModel(8, 16, 0)
    s = p.seq_create()
    p.append_slots(s, 20)                 # blocks 7, 6
    _, c = p.fork(s)
    p.append_slots(s, 1)                  # copy (6 -> 5) queued
    p.free_seq(c)                         # 6 loses its last reference ...
    assert 6 not in p.free and p.held == [6]   # ... but the queued copy reads it
    assert p.take_copies() == [(6, 5)]
    assert p.free[-1] == 6 and p.held == []
    # a copy into a block nobody maps any more is dropped
    _, d = p.fork(s)                      # s: [7, 5], 21 tokens
    p.append_slots(d, 1)                  # copy (5 -> 6) queued, d: [7, 6]
    p.free_seq(d)
    assert p.take_copies() == []
    assert p.free[-1] == 6


def test_copy_on_write_needs_a_free_block():
    p = am.PoolModel(2, 16, 0)
    s = p.seq_create()
    p.append_slots(s, 20)                 # both blocks
    _, c = p.fork(s)
    assert p.append_slots(c, 1)[0] == am.ERR_OUT_OF_BLOCKS
    assert p.tables[c] == p.tables[s] and p.take_copies() == []


def test_forked_sequences_read_their_own_tokens():
    """Content check, independent of how the pool places blocks: every token
    appended gets a unique value; a step's queued copies are applied, then
    its writes; each live sequence must read exactly its own history through
    its table, whatever forks (at any length), appends and frees came before."""
    rng = np.random.default_rng(5)
    p = am.PoolModel(160, 16, 77)
    content = {}
    history = {}
    live = []
    val = 0
    for step in range(400):
        writes = []
        for _ in range(int(rng.integers(1, 6))):
            op = rng.integers(0, 10)
            if op < 2 or not live:
                sid = p.seq_create()
                live.append(sid)
                history[sid] = []
            elif op < 6:
                sid = live[rng.integers(len(live))]
                n = int(rng.integers(1, 25))
                st, slots = p.append_slots(sid, n)
                if st != am.OK:
                    continue
                vals = list(range(val, val + n))
                val += n
                writes += list(zip(slots, vals))
                history[sid] += vals
            elif op < 8:
                par = live[rng.integers(len(live))]
                st, c = p.fork(par)
                live.append(c)
                history[c] = list(history[par])
            else:
                sid = live.pop(rng.integers(len(live)))
                p.free_seq(sid)
                del history[sid]
        for src, dst in p.take_copies():
            for o in range(16):
                if src * 16 + o in content:
                    content[dst * 16 + o] = content[src * 16 + o]
                else:
                    content.pop(dst * 16 + o, None)
        for slot, v in writes:
            content[slot] = v
        for sid in live:
            t = p.tables[sid]
            got = [content.get(t[i // 16] * 16 + i % 16) for i in range(p.lens[sid])]
            assert got == history[sid], (step, sid)


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(1)
    p = am.PoolModel(300, 16, 12345)
    live = []
    for _ in range(2000):
        op = rng.integers(0, 10)
        if op < 2 or not live:
            live.append(p.seq_create())
        elif op < 7:
            s = live[rng.integers(len(live))]
            p.append_slots(s, int(rng.integers(1, 40)))
        elif op < 8:
            s = live[rng.integers(len(live))]
            live.append(p.fork(s)[1])
        elif op < 9:
            p.take_copies()
        else:
            s = live.pop(rng.integers(len(live)))
            assert p.free_seq(s) == am.OK
        # invariants
        counts = {}
        for sid, t in p.tables.items():
            assert len(t) == -(-p.lens[sid] // 16)
            assert len(set(t)) == len(t)
            for b in t:
                counts[b] = counts.get(b, 0) + 1
        for b in range(300):
            assert p.refcount[b] == counts.get(b, 0)
        assert len(p.free) + len(p.held) + len(counts) == 300
        assert set(p.free).isdisjoint(counts) and set(p.held).isdisjoint(counts)
        assert set(p.held) <= {src for src, _ in p.copies}
        assert all(p.refcount[dst] >= 1 for _, dst in p.copies)


def test_average_tail_slack_is_about_half_a_block():
    """hyperinfer.ai 'What 16-token blocks buy you': across many sequences of
    varying length the unused tail averages about 8 tokens; for lengths spread
    evenly over residues it is (16 - 1) / 2 = 7.5."""
    rng = np.random.default_rng(2)
    p = am.PoolModel(200000, 16, 1)
    lens = rng.integers(1, 1500, size=3000)
    for n in lens:
        s = p.seq_create()
        assert p.append_slots(s, int(n))[0] == am.OK
    st = p.stats()
    avg = st["tail_slack_tokens"] / st["live_seqs"]
    assert abs(avg - 7.5) < 0.3
    assert all(len(p.tables[s]) * 16 - p.lens[s] <= 15 for s in p.tables)


def test_bytes_per_token_closed_form():
    g = _golden("devto_kv_sizes.json")
    for ex in g["examples"]:
        assert am.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"],
                                     ex["elem_bytes"]) == ex["bytes_per_token"]


def test_prefix_cache_maps_a_shared_system_prompt():
    """dev.to §5 "Automatic Prefix Caching" / hyperinfer.ai "Prefix caching":
    a request whose prompt starts with cached blocks maps them (no prefill for
    those tokens); a prompt that differs inside the second block maps only the
    first; eviction takes unreferenced leaves, least recently used first."""
    p = am.PoolModel(16, 16, 0)       # pops 15, 14, ...
    system = list(range(100, 132))    # two full blocks of system prompt
    a = p.seq_create()
    prompt_a = system + [7] * 8
    assert p.append_slots(a, 40)[0] == am.OK
    assert p.tables[a] == [15, 14, 13]
    assert p.prefix_register(a, prompt_a) == (am.OK, 2)     # the partial block is not cached
    assert p.refcount[15] == 2 and p.refcount[14] == 2 and p.stats()["cached_blocks"] == 2
    b = p.seq_create()
    assert p.prefix_match(b, system + [9] * 5) == (am.OK, 32)
    assert p.tables[b] == [15, 14] and p.refcount[15] == 3
    assert p.append_slots(b, 5) == (am.OK, [12 * 16 + i for i in range(5)])  # no copy: full blocks
    c = p.seq_create()
    other = system[:16] + [0] * 16
    assert p.prefix_match(c, other) == (am.OK, 16)
    assert p.tables[c] == [15]
    assert p.prefix_register(a, prompt_a) == (am.OK, 0)     # already cached: stamps only
    for s in (a, b, c):
        p.free_seq(s)
    assert p.refcount[15] == 1 and p.refcount[14] == 1      # the cache's own references
    assert 15 not in p.free and 14 not in p.free
    assert p.prefix_evict(1) == 1 and p.free[-1] == 14      # the leaf goes first
    assert p.prefix_evict(5) == 1 and p.free[-1] == 15
    assert p.stats()["cached_blocks"] == 0 and p.take_copies() == []


def test_prefix_cached_sequences_read_their_own_tokens():
    """Content check with prefix caching: prompts share a few system prompts;
    each request matches what it can, prefills the rest, registers its
    prompt, decodes a few tokens (forks too); blocks are evicted at random.
    Every live sequence must read back exactly its own tokens."""
    rng = np.random.default_rng(9)
    p = am.PoolModel(120, 16, 31)
    systems = [[int(x) for x in rng.integers(0, 50, size=n)] for n in (16, 37, 64)]
    content, history, live = {}, {}, []
    matched_total = 0
    for step in range(300):
        writes = []
        op = rng.integers(0, 10)
        if op < 3 or not live:
            prompt = systems[rng.integers(3)] + [int(x) for x in rng.integers(0, 50, size=int(rng.integers(0, 20)))]
            s = p.seq_create()
            st, m = p.prefix_match(s, prompt)
            matched_total += m
            rest = len(prompt) - m
            st, slots = p.append_slots(s, rest)
            if st != am.OK:
                p.free_seq(s)
                p.prefix_evict(8)
                continue
            writes += list(zip(slots, prompt[m:]))
            live.append(s)
            history[s] = list(prompt)
            p.prefix_register(s, prompt)  # its K/V are written below, before any reader
        elif op < 6:
            s = live[rng.integers(len(live))]
            tok = int(rng.integers(0, 50))
            st, slots = p.append_slots(s, 1)
            if st == am.OK:
                writes.append((slots[0], tok))
                history[s].append(tok)
        elif op < 7:
            par = live[rng.integers(len(live))]
            c = p.fork(par)[1]
            live.append(c)
            history[c] = list(history[par])
        elif op < 9:
            s = live.pop(rng.integers(len(live)))
            p.free_seq(s)
            del history[s]
        else:
            p.prefix_evict(int(rng.integers(1, 6)))
        for src, dst in p.take_copies():
            for o in range(16):
                if src * 16 + o in content:
                    content[dst * 16 + o] = content[src * 16 + o]
                else:
                    content.pop(dst * 16 + o, None)
        for slot, v in writes:
            content[slot] = v
        for s in live:
            t = p.tables[s]
            got = [content.get(t[i // 16] * 16 + i % 16) for i in range(p.lens[s])]
            assert got == history[s], (step, s)
        counts = {}
        for t in p.tables.values():
            for b in t:
                counts[b] = counts.get(b, 0) + 1
        for b in range(120):
            assert p.refcount[b] == counts.get(b, 0) + (1 if b in p.cache else 0)
    assert matched_total > 500  # the cache was actually used


def test_sliding_window_releases_whole_leading_blocks():
    """vaibhawkumar.in, "PagedAttention: the idea": sliding the window hands
    the oldest whole pages back to the allocator; a cut inside the first kept
    page only moves its start."""
    p = am.PoolModel(20, 16, 0)  # free list 0..19, taken from the end
    s = p.seq_create()
    assert p.append_slots(s, 100)[0] == am.OK
    assert p.tables[s] == [19, 18, 17, 16, 15, 14, 13]
    assert p.slide_window(s, 200) == (am.OK, 0)  # a window longer than the sequence
    assert p.slide_window(s, 40) == (am.OK, 3)   # start 60: blocks of 0..47 go
    assert p.tables[s] == [16, 15, 14, 13]
    assert p.free[-3:] == [19, 18, 17]
    st, t, n, w = p.export([s], 4, with_starts=True)
    assert (n, w) == ([52], [12])  # from the first kept block (positions 48..)
    assert p.append_slots(s, 1) == (am.OK, [13 * 16 + 100 % 16])
    assert p.slide_window(s, 50) == (am.OK, 0)  # never moves the start back
    assert p.starts[s] == 60
    assert p.slide_window(s, 0) == (am.OK, 3)   # start 101: blocks of 48..95 go
    st, t, n, w = p.export([s], 4, with_starts=True)
    assert t == [[13, -1, -1, -1]] and (n, w) == ([5], [5])  # an empty window
    st = p.stats()
    assert st["logical_tokens"] == 0 and st["tail_slack_tokens"] == 11
    assert p.prefix_register(s, list(range(101)))[0] == am.ERR_INVALID_ARG


def test_swap_out_and_in_block_by_block():
    """hyperinfer.ai, "What 16-token blocks buy you": swapping to CPU memory
    goes block by block.  The pairs name every block once, in table order."""
    p = am.PoolModel(10, 16, 0, num_host_blocks=4)
    s, o = p.seq_create(), p.seq_create()
    p.append_slots(s, 40)  # blocks 9, 8, 7
    p.append_slots(o, 1)   # block 6
    c = p.fork(s)[1]
    assert p.append_slots(c, 1)[0] == am.OK  # copy on write of block 7 queued
    assert p.swap_out(s) == (am.ERR_INVALID_ARG, [])  # copies first
    assert p.take_copies() == [(7, 5)]
    st, pairs = p.swap_out(s)
    assert st == am.OK and pairs == [(9, 3), (8, 2), (7, 1)]
    assert p.refcount[9] == p.refcount[8] == 1  # still mapped by the fork
    assert p.refcount[7] == 0 and p.free[-1] == 7
    assert p.append_slots(s, 1)[0] == am.ERR_INVALID_ARG
    assert p.fork(s)[0] == am.ERR_INVALID_ARG
    assert p.export([s], 4)[0] == am.ERR_INVALID_ARG
    st = p.stats()
    assert st["swapped_seqs"] == 1 and st["free_host_blocks"] == 1 and st["live_seqs"] == 3
    assert p.swap_out(o) == (am.OK, [(6, 0)])
    assert p.swap_out(c) == (am.ERR_OUT_OF_BLOCKS, [])  # no host block left
    free_before = list(p.free)
    st, pairs = p.swap_in(s)
    assert st == am.OK and pairs == [(3, free_before[-1]), (2, free_before[-2]),
                                     (1, free_before[-3])]
    assert p.host_free == [3, 2, 1]
    assert p.swap_in(s)[0] == am.ERR_INVALID_ARG
    assert p.free_seq(o) == am.OK and p.host_free == [3, 2, 1, 0]


def test_windows_and_swaps_keep_every_sequence_s_tokens():
    """Content check: appends, forks (copy on write), frees, window slides,
    swaps out and in, with the copies and swap transfers applied to a model
    of device and host memory.  Every resident sequence must read back
    exactly the tokens of its window."""
    rng = np.random.default_rng(17)
    bs = 16
    p = am.PoolModel(60, bs, 5, num_host_blocks=40)
    dev, host = {}, {}
    hist, live = {}, []
    slides = swaps = 0
    for step in range(600):
        writes = []
        op = rng.integers(0, 12)
        if op < 2 or not live:
            s = p.seq_create()
            live.append(s)
            hist[s] = []
        elif op < 6:
            s = live[rng.integers(len(live))]
            k = int(rng.integers(1, 30))
            st, slots = p.append_slots(s, k)
            if st == am.OK:
                toks = [int(x) for x in rng.integers(0, 1000, size=k)]
                writes += list(zip(slots, toks))
                hist[s] += toks
        elif op < 7:
            par = live[rng.integers(len(live))]
            st, c = p.fork(par)
            if st == am.OK:
                live.append(c)
                hist[c] = list(hist[par])
        elif op < 8:
            s = live.pop(rng.integers(len(live)))
            p.free_seq(s)
            del hist[s]
        elif op < 10:
            s = live[rng.integers(len(live))]
            if p.slide_window(s, int(rng.integers(0, 60)))[0] == am.OK:
                slides += 1
        else:
            for src, dst in p.take_copies():  # swapping needs the copies made
                for o in range(bs):
                    dev[dst * bs + o] = dev.get(src * bs + o)
            s = live[rng.integers(len(live))]
            if s in p.swapped:
                st, pairs = p.swap_in(s)
                src_mem, dst_mem = host, dev
            else:
                st, pairs = p.swap_out(s)
                src_mem, dst_mem = dev, host
            if st == am.OK:
                swaps += 1
                for a, b in pairs:
                    for o in range(bs):
                        dst_mem[b * bs + o] = src_mem.get(a * bs + o)
        for src, dst in p.take_copies():
            for o in range(bs):
                dev[dst * bs + o] = dev.get(src * bs + o)
        for slot, v in writes:
            dev[slot] = v
        for s in live:
            if s in p.swapped:
                continue
            t, first = p.tables[s], p.dropped[s]
            got = [dev.get(t[i // bs - first] * bs + i % bs)
                   for i in range(p.starts[s], p.lens[s])]
            assert got == hist[s][p.starts[s]:], (step, s)
        counts = {}
        for s, t in p.tables.items():
            if s not in p.swapped:
                for b in t:
                    counts[b] = counts.get(b, 0) + 1
        for b in range(p.num_blocks):
            assert p.refcount[b] == counts.get(b, 0)
        assert len(p.free) + len(p.held) + len(counts) == p.num_blocks
    assert slides > 50 and swaps > 50
