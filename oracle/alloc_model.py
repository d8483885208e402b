"""Reference model of the block allocator -- TEST INFRASTRUCTURE ONLY.

A plain Python model of the host-side block pool, written independently of
the library's C++ allocator so that block tables, slot mappings and
refcounts can be checked bit for bit.  Only tests, the smoke check and the
benchmark's CPU-baseline leg use it.

What it models (sources, by page title and section):
  * dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
    PagedAttention Fixes It":
      - §4 "How PagedAttention Solves Fragmentation": a pool of fixed-size
        physical blocks made once at startup; one block table per sequence
        mapping logical block i (tokens i*bs .. i*bs+bs-1) to a physical id;
        on-demand allocation -- a sequence takes a new block exactly when its
        length reaches a multiple of the block size.
      - §5 "Zero-Copy Forking": several block tables may point at the same
        physical block, whose reference count is the number of tables that
        map it; a block returns to the pool when that count reaches zero.
        A branch's first new token goes to a private block (copy on write).
  * hyperinfer.ai, "KV cache & paged attention deep dive", "PagedAttention:
    virtual memory for attention state" and "What 16-token blocks buy you":
    new blocks come from a free pool; evicting a sequence frees its blocks.
  * dev.to §2 "The Concrete Math of KV Cache Growth": bytes per token
    = 2 x layers x kv_heads x head_dim x bytes per element.

The pages give no placement policy, so the library fixes one and this model
restates it (it is what makes the tables reproducible):
  * The free list starts as [0, 1, ..., N-1].  If the shuffle seed is
    non-zero it is permuted by a Fisher-Yates pass, i from N-1 down to 1,
    swapping entry i with entry (splitmix64() mod (i+1)), where splitmix64
    is the generator of Steele, Lea and Flood (OOPSLA 2014) seeded with the
    shuffle seed.
  * Allocation pops from the end of the free list; freeing pushes a
    sequence's blocks in table order onto the end.
  * Sequence ids count up from 0 and are never reused.
  * Copy on write.  An append that would write into a partly filled last
    block mapped by more than one table first pops a block for the appending
    sequence, puts it in place of the shared one (which loses a reference)
    and queues the copy (shared, private); the OUT_OF_BLOCKS check counts
    that block.  Queued copies are handed out in order by take_copies.  A
    block whose count reaches zero while a queued copy reads it waits in a
    held list and joins the free list (in order) when the copies are handed
    out; a queued copy into a block whose count reaches zero is dropped.
  * Prefix caching (dev.to §5 "Automatic Prefix Caching"; hyperinfer.ai
    "Prefix caching: share the system prompt").  A cached full block is keyed
    by (the cached block before it, or -1 for a first block; its 16 token
    ids), so equal keys mean equal whole prefixes.  The cache holds one
    reference per block.  register walks a sequence's full blocks from the
    start: a key already cached continues the chain through the cached block;
    otherwise the sequence's block is cached, until a block that is cached
    under other tokens.  match maps the longest chain of cached blocks into an
    empty sequence.  Every registration or match of a block stamps it with
    the next value of a counter; evict drops, one at a time, the block with
    the lowest stamp (ties: lower id) among cached blocks that only the cache
    maps and that no cached key names as parent.
  * Sliding window (vaibhawkumar.in, "Why LLMs run out of VRAM: KV cache
    fragmentation and the PagedAttention fix", "PagedAttention: the idea"
    and its truncate sketch: sliding the window releases whole leading
    pages; the cut inside the first kept page only moves its start).  A
    sequence keeps its length (the positions it has seen), a window start
    and a count of released leading blocks; its table maps the blocks from
    the first kept one.  slide_window(w) moves the start to length - w (never
    backwards) and releases, in order, every leading block that lies wholly
    before the start.  The export gives lengths and starts relative to the
    first kept block.  A sequence with a moved window can no longer register
    its prefix.
  * Swapping (hyperinfer.ai "What 16-token blocks buy you": swapping to CPU
    memory goes block by block).  A second pool of host blocks, ids 0..H-1,
    free list [0, ..., H-1], allocation from the end, frees appended in table
    order.  swap_out takes a host block for every block of the table, in
    table order, gives the pairs (device, host), then drops the device
    blocks in table order; it needs an empty copy queue (the copies are made
    first).  swap_in takes device blocks from the free list, in table order,
    gives the pairs (host, device), then frees the host blocks in table
    order.  A swapped-out sequence can only be swapped in or freed.
"""

MASK64 = (1 << 64) - 1

OK = 0
ERR_INVALID_ARG = 1
ERR_OUT_OF_BLOCKS = 2
ERR_CAPACITY = 3
ERR_UNSUPPORTED = 4


class SplitMix64:
    """splitmix64 as published by Steele, Lea and Flood (2014)."""

    def __init__(self, seed):
        self.state = seed & MASK64

    def next(self):
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes):
    """dev.to §2: 2 (K and V) x layers x kv_heads x head_dim x bytes."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


class PoolModel:
    def __init__(self, num_blocks, block_size, shuffle_seed, num_host_blocks=0):
        self.num_blocks = num_blocks
        self.block_size = block_size
        free = list(range(num_blocks))
        if shuffle_seed != 0:
            rng = SplitMix64(shuffle_seed)
            for i in range(num_blocks - 1, 0, -1):
                j = rng.next() % (i + 1)
                free[i], free[j] = free[j], free[i]
        self.free = free
        self.refcount = [0] * num_blocks
        self.tables = {}  # seq id -> list of physical block ids
        self.lens = {}    # seq id -> tokens stored
        self.next_id = 0
        self.copies = []  # queued (source, destination) block copies
        self.held = []    # unreferenced blocks a queued copy still reads
        self.prefix = {}  # (parent block, block_size tokens) -> cached block
        self.cache = {}   # cached block -> [key, stamp, cached children]
        self.clock = 0
        self.starts = {}  # seq id -> window start (a position)
        self.dropped = {}  # seq id -> leading blocks released by the window
        self.swapped = set()  # seq ids whose tables hold host block ids
        self.num_host_blocks = num_host_blocks
        self.host_free = list(range(num_host_blocks))

    # -- sequences -------------------------------------------------------
    def seq_create(self):
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        self.starts[sid] = 0
        self.dropped[sid] = 0
        return sid

    def _resident(self, sid):
        return sid in self.tables and sid not in self.swapped

    def _blocks_for(self, ntokens):
        return -(-ntokens // self.block_size)

    def _shared_tail(self, sid, ntok):
        """Would this append write into a partly filled block another table maps?"""
        table = self.tables[sid]
        return (ntok > 0 and self.lens[sid] % self.block_size != 0
                and self.refcount[table[-1]] > 1)

    def _check_append(self, sid, ntok):
        if not self._resident(sid) or ntok < 0:
            return ERR_INVALID_ARG, 0
        n = self.lens[sid]
        extra = 1 if self._shared_tail(sid, ntok) else 0
        return OK, (self._blocks_for(n + ntok) - self.dropped[sid] - len(self.tables[sid])
                    + extra)

    def _drop(self, blk):
        """One table stops mapping blk."""
        self.refcount[blk] -= 1
        if self.refcount[blk] > 0:
            return
        self.copies = [c for c in self.copies if c[1] != blk]
        if any(c[0] == blk for c in self.copies):
            self.held.append(blk)
        else:
            self.free.append(blk)

    def _do_append(self, sid, ntok):
        n = self.lens[sid]
        table = self.tables[sid]
        if self._shared_tail(sid, ntok):
            shared = table[-1]
            mine = self.free.pop()
            self.refcount[mine] = 1
            table[-1] = mine
            self.copies.append((shared, mine))
            self._drop(shared)
        first = self.dropped[sid]  # logical block of table[0]
        need = self._blocks_for(n + ntok) - first - len(table)
        for _ in range(need):
            blk = self.free.pop()
            self.refcount[blk] = 1
            table.append(blk)
        slots = []
        for pos in range(n, n + ntok):
            slots.append(table[pos // self.block_size - first] * self.block_size
                         + pos % self.block_size)
        self.lens[sid] = n + ntok
        return slots

    def append_slots(self, sid, ntok):
        """Returns (status, slots); on error nothing changes."""
        st, need = self._check_append(sid, ntok)
        if st != OK:
            return st, []
        if need > len(self.free):
            return ERR_OUT_OF_BLOCKS, []
        return OK, self._do_append(sid, ntok)

    def append_slots_batch(self, sids, ntok):
        """ntok tokens to each sequence, in list order; all or nothing."""
        if len(set(sids)) != len(sids):
            return ERR_INVALID_ARG, []
        total = 0
        for sid in sids:
            st, need = self._check_append(sid, ntok)
            if st != OK:
                return st, []
            total += need
        if total > len(self.free):
            return ERR_OUT_OF_BLOCKS, []
        out = []
        for sid in sids:
            out.extend(self._do_append(sid, ntok))
        return OK, out

    def fork(self, parent):
        if not self._resident(parent):
            return ERR_INVALID_ARG, -1
        child = self.seq_create()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        self.starts[child] = self.starts[parent]
        self.dropped[child] = self.dropped[parent]
        for blk in self.tables[child]:
            self.refcount[blk] += 1
        return OK, child

    def free_seq(self, sid):
        if sid not in self.tables:
            return ERR_INVALID_ARG
        if sid in self.swapped:
            self.host_free.extend(self.tables[sid])
            self.swapped.discard(sid)
        else:
            for blk in self.tables[sid]:
                self._drop(blk)
        del self.tables[sid]
        del self.lens[sid]
        del self.starts[sid]
        del self.dropped[sid]
        return OK

    # -- sliding window and swapping ---------------------------------------
    def slide_window(self, sid, window):
        """Keeps the last `window` positions in the window; returns (status,
        blocks released)."""
        if not self._resident(sid) or window < 0:
            return ERR_INVALID_ARG, 0
        bs = self.block_size
        self.starts[sid] = max(self.starts[sid], self.lens[sid] - window)
        released = 0
        table = self.tables[sid]
        while table and self.starts[sid] - self.dropped[sid] * bs >= bs:
            self._drop(table.pop(0))
            self.dropped[sid] += 1
            released += 1
        return OK, released

    def swap_out(self, sid):
        """Returns (status, [(device block, host block)]) in table order."""
        if not self._resident(sid) or self.copies:
            return ERR_INVALID_ARG, []
        table = self.tables[sid]
        if len(table) > len(self.host_free):
            return ERR_OUT_OF_BLOCKS, []
        pairs = [(blk, self.host_free.pop()) for blk in table]
        for blk in table:
            self._drop(blk)
        self.tables[sid] = [h for _, h in pairs]
        self.swapped.add(sid)
        return OK, pairs

    def swap_in(self, sid):
        """Returns (status, [(host block, device block)]) in table order."""
        if sid not in self.swapped:
            return ERR_INVALID_ARG, []
        hosts = self.tables[sid]
        if len(hosts) > len(self.free):
            return ERR_OUT_OF_BLOCKS, []
        pairs = []
        for h in hosts:
            blk = self.free.pop()
            self.refcount[blk] = 1
            pairs.append((h, blk))
        self.host_free.extend(hosts)
        self.tables[sid] = [d for _, d in pairs]
        self.swapped.discard(sid)
        return OK, pairs

    def take_copies(self):
        """The queued copies, in order; clears them and frees held blocks."""
        out = list(self.copies)
        self.copies = []
        self.free.extend(self.held)
        self.held = []
        return out

    # -- prefix cache -----------------------------------------------------
    def _stamp(self, blk):
        self.clock += 1
        self.cache[blk][1] = self.clock

    def prefix_register(self, sid, tokens):
        """Caches the full blocks of sid's first len(tokens) tokens; returns
        (status, blocks newly cached)."""
        if (not self._resident(sid) or len(tokens) > self.lens[sid] or self.starts[sid] != 0
                or self.dropped[sid] != 0):
            return ERR_INVALID_ARG, 0
        added, parent = 0, -1
        bs = self.block_size
        for i in range(len(tokens) // bs):
            key = (parent, tuple(int(t) for t in tokens[i * bs:(i + 1) * bs]))
            if key in self.prefix:
                parent = self.prefix[key]
                self._stamp(parent)
                continue
            blk = self.tables[sid][i]
            if blk in self.cache:
                break
            self.prefix[key] = blk
            self.cache[blk] = [key, 0, 0]
            self._stamp(blk)
            self.refcount[blk] += 1
            if parent >= 0:
                self.cache[parent][2] += 1
            parent = blk
            added += 1
        return OK, added

    def prefix_match(self, sid, tokens):
        """Maps the cached chain matching tokens into the empty sid; returns
        (status, tokens matched)."""
        if not self._resident(sid) or self.lens[sid] != 0:
            return ERR_INVALID_ARG, 0
        parent = -1
        bs = self.block_size
        for i in range(len(tokens) // bs):
            key = (parent, tuple(int(t) for t in tokens[i * bs:(i + 1) * bs]))
            if key not in self.prefix:
                break
            parent = self.prefix[key]
            self._stamp(parent)
            self.refcount[parent] += 1
            self.tables[sid].append(parent)
        self.lens[sid] = len(self.tables[sid]) * bs
        return OK, self.lens[sid]

    def prefix_evict(self, max_blocks):
        n = 0
        while n < max_blocks:
            cand = [(e[1], b) for b, e in self.cache.items()
                    if self.refcount[b] == 1 and e[2] == 0]
            if not cand:
                break
            _, blk = min(cand)
            key = self.cache.pop(blk)[0]
            del self.prefix[key]
            if key[0] >= 0:
                self.cache[key[0]][2] -= 1
            self._drop(blk)
            n += 1
        return n

    # -- export ----------------------------------------------------------
    def export(self, sids, max_blocks, with_starts=False, with_shared=False):
        """(status, tables[nseq][max_blocks] padded with -1, lens), then with
        with_starts the window starts, then with with_shared, per sequence,
        how many leading entries of its table name a block that another of
        the exported tables also names; lengths and starts count from the
        first kept block."""
        extra = ((None,) if with_starts else ()) + ((None,) if with_shared else ())
        tables, lens, starts = [], [], []
        for sid in sids:
            if not self._resident(sid):
                return (ERR_INVALID_ARG, None, None) + extra
            t = self.tables[sid]
            if len(t) > max_blocks:
                return (ERR_CAPACITY, None, None) + extra
            tables.append(t + [-1] * (max_blocks - len(t)))
            base = self.dropped[sid] * self.block_size
            lens.append(self.lens[sid] - base)
            starts.append(self.starts[sid] - base)
        out = (OK, tables, lens) + ((starts,) if with_starts else ())
        if with_shared:
            shared = []
            for i, sid in enumerate(sids):
                others = set()
                for j, other in enumerate(sids):
                    if j != i:
                        others.update(self.tables[other])
                k = 0
                while k < len(self.tables[sid]) and self.tables[sid][k] in others:
                    k += 1
                shared.append(k)
            out += (shared,)
        return out

    def stats(self):
        used = self.num_blocks - len(self.free)
        res = [s for s in self.tables if s not in self.swapped]
        bs = self.block_size
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": sum(1 for r in self.refcount if r > 1),
            "live_seqs": len(self.tables),
            "cached_blocks": len(self.cache),
            "swapped_seqs": len(self.swapped),
            "free_host_blocks": len(self.host_free),
            "logical_tokens": sum(self.lens[s] - self.starts[s] for s in self.tables),
            "mapped_blocks": sum(len(self.tables[s]) for s in res),
            "tail_slack_tokens": sum((self.dropped[s] + len(self.tables[s])) * bs - self.lens[s]
                                     for s in res),
        }


def execute_plan(model, ops):
    """Runs a workload plan (see workloads) on the model.  Returns
    (ids, prefill_slots): the model's id for each plan sequence, and the slots
    of every prefill token in plan order."""
    ids = []
    slots = []
    for op in ops:
        if op[0] == "create":
            ids.append(model.seq_create())
        elif op[0] == "fork":
            st, c = model.fork(ids[op[1]])
            assert st == OK, st
            ids.append(c)
        elif op[0] == "free":
            assert model.free_seq(ids[op[1]]) == OK
        elif op[0] == "prefill":
            st, s = model.append_slots(ids[op[1]], op[2])
            assert st == OK, st
            slots.extend(s)
        else:
            raise ValueError(op)
    return ids, slots
