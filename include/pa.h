/*
 * pa.h -- C ABI of libpa: paged KV cache and PagedAttention decode on AMD
 * Instinct MI355X (gfx950).
 *
 * What the calls compute is fixed by three pages (cited by title and
 * section):
 *   [devto] dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and
 *           How PagedAttention Fixes It"
 *   [hi]    hyperinfer.ai, "KV cache & paged attention deep dive"
 *   [vk]    vaibhawkumar.in, "Why LLMs run out of VRAM: KV cache
 *           fragmentation and the PagedAttention fix"
 *
 * Conventions shared by every call:
 *   - Every function returns a pa_status; on failure pa_last_error() gives a
 *     message (thread-local, valid until the next failing call on the thread).
 *   - The library never allocates or frees device memory.  Device buffers
 *     (caches, q, out, tables, workspace) belong to the caller and are
 *     borrowed until the launched work completes on `stream`.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Kernel calls are asynchronous: argument errors that the host can see are
 *     returned at once, device-side faults appear at the caller's next
 *     synchronisation.
 *   - All arrays are dense, row-major, without padding.
 *
 * Cache layout (per layer, one K and one V tensor, both [num_blocks][Hkv]
 * pieces of one block of one KV head; bs = block_size, o = offset in block,
 * b = bytes per element, p = 4 / b):
 *   k_cache[block][kv_head][o][dim]                   token-major K
 *   v_cache[block][kv_head][o / 16][vt(o % 16, dim)]  V as bs/16 tiles of 16
 *                                                      tokens x D dims, with
 *   vt(u, d) = ((((d / 16p) * 4 + u / 4) * 16 + d % 16) * p + (d / 16) % p) * 4 + u % 4,
 * so each 16-byte piece of a V tile holds p dims (16 apart) of 4 consecutive
 * tokens, and a tile is read 1 KiB at a time with 16 bytes per lane.  head_dim
 * is a multiple of 16p (64 and 128 are).  The pages fix only that a block
 * holds a fixed number of consecutive tokens ([devto] §4); the orders are
 * this library's choice: every 16-token tile of any block size has the
 * layout the decode kernels consume.
 *
 * A token's slot is block * block_size + offset; token t of a sequence lives
 * in block block_tables[seq][t / block_size] at offset t % block_size
 * ([devto] §4, the logical-to-physical block figure).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* bad pointer, shape, id or size */
    PA_ERR_OUT_OF_BLOCKS = 2, /* the pool cannot supply the blocks asked for */
    PA_ERR_CAPACITY = 3,      /* a caller-sized buffer is too small */
    PA_ERR_UNSUPPORTED = 4,   /* valid request the library does not implement */
    PA_ERR_HIP = 5            /* a HIP runtime call or launch failed */
} pa_status;

typedef enum {
    PA_F32 = 0,
    PA_F16 = 1,
    PA_BF16 = 2,
    PA_FP8_E4M3 = 3 /* OCP E4M3FN: bias 7, max 448, no infinities */
} pa_dtype;

/* ------------------------------------------------------------------------ */
/* Block pool (host only).                                                  */
/* ------------------------------------------------------------------------ */

typedef struct pa_pool pa_pool;

typedef struct {
    int32_t num_blocks;    /* physical blocks, fixed at init */
    int32_t block_size;    /* tokens per block: 16, 32, 64, 128 or 256 */
    int32_t num_layers;    /* used only for the byte counts below */
    int32_t num_kv_heads;
    int32_t head_dim;
    pa_dtype kv_dtype;
    uint64_t shuffle_seed; /* 0: free list in id order; else a seeded permutation */
    int32_t num_host_blocks; /* host swap space in blocks (0: no swapping) */
} pa_pool_config;

typedef struct {
    int32_t num_blocks;
    int32_t free_blocks;
    int32_t used_blocks;       /* blocks with refcount > 0 */
    int32_t shared_blocks;     /* blocks with refcount > 1 */
    int32_t live_seqs;         /* swapped-out ones included */
    int32_t cached_blocks;     /* blocks the prefix cache holds */
    int32_t swapped_seqs;      /* live sequences whose blocks are in host swap space */
    int32_t free_host_blocks;
    int64_t logical_tokens;    /* sum over live sequences of the tokens in their windows */
    int64_t mapped_blocks;     /* sum of device block-table lengths (a shared block counts per
                                  table) */
    int64_t tail_slack_tokens; /* sum over resident sequences of unused slots after their last
                                  token */
} pa_pool_stats;

/* Creates the pool: every block of the fixed-size physical pool exists from
 * the start and sits on the free list ([devto] §4 "Centralized Physical Block
 * Pool"; [hi] "PagedAttention: virtual memory for attention state").
 * Placement policy: the free list starts as ids 0..N-1; a non-zero
 * shuffle_seed permutes it by a Fisher-Yates pass (i from N-1 down to 1,
 * swap with splitmix64() mod (i+1), splitmix64 of Steele, Lea and Flood
 * seeded with shuffle_seed).  Blocks are taken from the end of the list and
 * returned to the end.  *out receives the pool; the caller frees it with
 * pa_block_pool_destroy.  Errors: PA_ERR_INVALID_ARG for non-positive sizes
 * or an unknown dtype, PA_ERR_UNSUPPORTED for another block_size.  The pages
 * use 16-token blocks and also name 32 and pages of 256 or more ([devto] §4
 * and §6; [vk] paged-cache sketch). */
pa_status pa_block_pool_init(const pa_pool_config *cfg, pa_pool **out);

/* Frees the pool object (NULL is ignored). */
void pa_block_pool_destroy(pa_pool *pool);

/* KV bytes one token occupies over all layers: 2 x layers x kv_heads x
 * head_dim x bytes per element ([devto] §2 "The Concrete Math of KV Cache
 * Growth"; [hi] "What the KV cache is").  Page size is counted in tokens and
 * bytes follow from the dtype ([vk] "Practical pitfalls", item 3).
 * Returns 0 for a NULL pool. */
uint64_t pa_kv_bytes_per_token(const pa_pool *pool);

/* Bytes of one block of one layer in one of the two tensors (K or V):
 * block_size x kv_heads x head_dim x bytes per element.  The caller sizes
 * each cache tensor as num_blocks times this.  0 for a NULL pool. */
uint64_t pa_block_bytes(const pa_pool *pool);

/* New empty sequence; ids count up from 0 and are never reused. */
pa_status pa_seq_create(pa_pool *pool, int32_t *seq_out);

/* Reserves slots for ntok more tokens of `seq` and writes their slot ids
 * (block * block_size + offset) to slots_out[0..ntok).  A block is taken
 * from the free list exactly when the sequence length reaches a multiple of
 * block_size ([devto] §4 "On-Demand Allocation").  Copy on write ([devto]
 * §5 "Parallel Sampling & Tree Search": a branch's first new token goes to a
 * private block): if the sequence's last block is partly filled and another
 * table also maps it (refcount > 1), a free block is taken first, replaces
 * the shared one in this table (which loses one reference), and the copy
 * (shared -> private) is queued for pa_pool_take_copies; the slots then lie
 * in the private block.  The caller must make the queued copies on the device
 * (pa_copy_blocks) before writing these slots.  All or nothing: on
 * PA_ERR_OUT_OF_BLOCKS nothing changes (a needed private copy counts as one
 * block). */
pa_status pa_seq_append_slots(pa_pool *pool, int32_t seq, int32_t ntok, int32_t *slots_out);

/* pa_seq_append_slots for nseq distinct sequences, ntok tokens each, in the
 * given order; slots_out receives nseq*ntok slots, sequence-major.  All or
 * nothing over the whole batch.  This is the per-step host work of a decode
 * step (ntok = 1). */
pa_status pa_seq_append_slots_batch(pa_pool *pool, const int32_t *seqs, int32_t nseq,
                                    int32_t ntok, int32_t *slots_out);

/* New sequence whose table maps the same physical blocks as `parent`, each
 * block's reference count incremented ([devto] §5 "Parallel Sampling & Tree
 * Search": tables point at the same prompt blocks; [hi] "Prefix caching").
 * The child has the parent's length. */
pa_status pa_seq_fork(pa_pool *pool, int32_t parent, int32_t *child_out);

/* Drops the sequence; each of its blocks loses one reference and returns to
 * the free list (in table order) when the count reaches zero ([hi] "What
 * 16-token blocks buy you": evicting a sequence frees its blocks).  A block
 * that a queued copy still reads is held back and joins the free list when
 * the copies are taken; a queued copy into a freed block is dropped. */
pa_status pa_seq_free(pa_pool *pool, int32_t seq);

/* Sliding window ([vk] "PagedAttention: the idea": sliding the window
 * releases the oldest whole pages to the allocator; a cut inside the first
 * kept page only moves its start, nothing is copied).  Moves the window start
 * of `seq` to length - window (never backwards) and drops, in table order,
 * every leading block that lies wholly before the start; each loses one
 * reference and is freed at zero like a freed sequence's blocks.  Later
 * appends continue at the sequence's length; pa_export_block_tables gives
 * the kept blocks with lengths and window starts counted from the first kept
 * block, and the decode calls take those starts.  A sequence whose window
 * has moved can no longer register its prefix.  *released_out (may be NULL):
 * blocks dropped from the table. */
pa_status pa_seq_slide_window(pa_pool *pool, int32_t seq, int32_t window,
                              int32_t *released_out);

/* Swapping a sequence out to host memory and back, block by block ([hi]
 * "What 16-token blocks buy you": swapping to CPU RAM goes one block at a
 * time, with no contiguous reorganisation).  The pool manages host block ids
 * 0..num_host_blocks-1 (a free list in id order, taken from and returned to
 * the end); the caller owns the host memory (pinned, laid out like a cache
 * of num_host_blocks blocks) and moves the bytes with pa_swap_blocks.
 *
 * pa_seq_swap_out: for each block of the table, in order, takes a host block
 * and writes the pair (device block, host block) to pairs_out; then every
 * device block loses the table's reference (freed at zero).  The caller must
 * copy the pairs (pa_swap_blocks, to host) before any later write to those
 * device blocks (launch it next on the same stream).  Needs an empty
 * copy-on-write queue (take and make those copies first).  A swapped-out
 * sequence can only be swapped in or freed.
 * pa_seq_swap_in: takes a device block for each host block, in table order,
 * writes the pairs (host block, device block), and frees the host blocks; the
 * caller copies the pairs (pa_swap_blocks, to device) before the next decode
 * of the sequence.  The sequence keeps its length and window.
 * Both: *count_out = blocks of the table; PA_ERR_OUT_OF_BLOCKS if the other
 * side has too few free blocks, then PA_ERR_CAPACITY if max_pairs is smaller
 * (or pairs_out NULL); nothing changes on an error. */
pa_status pa_seq_swap_out(pa_pool *pool, int32_t seq, int32_t *pairs_out, int32_t max_pairs,
                          int32_t *count_out);
pa_status pa_seq_swap_in(pa_pool *pool, int32_t seq, int32_t *pairs_out, int32_t max_pairs,
                         int32_t *count_out);

/* Current length (positions appended so far) of a live sequence. */
pa_status pa_seq_length(const pa_pool *pool, int32_t seq, int32_t *len_out);

/* Reference count of one physical block. */
pa_status pa_block_refcount(const pa_pool *pool, int32_t block, int32_t *refcount_out);

/* Writes the block tables of nseq resident sequences into tables_out
 * [nseq][max_blocks] (int32, entries past a table's end set to -1), their
 * lengths into lens_out[nseq], their window starts into starts_out[nseq] and
 * into shared_out[nseq] how many leading entries of each table hold a block
 * that another of these nseq tables also holds (any output may be NULL).
 * Lengths and starts count from the first kept block (see
 * pa_seq_slide_window); without a window they are the length and 0.  The
 * shared counts are a hint for the decode calls' seq_shared: blocks shared
 * through a common prefix ([devto] §5 "Automatic Prefix Caching"; [hi]
 * "Prefix caching: share the system prompt") are read once per sequence
 * that holds them, so they are worth keeping in the GPU caches.
 * PA_ERR_CAPACITY if a table has more than max_blocks entries. */
pa_status pa_export_block_tables(const pa_pool *pool, const int32_t *seqs, int32_t nseq,
                                 int32_t max_blocks, int32_t *tables_out, int32_t *lens_out,
                                 int32_t *starts_out, int32_t *shared_out);

/* Share plan of a decode batch: which sequences hold the same leading blocks,
 * so that a decode launch can read those blocks once per KV head for all of
 * them ([devto] §5 "Zero-Copy Forking" and "Automatic Prefix Caching": the
 * sharers' tables point at one copy of the prompt's blocks; [hi] "Prefix
 * caching: share the system prompt": one copy of the prefix KV serves every
 * request).  int32 words, for a batch of B sequences in export order:
 *   [0]                  PA_SHARE_PLAN_MAGIC
 *   [1]                  number of groups, ng
 *   [2 + b]              leading table entries of b whose block another of the
 *                        B tables also holds (the hint of pa_export_block_tables)
 *   [2 + B + b]          group of b, or -1
 *   [2 + 2B + b]         rank of b in its group (0 when none)
 *   [2 + 3B + b]         leading blocks of b its group shares (0 when none)
 *   [2 + 4B + g]         members of group g (g < ng)
 *   [2 + 5B + g]         leading blocks group g shares
 *   [2 + 6B + i]         members, group by group, each in rank order
 *   [2 + 7B + g]         index in that list of group g's first member
 * A group: at least two sequences without a slid window whose tables begin
 * with the same block; it shares the longest run of leading entries all its
 * members hold alike, counting only blocks before each member's last token
 * (so the shared tokens are the same for all, and the block a step appends
 * to stays the member's own).  Groups are numbered by their first member and
 * members are in batch order.  A plan is valid for the tables and lengths
 * it was exported with. */
#define PA_SHARE_PLAN_MAGIC 0x31534150
#define PA_SHARE_PLAN_WORDS(nseq) (2 + 8 * (size_t)(nseq))

/* Writes the share plan of nseq resident sequences (as listed for
 * pa_export_block_tables) into plan_out[PA_SHARE_PLAN_WORDS(nseq)].
 * PA_ERR_INVALID_ARG for an unknown or swapped-out sequence. */
pa_status pa_export_share_plan(const pa_pool *pool, const int32_t *seqs, int32_t nseq,
                               int32_t *plan_out);

pa_status pa_pool_get_stats(const pa_pool *pool, pa_pool_stats *out);

/* Hands out the block copies the appends since the last call queued (copy on
 * write, see pa_seq_append_slots), in the order they were made, as int32
 * pairs pairs_out[i][0] = source block, pairs_out[i][1] = destination block,
 * and clears the queue; held blocks then join the free list.  *count_out is
 * the number of queued copies; if it exceeds max_pairs (or pairs_out is
 * NULL) nothing is written or cleared and PA_ERR_CAPACITY is returned, so a
 * call with max_pairs = 0 asks for the count.  No block is both a source and
 * a destination in one set of copies. */
pa_status pa_pool_take_copies(pa_pool *pool, int32_t *pairs_out, int32_t max_pairs,
                              int32_t *count_out);

/* Prefix caching ([devto] §5 "Automatic Prefix Caching": a request whose
 * prompt matches computed blocks maps those physical blocks and skips their
 * prefill; [hi] "Prefix caching: share the system prompt": one copy of the
 * prefix KV, mapped by every request).  A cached block is identified by its
 * block_size token ids and the cached block holding the block_size tokens
 * before it (none for a first block), so a match means the whole prefix up to
 * it is equal; the cache holds one reference on each of its blocks.
 *
 * pa_prefix_register: puts the full blocks of `seq`'s first ntok tokens
 * (token ids `tokens`, ntok <= its length) into the cache, block by block from
 * the start; a block whose key is already cached is skipped (its cached block
 * continues the chain), and registration stops at a block cached under other
 * tokens.  *added_out (may be NULL): blocks newly cached.  Call it once the
 * K/V of those tokens are in the cache. */
pa_status pa_prefix_register(pa_pool *pool, int32_t seq, const int32_t *tokens, int32_t ntok,
                             int32_t *added_out);

/* For an empty sequence (new request, length 0): maps the longest run of
 * cached full blocks matching tokens[0..ntok) from the start into its table
 * (each gains a reference) and sets its length to the tokens they hold,
 * written to *matched_out (a multiple of block_size).  The caller prefills
 * the remaining tokens with pa_seq_append_slots as usual. */
pa_status pa_prefix_match(pa_pool *pool, int32_t seq, const int32_t *tokens, int32_t ntok,
                          int32_t *matched_out);

/* Drops up to max_blocks cached blocks that no table maps, least recently
 * registered or matched first (ties: lower block id), only blocks no other
 * cached block names as its parent; each returns to the free list.
 * *evicted_out (may be NULL): blocks dropped. */
pa_status pa_prefix_evict(pa_pool *pool, int32_t max_blocks, int32_t *evicted_out);

/* ------------------------------------------------------------------------ */
/* Kernels (device, asynchronous on `stream`).                              */
/* ------------------------------------------------------------------------ */

/* Kernel choice for pa_decode. */
enum {
    PA_KERNEL_AUTO = 0, /* library picks by dtype, head_dim and group size */
    PA_KERNEL_VALU = 1, /* vector-ALU kernel (fp32 math); every dtype;
                           group 1, 2 or 4 (8 at head_dim 64) */
    PA_KERNEL_MFMA = 2  /* matrix-core kernel; 16-bit q, 16-bit or FP8 KV;
                           group 1..16 */
};

typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;  /* must divide num_q_heads; group G = Hq / Hkv */
    int32_t head_dim;      /* 64 or 128 */
    int32_t block_size;    /* 16, 32, 64, 128 or 256; as the pool's */
    int32_t num_blocks;    /* blocks in each cache tensor (bounds for ids/slots) */
    pa_dtype q_dtype;      /* q, out and the new tokens' K/V */
    pa_dtype kv_dtype;     /* cache storage: equal to q_dtype, or FP8 with 16-bit q */
    int32_t kernel;        /* PA_KERNEL_* */
} pa_kv_desc;

/* Writes the K and V of num_tokens new tokens into their cache slots
 * (s = slot_mapping[t], o = s % bs, in the layout above):
 *   k_cache[s / bs][g][o][d] = cvt(k[t][g][d])
 *   v_cache[s / bs][g][o / 16][vt(o % 16, d)] = cvt(v[t][g][d])
 * for every KV head g and dim d ([devto] §1: the new token's K and V are
 * appended to the cache; §4: a slot is a place in a physical block).
 * k, v: device [num_tokens][Hkv][D] in desc->q_dtype.  slot_mapping: device
 * int32 [num_tokens]; a negative slot skips the token; slots must be
 * distinct.  cvt is a bit copy when kv_dtype == q_dtype; for FP8 it is
 * e4m3(x * fl32(1/k_scale)) (resp. v_scale) rounded to nearest, ties to even,
 * saturating at +-448 ([devto] §6 "Enable FP8 KV Cache"; [hi] "KV
 * quantization cuts memory in half"); k_scale and v_scale are the
 * dequantisation factors and are ignored for other dtypes.  A slot outside
 * [0, num_blocks * block_size) is skipped by the kernel. */
pa_status pa_cache_append(const void *k, const void *v, void *k_cache, void *v_cache,
                          const int32_t *slot_mapping, int32_t num_tokens,
                          const pa_kv_desc *desc, float k_scale, float v_scale, void *stream);

/* partition_size for pa_decode. */
#define PA_PARTITION_NONE 0       /* one pass per (sequence, KV head), no workspace */
#define PA_PARTITION_BALANCED (-1) /* tokens split evenly over the GPU's waves */

/* Workspace bytes pa_decode needs for this shape and partitioning (0 for
 * PA_PARTITION_NONE).  partition_size > 0 must be a multiple of 16.  For
 * PA_PARTITION_BALANCED with the MFMA kernel and a shape that can read a
 * share plan's groups once per KV head (see seq_shared), this includes the
 * room for those reads' partial states, (W + Hkv x num_seqs / 2) x
 * 4 x 16 / G slots of G x (head_dim + 2) floats (W: the launch's waves),
 * and, from the next 256-byte boundary, 16 bytes per (sequence, KV head) in
 * which the decode records where the merge finds that pair's partial
 * states; a launch given less, but no less than the size without that room,
 * reads every sequence's blocks itself. */
size_t pa_decode_workspace_bytes(const pa_kv_desc *desc, int32_t num_seqs, int32_t max_seq_len,
                                 int32_t partition_size);

/* Runs W of a PA_PARTITION_BALANCED launch of this shape on the current
 * device: the waves of the balanced kernel the GPU holds at once (CUs x
 * resident waves per CU; 1,024 on an MI355X).  0 for a shape the balanced
 * mode does not take, or when the device cannot be queried. */
int32_t pa_decode_balanced_waves(const pa_kv_desc *desc);

/* Single-query attention for each sequence b and query head h
 * ([devto] §1, Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V; §4 "The
 * PagedAttention CUDA Kernel": the query reads K and V through the block
 * table):
 *   out[b][h][:] = sum_t w_t * v_scale * V_t / sum_t w_t,
 *   w_t = exp(scale * k_scale * <q[b][h], K_t> - max),  t in [w_b, seq_lens[b]),
 * with K_t, V_t the rows of KV head h / (Hq / Hkv) found through
 * block_tables[b][t / bs], and w_b = seq_starts[b] the window start (0 when
 * seq_starts is NULL; [vk] "PagedAttention: the idea": a slid window leaves
 * the earlier tokens of its first kept page out).  A zero-length sequence or
 * an empty window (w_b = seq_lens[b]) gives a zero row.
 *   q, out: device [num_seqs][Hq][D] in desc->q_dtype (out may not alias q).
 *   block_tables: device int32 [num_seqs][max_blocks_per_seq].
 *   seq_lens: device int32 [num_seqs], each in [0, max_seq_len] and
 *     <= max_blocks_per_seq * block_size; a row whose length, window start or
 *     block ids are out of range is written as NaN instead of being read.
 *   seq_starts: device int32 [num_seqs] or NULL; each in [0, seq_lens[b]]
 *     (not read for zero-length rows).  pa_export_block_tables gives them.
 *   seq_shared: device int32 [PA_SHARE_PLAN_WORDS(num_seqs)] or NULL: the
 *     batch's share plan (pa_export_share_plan, for these tables and
 *     lengths; with any other plan the outputs are unspecified, though
 *     every access stays inside the buffers).  With the MFMA kernel, the
 *     leading entries other tables also hold are read with loads that keep
 *     them in the GPU caches (all others with streaming loads, read once).
 *     With PA_PARTITION_BALANCED, 16 % G == 0, G x head_dim
 *     a power-of-two multiple of 256 up to 2048, and a workspace of
 *     pa_decode_workspace_bytes(), the blocks a group shares are read once
 *     per KV head for all its members: the group is cut into rows of
 *     4 x 16 / G members, whose query heads fill four 16-column MFMA tiles,
 *     and the launch's waves take pieces of those rows as they take pieces
 *     of sequences; the merge folds each member's row state in with its own
 *     pieces.  The VALU kernel ignores the plan.  The result does not depend
 *     on the plan beyond rounding (tokens are summed in another order).
 *   partition_size: PA_PARTITION_NONE, PA_PARTITION_BALANCED, or a positive
 *     multiple of block_size: each (sequence, KV head) is split into chunks
 *     of that many tokens whose partial softmax states are merged by a second
 *     kernel.  The partitioned modes need `workspace` (device, 16-byte
 *     aligned, at least pa_decode_workspace_bytes(...) bytes, no initial
 *     contents required; two launches that may run at the same time must
 *     not share one).
 * Accumulation is fp32; out is rounded to nearest even. */
pa_status pa_decode(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *seq_lens, const int32_t *seq_starts,
                    const int32_t *seq_shared, int32_t num_seqs, int32_t max_seq_len,
                    float scale, float k_scale, float v_scale, void *out,
                    void *workspace, size_t workspace_bytes, int32_t partition_size,
                    const pa_kv_desc *desc, void *stream);

/* Makes the copies pa_pool_take_copies handed out, for one layer's caches:
 * for each pair (src, dst) of the device int32 array pairs[num_pairs][2], the
 * K and V of block dst (all KV heads) become those of block src ([devto] §5:
 * the private block of a branch starts as a copy of the shared one).  Ids
 * outside [0, num_blocks) and src == dst are skipped.  num_pairs in
 * [0, 65535]. */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int32_t num_pairs,
                         const pa_kv_desc *desc, void *stream);

/* Moves the bytes of pa_seq_swap_out / pa_seq_swap_in for one layer's
 * caches ([hi] "What 16-token blocks buy you": swapping to CPU RAM is block
 * by block).  host_k, host_v: pinned host memory (hipHostMalloc, e.g. a
 * pinned torch tensor), each num_host_blocks blocks laid out like the device
 * caches.  pairs: device int32 [num_pairs][2].  to_host != 0: pairs are
 * (device block, host block) and each host block's K and V become the device
 * block's; to_host == 0: pairs are (host block, device block) and the other
 * way round.  Pairs with ids out of range are skipped.  The kernel reads and
 * writes the host memory through its device mapping, asynchronously on
 * `stream`: the host buffers must stay alive and untouched until the stream
 * has passed it.  PA_ERR_INVALID_ARG if a host buffer is not pinned memory the
 * device can address; num_pairs in [0, 65535]. */
pa_status pa_swap_blocks(void *k_cache, void *v_cache, void *host_k, void *host_v,
                         int32_t num_host_blocks, const int32_t *pairs, int32_t num_pairs,
                         int32_t to_host, const pa_kv_desc *desc, void *stream);

/* One decode step with the step's append folded in: the same result, cache
 * bytes and output bits as
 *   pa_cache_append(k_new, v_new, k_cache, v_cache, slot_mapping, num_seqs, ...)
 *   pa_decode(q, k_cache, v_cache, ...)
 * issued in that order, with one launch fewer ([devto] §1: each step appends
 * the new token's K and V, then attends over all cached tokens, itself
 * included).  Token b of k_new / v_new ([num_seqs][Hkv][D], q's dtype) is
 * sequence b's token at position seq_lens[b] - 1; slot_mapping[b] must be
 * that position's cache slot (what pa_seq_append_slots returned for it) or
 * negative (nothing is written and the cache slot is read as it is).  With
 * the MFMA kernel the wave that reads a sequence's last block writes the
 * token there first; a row whose slot is neither negative nor that slot is
 * written as NaN, and its token is not stored; a sequence whose length is out
 * of range stores nothing.  With the VALU kernel the append is a separate
 * launch.  Other arguments and errors as for pa_decode; k_scale / v_scale
 * are also the FP8 quantisation scales as in pa_cache_append. */
pa_status pa_decode_append(const void *q, const void *k_new, const void *v_new,
                           const int32_t *slot_mapping, void *k_cache, void *v_cache,
                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *seq_lens, const int32_t *seq_starts,
                           const int32_t *seq_shared, int32_t num_seqs, int32_t max_seq_len,
                           float scale, float k_scale, float v_scale,
                           void *out, void *workspace, size_t workspace_bytes,
                           int32_t partition_size, const pa_kv_desc *desc, void *stream);

/* A partitioned pa_decode as two launches (same arguments as pa_decode;
 * partition_size must not be PA_PARTITION_NONE and `workspace` as for
 * pa_decode).  pa_decode_partials runs the per-partition kernel and leaves
 * each partition's softmax state (running max, sum, unnormalised output) in
 * the workspace; with PA_PARTITION_BALANCED it also writes to `out` the rows
 * of every (sequence, KV head) that one work item covers whole.
 * pa_decode_merge combines the partial states into the other rows of `out`;
 * it takes the same seq_shared (the share plan, or NULL), since where the
 * partial states lie depends on it.
 * Issued in this order on one stream, with the same `out`, they compute what
 * pa_decode computes, bit for bit (it launches the same two kernels); a caller
 * may time or schedule the two separately.  `out` must not be NULL
 * (PA_ERR_INVALID_ARG). */
pa_status pa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *seq_lens, const int32_t *seq_starts,
                             const int32_t *seq_shared, int32_t num_seqs, int32_t max_seq_len,
                             float scale, float k_scale, float v_scale, void *out,
                             void *workspace, size_t workspace_bytes, int32_t partition_size,
                             const pa_kv_desc *desc, void *stream);
pa_status pa_decode_merge(const int32_t *seq_lens, const int32_t *seq_shared, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t max_seq_len, void *out,
                          const void *workspace, size_t workspace_bytes, int32_t partition_size,
                          const pa_kv_desc *desc, void *stream);

/* ------------------------------------------------------------------------ */
/* Measurement.                                                             */
/* ------------------------------------------------------------------------ */

/* Read ceiling of the device: one launch that reads the `bytes` bytes at buf
 * (device memory, 16-byte aligned, a multiple of 16 bytes) once, 16 bytes per
 * lane per load, `loads_in_flight` (4, 8 or 16) loads issued before their
 * values are used, over `workgroups` workgroups of 256 threads, with the
 * nontemporal hint when `nontemporal` is non-zero, and, when `one_per_cu` is
 * non-zero, an LDS request that lets a compute unit hold one workgroup (one
 * wave per SIMD, as the balanced decode launch runs).  The values are folded
 * and nothing is written except, at most, one word at `sink` (device memory,
 * 4 bytes).  The rate it reaches is the practical roof of a kernel whose time
 * is its reads: decode is bound by how fast the cache is read (vaibhawkumar.in,
 * "Why fragmentation matters more than bandwidth").  Asynchronous on
 * `stream`; PA_ERR_INVALID_ARG for the shapes above, PA_ERR_HIP if the launch
 * fails. */
pa_status pa_read_probe(const void *buf, size_t bytes, int32_t loads_in_flight,
                        int32_t workgroups, int32_t nontemporal, int32_t one_per_cu, void *sink,
                        void *stream);

/* ------------------------------------------------------------------------ */
/* Allocation-free decode step.                                             */
/* ------------------------------------------------------------------------ */

/* Scratch the library holds on each GPU for pa_decode_append_noalloc. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* For callers that cannot allocate device memory at the time of the call:
 * code being captured into a HIP graph, tight serving loops, or harnesses
 * that forbid hipMalloc.  The same step as pa_decode_append, with the same
 * arguments except the workspace: the partial softmax states of the
 * partitioned modes go to a scratch array of PA_NOALLOC_SCRATCH_BYTES that the
 * library holds in each GPU's memory from its first use on that GPU until the
 * process ends.  The call allocates and frees nothing (no hipMalloc, hipFree
 * or allocating library routine); the caller still passes every input and
 * output.  The scratch needs no initial contents.
 *   Limit: PA_ERR_CAPACITY, before anything is launched, when the partial
 *   states exceed PA_NOALLOC_SCRATCH_BYTES: those of
 *   pa_decode_workspace_bytes(desc, num_seqs, max_seq_len, partition_size),
 *   or with PA_PARTITION_BALANCED those of a launch without a share plan's
 *   rows (that holds up to about 7,000 (sequence, KV head) pairs at group 4
 *   and head_dim 128); a share plan's rows are read once per KV head only
 *   when their room fits in the scratch as well.  PA_PARTITION_NONE needs no
 *   scratch.
 *   Sharing: every call on one GPU uses that GPU's one scratch array, and it
 *   keeps the last call's contents.  Calls that may overlap on one GPU (on
 *   different streams, or from different threads) race on it and give wrong
 *   results; issue them on one stream, or use pa_decode_append with a
 *   workspace of their own.
 * Errors otherwise as for pa_decode_append, plus PA_ERR_HIP if the scratch's
 * device address cannot be found. */
pa_status pa_decode_append_noalloc(const void *q, const void *k_new, const void *v_new,
                                   const int32_t *slot_mapping, void *k_cache, void *v_cache,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *seq_lens, const int32_t *seq_starts,
                                   const int32_t *seq_shared, int32_t num_seqs,
                                   int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                   void *out, int32_t partition_size, const pa_kv_desc *desc,
                                   void *stream);

/* Message describing the last failure on this thread ("" if none). */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
