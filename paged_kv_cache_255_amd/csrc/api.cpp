// C ABI of the device calls: argument checks, kernel choice, launches.
// The block pool calls live in pool.cpp; pa.h documents every entry point.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "pa.h"
#include "pa_internal.hpp"
#include "work.hpp"

namespace pa {

hipError_t launch_decode_valu(const DecodeArgs &a, pa_dtype qt, pa_dtype kt, int D,
                              int32_t num_items, hipStream_t s);
bool valu_supports(pa_dtype qt, pa_dtype kt, int D, int G);
hipError_t launch_decode_mfma(const DecodeArgs &a, pa_dtype qt, pa_dtype kt, int D,
                              int32_t num_items, hipStream_t s);
bool mfma_supports(pa_dtype qt, pa_dtype kt, int D, int G);
int mfma_waves_per_cu(pa_dtype qt, pa_dtype kt, int D);
hipError_t launch_merge(const DecodeArgs &a, pa_dtype qt, int D, hipStream_t s);
hipError_t launch_append(const void *k, const void *v, void *kc, void *vc, const int32_t *slots,
                         int32_t T, int32_t H, int32_t NB, int32_t TS, int D, pa_dtype qt,
                         pa_dtype kt, float k_inv, float v_inv, hipStream_t s);
hipError_t launch_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                              const int32_t *pairs, int32_t num_pairs, int64_t block_bytes,
                              int32_t n_src, int32_t n_dst, hipStream_t s);
hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs,
                              int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                              hipStream_t s);
hipError_t launch_read_probe(const void *buf, int64_t pieces, int32_t loads, int32_t wgs,
                             bool stream, bool one_per_cu, uint32_t *sink, hipStream_t s);

namespace {

pa_status hip_fail(hipError_t e, const char *what)
{
    std::string m = std::string(what) + ": " + hipGetErrorString(e);
    return fail(PA_ERR_HIP, m.c_str());
}

// hipGetLastError reports the thread's last failed HIP call of any caller in
// the process (a framework probing devices may leave one behind), so the
// launchers clear it first: the check after a launch then sees that launch.
void clear_stale_hip_error() { (void)hipGetLastError(); }

bool valid_dtype(pa_dtype t) { return dtype_bytes(t) != 0; }

// log2(block_size / 16) for the block sizes the kernels take, else -1.
int tile_shift_of(int32_t block_size)
{
    for (int sh = 0; sh <= 4; ++sh)
        if (block_size == (kTile << sh))
            return sh;
    return -1;
}

// The (q, kv) storage pairs the path defines: matching 16/32-bit types, or
// FP8 storage under 16-bit activations.
bool valid_pair(pa_dtype q, pa_dtype kv)
{
    if (q == kv)
        return q != PA_FP8_E4M3;
    return kv == PA_FP8_E4M3 && (q == PA_BF16 || q == PA_F16);
}

pa_status check_desc(const pa_kv_desc *d)
{
    if (!d)
        return fail(PA_ERR_INVALID_ARG, "null desc");
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    if (d->num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "num_blocks must be positive");
    if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_dtype))
        return fail(PA_ERR_INVALID_ARG, "unknown dtype");
    if (!valid_pair(d->q_dtype, d->kv_dtype))
        return fail(PA_ERR_UNSUPPORTED, "unsupported (q, kv) dtype pair");
    if (tile_shift_of(d->block_size) < 0)
        return fail(PA_ERR_UNSUPPORTED, "block_size must be 16, 32, 64, 128 or 256");
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if ((int64_t)d->num_blocks * d->block_size > INT32_MAX)
        return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size overflows int32 slots");
    if ((int64_t)d->num_blocks * d->num_kv_heads * d->block_size * d->head_dim > (int64_t)1 << 40)
        return fail(PA_ERR_INVALID_ARG, "cache too large");
    return PA_OK;
}

// Waves the balanced split uses on the current device: all the waves of the
// balanced kernel that the GPU holds at once (CUs x resident waves per CU),
// so every run starts at launch and they finish together.  0 if unknown.
int32_t balanced_waves(const pa_kv_desc *d)
{
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int>, int32_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    const auto key = std::make_tuple(dev, (int)d->q_dtype, (int)d->kv_dtype, d->head_dim);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int32_t w = cus * mfma_waves_per_cu(d->q_dtype, d->kv_dtype, d->head_dim);
    cache[key] = w;
    return w;
}

// The kernel a launch runs: PA_KERNEL_AUTO takes MFMA where it applies.
int resolved_kernel(const pa_kv_desc *d)
{
    const int G = d->num_q_heads / d->num_kv_heads;
    if (d->kernel != PA_KERNEL_AUTO)
        return d->kernel;
    return mfma_supports(d->q_dtype, d->kv_dtype, d->head_dim, G) ? PA_KERNEL_MFMA
                                                                    : PA_KERNEL_VALU;
}

// Whether a balanced launch of this shape can read a share plan's groups once
// per KV head: the MFMA kernel, 16 / G members per 16-column tile, and a
// G x D the one-wave segment merge handles (a power-of-two multiple of 256 up
// to 2048).
bool prefix_capable(const pa_kv_desc *d)
{
    const int G = d->num_q_heads / d->num_kv_heads;
    const int gd = G * d->head_dim;
    return resolved_kernel(d) == PA_KERNEL_MFMA &&
           mfma_supports(d->q_dtype, d->kv_dtype, d->head_dim, G) && 16 % G == 0 &&
           gd % 256 == 0 && (gd / 256 == 1 || gd / 256 == 2 || gd / 256 == 4 || gd / 256 == 8);
}

// Partial-state slots of a balanced launch with W waves: one per (run,
// sequence segment) pair, W + B Hkv; with prefix rows, (W + Hkv B / 2) row
// pieces of 4 x 16 / G member slots each on top.
int64_t balanced_seq_slots(const pa_kv_desc *d, int32_t W, int32_t num_seqs)
{
    return (int64_t)W + (int64_t)num_seqs * d->num_kv_heads;
}
int64_t balanced_row_slots(const pa_kv_desc *d, int32_t W, int32_t num_seqs)
{
    const int G = d->num_q_heads / d->num_kv_heads;
    return ((int64_t)W + (int64_t)d->num_kv_heads * (num_seqs / 2)) * (4 * (16 / G));
}
size_t slot_bytes(const pa_kv_desc *d, int64_t slots)
{
    const int64_t G = d->num_q_heads / d->num_kv_heads;
    return (size_t)(slots * G * (2 + d->head_dim) * (int64_t)sizeof(float));
}
// With prefix rows the workspace also holds, after the slots (at a 256-byte
// boundary), the decode's record of where each segment's parts are: four
// int32 per (KV head, sequence).
size_t seg_dir_offset(const pa_kv_desc *d, int64_t slots)
{
    return (slot_bytes(d, slots) + 255) / 256 * 256;
}
size_t prefix_bytes(const pa_kv_desc *d, int64_t slots, int32_t num_seqs)
{
    return seg_dir_offset(d, slots) + (size_t)num_seqs * d->num_kv_heads * 4 * sizeof(int32_t);
}

int32_t parts_for(int32_t max_seq_len, int32_t partition)
{
    if (partition <= 0)
        return 1;
    int32_t p = (max_seq_len + partition - 1) / partition;
    return p < 1 ? 1 : p;
}

} // namespace

} // namespace pa

using namespace pa;

extern "C" {

pa_status pa_cache_append(const void *k, const void *v, void *k_cache, void *v_cache,
                          const int32_t *slot_mapping, int32_t num_tokens, const pa_kv_desc *desc,
                          float k_scale, float v_scale, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK)
        return st;
    if (num_tokens < 0)
        return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_tokens == 0)
        return PA_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    float k_inv = 1.f, v_inv = 1.f;
    if (desc->kv_dtype == PA_FP8_E4M3) {
        if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == INFINITY || v_scale == INFINITY)
            return fail(PA_ERR_INVALID_ARG, "FP8 scales must be positive and finite");
        k_inv = 1.0f / k_scale;
        v_inv = 1.0f / v_scale;
    }
    clear_stale_hip_error();
    hipError_t e = launch_append(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                 desc->num_kv_heads, desc->num_blocks,
                                 tile_shift_of(desc->block_size), desc->head_dim,
                                 desc->q_dtype, desc->kv_dtype, k_inv, v_inv,
                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "cache append launch");
    return PA_OK;
}

pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int32_t num_pairs,
                         const pa_kv_desc *desc, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK)
        return st;
    if (num_pairs < 0 || num_pairs > 65535)
        return fail(PA_ERR_INVALID_ARG, "num_pairs must be in [0, 65535]");
    if (num_pairs == 0)
        return PA_OK;
    if (!k_cache || !v_cache || !pairs)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    const int64_t block_bytes = (int64_t)desc->block_size * desc->num_kv_heads * desc->head_dim *
                                dtype_bytes(desc->kv_dtype);
    clear_stale_hip_error();
    hipError_t e = launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, block_bytes,
                                      desc->num_blocks, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "block copy launch");
    return PA_OK;
}

pa_status pa_swap_blocks(void *k_cache, void *v_cache, void *host_k, void *host_v,
                         int32_t num_host_blocks, const int32_t *pairs, int32_t num_pairs,
                         int32_t to_host, const pa_kv_desc *desc, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK)
        return st;
    if (num_pairs < 0 || num_pairs > 65535 || num_host_blocks < 0)
        return fail(PA_ERR_INVALID_ARG, "num_pairs must be in [0, 65535]");
    if (num_pairs == 0)
        return PA_OK;
    if (!k_cache || !v_cache || !host_k || !host_v || !pairs)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    // the host buffers must be pinned memory the device can address
    void *dk = nullptr, *dv = nullptr;
    if (hipHostGetDevicePointer(&dk, host_k, 0) != hipSuccess ||
        hipHostGetDevicePointer(&dv, host_v, 0) != hipSuccess || !dk || !dv) {
        (void)hipGetLastError();
        return fail(PA_ERR_INVALID_ARG, "host swap buffers must be pinned (hipHostMalloc) memory");
    }
    const int64_t block_bytes = (int64_t)desc->block_size * desc->num_kv_heads * desc->head_dim *
                                dtype_bytes(desc->kv_dtype);
    clear_stale_hip_error();
    hipError_t e = to_host ? launch_swap_blocks(k_cache, v_cache, dk, dv, pairs, num_pairs,
                                                block_bytes, desc->num_blocks, num_host_blocks,
                                                static_cast<hipStream_t>(stream))
                           : launch_swap_blocks(dk, dv, k_cache, v_cache, pairs, num_pairs,
                                                block_bytes, num_host_blocks, desc->num_blocks,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "swap launch");
    return PA_OK;
}

pa_status pa_read_probe(const void *buf, size_t bytes, int32_t loads_in_flight,
                        int32_t workgroups, int32_t nontemporal, int32_t one_per_cu, void *sink,
                        void *stream)
{
    if (!buf || !sink)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return fail(PA_ERR_INVALID_ARG, "buffer must be 16-byte aligned, a positive multiple "
                                        "of 16 bytes");
    if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16)
        return fail(PA_ERR_INVALID_ARG, "loads_in_flight must be 4, 8 or 16");
    if (workgroups < 1 || workgroups > (1 << 20))
        return fail(PA_ERR_INVALID_ARG, "workgroups must be in [1, 2^20]");
    clear_stale_hip_error();
    hipError_t e = launch_read_probe(buf, (int64_t)(bytes / 16), loads_in_flight, workgroups,
                                     nontemporal != 0, one_per_cu != 0,
                                     static_cast<uint32_t *>(sink),
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "read probe launch");
    return PA_OK;
}

size_t pa_decode_workspace_bytes(const pa_kv_desc *desc, int32_t num_seqs, int32_t max_seq_len,
                                 int32_t partition_size)
{
    if (!desc || num_seqs <= 0 || max_seq_len < 0 || partition_size == 0 ||
        partition_size < PA_PARTITION_BALANCED || desc->num_kv_heads <= 0 ||
        desc->num_q_heads <= 0 || desc->head_dim <= 0)
        return 0;
    int64_t slots;
    if (partition_size == PA_PARTITION_BALANCED) {
        const int32_t W = balanced_waves(desc);
        if (W <= 0)
            return 0;
        slots = balanced_seq_slots(desc, W, num_seqs);
        if (prefix_capable(desc))
            return prefix_bytes(desc, slots + balanced_row_slots(desc, W, num_seqs), num_seqs);
    } else {
        slots = (int64_t)num_seqs * desc->num_kv_heads * parts_for(max_seq_len, partition_size);
    }
    return slot_bytes(desc, slots);
}

int32_t pa_decode_balanced_waves(const pa_kv_desc *desc)
{
    if (check_desc(desc) != PA_OK || resolved_kernel(desc) != PA_KERNEL_MFMA)
        return 0;
    const int G = desc->num_q_heads / desc->num_kv_heads;
    if (!mfma_supports(desc->q_dtype, desc->kv_dtype, desc->head_dim, G))
        return 0;
    return balanced_waves(desc);
}

} // extern "C"

namespace {

// Partial-state scratch of pa_decode_append_noalloc: one array in each GPU's
// memory, for the life of the process.  In host code `scratch` names a host
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is passed on.
constexpr size_t kNoallocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

pa_status noalloc_scratch(void **out)
{
    static std::mutex mu;
    static std::map<int, void *> addr; // device -> address of its scratch
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "no current device for the allocation-free scratch");
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr.find(dev);
    if (it == addr.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                            "device address of the allocation-free scratch");
        }
        it = addr.emplace(dev, p).first;
    }
    *out = it->second;
    return PA_OK;
}

enum Phase { kAll, kPartials, kMerge };

// The step's new tokens when pa_decode_append is the caller (else all null).
struct NewTokens {
    const void *k = nullptr;
    const void *v = nullptr;
    const int32_t *slots = nullptr;
};

pa_status decode_impl(Phase phase, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *seq_lens, const int32_t *seq_starts,
                      const int32_t *seq_shared, int32_t num_seqs,
                      int32_t max_seq_len, float scale, float k_scale, float v_scale, void *out,
                      void *workspace, size_t workspace_bytes, int32_t partition_size,
                      const pa_kv_desc *desc, void *stream, const NewTokens &nt = NewTokens{})
{
    pa_status st = check_desc(desc);
    if (st != PA_OK)
        return st;
    if (num_seqs < 0 || max_seq_len < 0 || max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARG, "negative size");
    if (num_seqs == 0)
        return PA_OK;
    // every phase may write rows of out: the balanced partials kernel writes
    // the rows one work item covers whole
    if (!seq_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (phase != kMerge) {
        if (!q || !k_cache || !v_cache || !block_tables)
            return fail(PA_ERR_INVALID_ARG, "null pointer");
        if (q == out)
            return fail(PA_ERR_INVALID_ARG, "out may not alias q");
        if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
            return fail(PA_ERR_INVALID_ARG, "scales must be positive");
    }
    const bool balanced = partition_size == PA_PARTITION_BALANCED;
    if (!balanced && (partition_size < 0 || partition_size % kTile != 0))
        return fail(PA_ERR_INVALID_ARG,
                    "partition_size must be 0, PA_PARTITION_BALANCED or a positive multiple of 16");
    if (phase != kAll && partition_size == 0)
        return fail(PA_ERR_INVALID_ARG, "partials/merge need a partitioned mode");
    if ((int64_t)max_blocks_per_seq * desc->block_size < (int64_t)max_seq_len)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len exceeds max_blocks_per_seq * block_size");

    const int D = desc->head_dim;
    const int G = desc->num_q_heads / desc->num_kv_heads;
    DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.seq_starts = seq_starts;
    a.share = seq_shared;
    a.out = out;
    a.ws = static_cast<float *>(workspace);
    a.num_seqs = num_seqs;
    a.num_q_heads = desc->num_q_heads;
    a.num_kv_heads = desc->num_kv_heads;
    a.group = G;
    a.num_blocks = desc->num_blocks;
    a.tile_shift = tile_shift_of(desc->block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_seq_len = max_seq_len;
    a.partition = partition_size;
    a.max_parts = balanced ? 1 : parts_for(max_seq_len, partition_size);
    a.score_scale = scale * k_scale * kLog2e;
    a.v_scale = v_scale;
    const bool appending = nt.slots != nullptr;
    if (appending) {
        if (!nt.k || !nt.v)
            return fail(PA_ERR_INVALID_ARG, "null pointer");
        if (nt.k == out || nt.v == out)
            return fail(PA_ERR_INVALID_ARG, "out may not alias the new tokens");
        a.k_new = nt.k;
        a.v_new = nt.v;
        a.slots = nt.slots;
        a.k_inv = desc->kv_dtype == PA_FP8_E4M3 ? 1.0f / k_scale : 1.f;
        a.v_inv = desc->kv_dtype == PA_FP8_E4M3 ? 1.0f / v_scale : 1.f;
    }

    const int kernel = resolved_kernel(desc);
    int64_t items64;
    size_t need = 0;
    if (balanced) {
        if (kernel != PA_KERNEL_MFMA)
            return fail(PA_ERR_UNSUPPORTED, "balanced partitioning needs the MFMA kernel");
        a.waves = balanced_waves(desc);
        if (a.waves <= 0)
            return fail(PA_ERR_HIP, "could not query the device for the balanced split");
        items64 = a.waves;
        a.num_slots = balanced_seq_slots(desc, a.waves, num_seqs);
        need = slot_bytes(desc, a.num_slots);
        // prefix rows: with a plan, a capable shape and room for their
        // partial states after the sequences' slots (the same decision for
        // the partials and the merge launch; a plan groups no sequence with
        // a slid window)
        const int64_t with_rows = a.num_slots + balanced_row_slots(desc, a.waves, num_seqs);
        if (seq_shared && prefix_capable(desc) && with_rows < ((int64_t)1 << 31) &&
            workspace_bytes >= prefix_bytes(desc, with_rows, num_seqs)) {
            a.prefix = 1;
            a.prefix_base = a.num_slots;
            a.num_slots = with_rows;
            a.seg_dir = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                    seg_dir_offset(desc, with_rows));
        }
    } else {
        items64 = (int64_t)num_seqs * desc->num_kv_heads * a.max_parts;
        a.waves = 0;
        a.num_slots = items64;
        if (partition_size != 0)
            need = pa_decode_workspace_bytes(desc, num_seqs, max_seq_len, partition_size);
    }
    if (items64 > (int64_t)1 << 30)
        return fail(PA_ERR_INVALID_ARG, "too many work items");
    const int32_t items = (int32_t)items64;
    if (partition_size != 0 && (!workspace || need == 0 || workspace_bytes < need))
        return fail(PA_ERR_CAPACITY, "workspace smaller than pa_decode_workspace_bytes()");
    if (partition_size != 0 && (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
        return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    clear_stale_hip_error();
    if (appending) {
        if (desc->kv_dtype == PA_FP8_E4M3 && (k_scale == INFINITY || v_scale == INFINITY))
            return fail(PA_ERR_INVALID_ARG, "FP8 scales must be positive and finite");
        if (kernel == PA_KERNEL_MFMA) {
            a.append = 1; // the decode kernel writes the tokens itself
        } else {
            e = launch_append(nt.k, nt.v, const_cast<void *>(k_cache), const_cast<void *>(v_cache),
                              nt.slots, num_seqs, desc->num_kv_heads, desc->num_blocks,
                              a.tile_shift, D, desc->q_dtype, desc->kv_dtype, a.k_inv, a.v_inv,
                              s);
            if (e != hipSuccess)
                return hip_fail(e, "cache append launch");
        }
    }
    if (phase != kMerge) {
        if (kernel == PA_KERNEL_MFMA) {
            if (!mfma_supports(desc->q_dtype, desc->kv_dtype, D, G))
                return fail(PA_ERR_UNSUPPORTED, "MFMA kernel: needs 16-bit q and a group of <= 16");
            e = launch_decode_mfma(a, desc->q_dtype, desc->kv_dtype, D, items, s);
        } else if (kernel == PA_KERNEL_VALU) {
            if (!valu_supports(desc->q_dtype, desc->kv_dtype, D, G))
                return fail(PA_ERR_UNSUPPORTED,
                            "VALU kernel: unsupported (dtype, head_dim, group)");
            e = launch_decode_valu(a, desc->q_dtype, desc->kv_dtype, D, items, s);
        } else {
            return fail(PA_ERR_INVALID_ARG, "unknown kernel choice");
        }
        if (e != hipSuccess)
            return hip_fail(e, "decode launch");
    }
    if (phase != kPartials && partition_size != 0) {
        e = launch_merge(a, desc->q_dtype, D, s);
        if (e != hipSuccess)
            return hip_fail(e, "merge launch");
    }
    return PA_OK;
}

} // namespace

extern "C" {

pa_status pa_decode(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *seq_lens, const int32_t *seq_starts,
                    const int32_t *seq_shared, int32_t num_seqs, int32_t max_seq_len,
                    float scale, float k_scale, float v_scale, void *out,
                    void *workspace, size_t workspace_bytes, int32_t partition_size,
                    const pa_kv_desc *desc, void *stream)
{
    return decode_impl(kAll, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                       seq_starts, seq_shared, num_seqs, max_seq_len, scale, k_scale, v_scale,
                       out, workspace, workspace_bytes, partition_size, desc, stream);
}

pa_status pa_decode_append(const void *q, const void *k_new, const void *v_new,
                           const int32_t *slot_mapping, void *k_cache, void *v_cache,
                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *seq_lens, const int32_t *seq_starts,
                           const int32_t *seq_shared, int32_t num_seqs, int32_t max_seq_len,
                           float scale, float k_scale, float v_scale,
                           void *out, void *workspace, size_t workspace_bytes,
                           int32_t partition_size, const pa_kv_desc *desc, void *stream)
{
    if (num_seqs > 0 && !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    NewTokens nt;
    nt.k = k_new;
    nt.v = v_new;
    nt.slots = slot_mapping;
    return decode_impl(kAll, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                       seq_starts, seq_shared, num_seqs, max_seq_len, scale, k_scale, v_scale,
                       out, workspace, workspace_bytes, partition_size, desc, stream, nt);
}

pa_status pa_decode_append_noalloc(const void *q, const void *k_new, const void *v_new,
                                   const int32_t *slot_mapping, void *k_cache, void *v_cache,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *seq_lens, const int32_t *seq_starts,
                                   const int32_t *seq_shared, int32_t num_seqs,
                                   int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                   void *out, int32_t partition_size, const pa_kv_desc *desc,
                                   void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK)
        return st;
    if (num_seqs > 0 && !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (num_seqs > 0 && partition_size != PA_PARTITION_NONE) {
        // the room without prefix rows; the scratch is offered whole, so a
        // plan's rows are read when their room fits as well
        size_t need = pa_decode_workspace_bytes(desc, num_seqs, max_seq_len, partition_size);
        if (need != 0 && partition_size == PA_PARTITION_BALANCED)
            need = slot_bytes(desc, balanced_seq_slots(desc, balanced_waves(desc), num_seqs));
        if (need == 0)
            return fail(PA_ERR_INVALID_ARG, "bad partition_size or shape (or no device to size "
                                            "the balanced split for)");
        if (need > kNoallocScratchBytes) {
            char m[160];
            std::snprintf(m, sizeof m,
                          "this call needs %zu bytes of partial states; the allocation-free "
                          "entry point holds %zu",
                          need, (size_t)kNoallocScratchBytes);
            return fail(PA_ERR_CAPACITY, m);
        }
        st = noalloc_scratch(&ws);
        if (st != PA_OK)
            return st;
        ws_bytes = kNoallocScratchBytes;
    }
    NewTokens nt;
    nt.k = k_new;
    nt.v = v_new;
    nt.slots = slot_mapping;
    return decode_impl(kAll, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                       seq_starts, seq_shared, num_seqs, max_seq_len, scale, k_scale, v_scale,
                       out, ws, ws_bytes, partition_size, desc, stream, nt);
}

pa_status pa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *seq_lens, const int32_t *seq_starts,
                             const int32_t *seq_shared, int32_t num_seqs, int32_t max_seq_len,
                             float scale, float k_scale, float v_scale, void *out,
                             void *workspace, size_t workspace_bytes, int32_t partition_size,
                             const pa_kv_desc *desc, void *stream)
{
    return decode_impl(kPartials, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       seq_lens, seq_starts, seq_shared, num_seqs, max_seq_len, scale, k_scale,
                       v_scale, out, workspace, workspace_bytes, partition_size, desc, stream);
}

pa_status pa_decode_merge(const int32_t *seq_lens, const int32_t *seq_shared, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t max_seq_len, void *out,
                          const void *workspace, size_t workspace_bytes, int32_t partition_size,
                          const pa_kv_desc *desc, void *stream)
{
    return decode_impl(kMerge, nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq, seq_lens,
                       nullptr, seq_shared, num_seqs, max_seq_len, 1.f, 1.f, 1.f, out,
                       const_cast<void *>(workspace), workspace_bytes, partition_size, desc,
                       stream);
}

} // extern "C"
