#!/usr/bin/env python3
"""PagedAttention decode benchmark on one MI355X.

Default workload: one decode step of a Llama-3-8B-shaped attention layer
(32 query heads on 8 KV heads, head_dim 128, bf16, 16-token blocks) for a
batch of 32 sequences with lengths uniform in [512, 4096], blocks scattered
over a pool 1.25x the size they need (dev.to, "Why LLMs Run Out of VRAM...",
§2 Example 2 and §4).

A timed step is the whole device-side hot path for the batch:
pa_decode_append, which appends the new token's K/V and decodes in one
kernel (then the merge kernel in the partitioned modes); --separate-append
times pa_cache_append + pa_decode instead.  Inputs are resident in HBM when
timing starts, the per-step metadata included: the host allocator
(pa_seq_append_slots_batch: one new slot per sequence, a new block at every
16th token; pa_export_block_tables) runs for every step first and the
tables, lengths and slots of all steps go to the device in one copy.
--upload-per-step instead runs the allocator and a pinned-memory copy of that
step's metadata inside every timed step (the host-inclusive rate).  The
caches are rotated over R replicas (one per step, like the layers of a
model) so that the working set exceeds the 256 MB Infinity Cache and reads
come from HBM.

Printed: one JSON line.  `value` is KV-read GB/s over whole steps
(algorithmic bytes: every valid token's K and V row of each KV head once);
`roofline` is for the decode kernel alone: K launches of it back to back on
the last step's inputs, between two events; `cpu_baseline` times the CPU
oracle on a bounded sample.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload 2..5 (2 = headline)")
    ap.add_argument("--partition", type=int, default=None,
                    help="tokens per work item (0 = single pass, -1 = balanced)")
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--block-size", type=int, default=16, choices=[16, 32, 64, 128, 256],
                    help="tokens per physical block (the workloads use 16)")
    ap.add_argument("--replicas", type=int, default=None, help="cache replicas rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only sweep the read-ceiling probe (pa_read_probe: loads in flight, "
                         "workgroups, nontemporal hint) over a 4 GiB buffer, print one JSON "
                         "line per setting and exit")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the read-ceiling probe in a decode run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device-to-device copies of 1 GiB (calibrates the HBM "
                         "byte counters a profiler reports) and exit")
    ap.add_argument("--no-reuse-hint", action="store_true",
                    help="pass no share plan (seq_shared): every block is read with streaming "
                         "loads and every sequence reads its shared blocks itself")
    ap.add_argument("--separate-append", action="store_true",
                    help="a step calls pa_cache_append then pa_decode instead of "
                         "pa_decode_append")
    ap.add_argument("--upload-per-step", action="store_true",
                    help="run the host allocator and copy the step's metadata inside each "
                         "timed step")
    ap.add_argument("--feature", choices=["copy", "swap", "window", "prefix", "prefill"],
                    default=None,
                    help="measure one of the paths beside the decode step on the workload's "
                         "shapes (block copies of copy on write, swap transfers, windowed "
                         "decode, prefix-cache host work, the prefill append of --config) "
                         "and print one JSON line for it")
    ap.add_argument("--traffic-record", nargs=5, default=None,
                    metavar=("BENCH_LINE", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                             "COPY_WRITE_CSV"),
                    help="write profiles/decode_mfma_balanced_<workload>.traffic.json from "
                         "the JSON line of a bench run and the rocprofv3 --pmc FETCH_SIZE and "
                         "WRITE_SIZE counter CSVs of that same command and of "
                         "--copy-calibration, then exit (no GPU needed)")
    return ap.parse_args()


def main():
    args = parse()
    if args.traffic_record:
        write_traffic_record(*args.traffic_record)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              "shards by sequence or KV head with no collective, see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_255_amd as pa
    import workloads
    from paged_kv_cache_255_amd.plan import execute_plan

    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.read_ceiling:
        read_ceiling_sweep(torch, pa, args)
        return
    if args.feature:
        FEATURES[args.feature](args, torch, pa, workloads, execute_plan)
        return

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    w = workloads.config(args.config, block_size=args.block_size)
    bs = w.block_size
    partition = w.partition_size if args.partition is None else args.partition
    kernel = {"auto": pa.KERNEL_AUTO, "valu": pa.KERNEL_VALU, "mfma": pa.KERNEL_MFMA}[args.kernel]
    B, Hq, Hkv, D, L = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_layers
    eb = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    K, W = args.steps, args.warmup
    total_steps = W + K

    # pool with room for every token the steps append
    grow_blocks = B * (math.ceil((total_steps + 1) / bs) + 1)
    nblocks = w.num_blocks + grow_blocks
    pool = pa.pa_block_pool_init(nblocks, Hkv, D, w.kv_dtype, block_size=bs,
                                 shuffle_seed=w.shuffle_seeds[0])
    ids, pre_slots = execute_plan(pool, w.ops)
    dec = np.array([ids[s] for s in w.decode_seqs], dtype=np.int32)
    lens0 = np.array(w.decode_lengths(), dtype=np.int64) - 1  # before the first step
    max_len = int(lens0.max()) + total_steps
    maxb = math.ceil(max_len / bs)

    step_bytes_1 = Hkv * D * 2 * eb * L  # per token
    per_replica = nblocks * Hkv * bs * D * eb * 2 * L
    R = args.replicas or max(1, math.ceil(1.2e9 / max(1, int(lens0.sum()) * step_bytes_1)))
    log(f"[bench] {w.name}: B={B} Hq={Hq} Hkv={Hkv} D={D} layers={L} kv={w.kv_dtype} "
        f"pool={nblocks} blocks, replicas={R} ({R * per_replica / 1e9:.2f} GB of cache), "
        f"partition={partition} kernel={args.kernel} block_size={bs}")

    # caches: every replica and layer gets the same prefill through the append kernel
    desc = pa.kv_desc(Hq, Hkv, D, nblocks, w.q_dtype, w.kv_dtype, block_size=bs, kernel=kernel)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "e4m3": torch.uint8}[w.kv_dtype]
    nelem = nblocks * Hkv * bs * D
    caches = []  # index layer * R + replica
    d_pre = torch.from_numpy(pre_slots).to(dev)
    ks = vs = 1.0
    for layer in range(L):
        k_pre, v_pre = workloads.prefill_tensors(w, layer, dev)
        if w.kv_dtype == "e4m3" and layer == 0:
            ks, vs = workloads.fp8_scale(k_pre), workloads.fp8_scale(v_pre)
        kc = torch.zeros(nelem, dtype=tdt, device=dev)
        vc = torch.zeros(nelem, dtype=tdt, device=dev)
        pa.pa_cache_append(k_pre, v_pre, kc, vc, d_pre, desc, ks, vs)
        caches.append((kc, vc))
        for _ in range(1, R):
            caches.append((kc.clone(), vc.clone()))
        del k_pre, v_pre
    torch.cuda.synchronize()
    q, k_new, v_new = workloads.step_tensors(w, 0, dev)
    out = torch.empty_like(q)
    ws = None
    ws_bytes = 0
    if partition != 0:
        ws_bytes = pa.pa_decode_workspace_bytes(desc, B, max_len, partition)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    # Per-step metadata (slots, tables, lengths, share plan), one row per step.
    plan_off = 4 * (2 * B + B * maxb)  # byte offset of the share plan in a row
    meta_words = B + B * maxb + B + pa.share_plan_words(B)
    lib = pa._lib
    pool_h = pool.handle
    dec_p = dec.ctypes.data

    def host_step(dst_ptr):
        rc = lib.pa_seq_append_slots_batch(pool_h, dec_p, B, 1, dst_ptr)
        rc |= lib.pa_export_block_tables(pool_h, dec_p, B, maxb, dst_ptr + 4 * B,
                                         dst_ptr + 4 * (B + B * maxb), None, None)
        rc |= lib.pa_export_share_plan(pool_h, dec_p, B, dst_ptr + plan_off)
        if rc:
            raise RuntimeError("host step failed: " + pa.pa_last_error())

    upload = args.upload_per_step
    if upload:
        # a pinned staging ring; each step copies its row to the device buffer
        NBUF = 8
        staging = torch.empty((NBUF, meta_words), dtype=torch.int32, pin_memory=True)
        staged = [torch.cuda.Event() for _ in range(NBUF)]  # copy out of staging[buf] done
        d_meta = torch.empty((1, meta_words), dtype=torch.int32, device=dev)
        stage_ptrs = [staging[i].data_ptr() for i in range(NBUF)]
    else:
        # every step's metadata, made by the host allocator up front
        h_meta = torch.empty((total_steps, meta_words), dtype=torch.int32, pin_memory=True)
        for i in range(total_steps):
            host_step(h_meta[i].data_ptr())
        d_meta = h_meta.to(dev)
    meta_row = d_meta.stride(0) * 4

    stream = torch.cuda.current_stream()
    s_h = stream.cuda_stream
    dref = ctypes.byref(desc)
    kc_p = [(c[0].data_ptr(), c[1].data_ptr()) for c in caches]
    qp, kn, vn, op = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), out.data_ptr()
    ws_p = ws.data_ptr() if ws is not None else None
    scale = w.scale
    meta_base = d_meta.data_ptr()

    separate = args.separate_append
    # the share plan goes with the launches when some sequence of the batch
    # shares blocks with another (a plan of zero counts and no groups would
    # add a read for nothing)
    if upload:
        first_plan = pa.pa_export_share_plan(pool, dec)
    else:
        first_plan = h_meta[0].numpy()[plan_off // 4:]
    any_shared = bool(first_plan[1] > 0 or (first_plan[2:2 + B] > 0).any())
    no_hint = args.no_reuse_hint or not any_shared

    def step(i):
        if upload:
            buf = i % NBUF
            if i >= NBUF:
                staged[buf].synchronize()  # the copy that last read this buffer is done
            host_step(stage_ptrs[buf])
            d_meta[0].copy_(staging[buf], non_blocking=True)
            staged[buf].record(stream)
            row = meta_base
        else:
            row = meta_base + i * meta_row
        slots_p, tables_p, lens_p = row, row + 4 * B, row + 4 * (B + B * maxb)
        shared_p = None if no_hint else row + plan_off
        r = i % R
        for layer in range(L):
            kcp, vcp = kc_p[layer * R + r]
            if separate:
                rc = lib.pa_cache_append(kn, vn, kcp, vcp, slots_p, B, dref, ks, vs, s_h)
                rc |= lib.pa_decode(qp, kcp, vcp, tables_p, maxb, lens_p, None, shared_p, B,
                                    max_len, scale, ks, vs, op, ws_p, ws_bytes, partition, dref,
                                    s_h)
            else:
                rc = lib.pa_decode_append(qp, kn, vn, slots_p, kcp, vcp, tables_p, maxb, lens_p,
                                          None, shared_p, B, max_len, scale, ks, vs, op, ws_p,
                                          ws_bytes, partition, dref, s_h)
            if rc:
                raise RuntimeError("launch failed: " + pa.pa_last_error())

    # pass 1 (the headline): K whole steps, nothing recorded between kernels
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(W, W + K):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / K
    last = W + K - 1

    # pass 1b: the same K steps again, an event recorded after each one, for
    # the spread of per-step times (the events themselves may add a little
    # to each step, so the headline stays pass 1's)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    step_ev[0].record()
    for j, i in enumerate(range(W, W + K)):
        step(i)
        step_ev[j + 1].record()
    torch.cuda.synchronize()
    step_us = np.array([step_ev[j].elapsed_time(step_ev[j + 1]) * 1e3 for j in range(K)])

    # pass 2: the decode kernel alone (no append, no merge), K * L launches back
    # to back on the last step's metadata, rotating over the replicas, between
    # two events: an event pair around each single launch would add the
    # queue's dispatch latency to every sample.
    row = meta_base if upload else meta_base + last * meta_row
    tables_p, lens_p = row + 4 * B, row + 4 * (B + B * maxb)
    shared_p = None if no_hint else row + plan_off

    def decode_kernel(r, layer):
        kcp, vcp = kc_p[layer * R + r]
        if partition == 0:
            rc = lib.pa_decode(qp, kcp, vcp, tables_p, maxb, lens_p, None, shared_p, B, max_len,
                               scale, ks, vs, op, None, 0, 0, dref, s_h)
        else:
            rc = lib.pa_decode_partials(qp, kcp, vcp, tables_p, maxb, lens_p, None, shared_p, B,
                                        max_len, scale, ks, vs, op, ws_p, ws_bytes, partition,
                                        dref, s_h)
        if rc:
            raise RuntimeError("launch failed: " + pa.pa_last_error())

    for j in range(min(K, 10)):
        decode_kernel(j % R, 0)
    torch.cuda.synchronize()
    k_start = torch.cuda.Event(enable_timing=True)
    k_end = torch.cuda.Event(enable_timing=True)
    k_start.record()
    for j in range(K):
        for layer in range(L):
            decode_kernel(j % R, layer)
    k_end.record()
    torch.cuda.synchronize()
    kern_us = k_start.elapsed_time(k_end) * 1e3 / (K * L)
    probe = None if args.no_probe else read_probe(torch, pa, dev, reps=max(K, 10))

    # algorithmic KV bytes: step i decodes lens0 + i + 1 tokens per sequence
    tokens = np.array([int((lens0 + i + 1).sum()) for i in range(W, W + K)], dtype=np.float64)
    bytes_steps = tokens * step_bytes_1
    gbs = bytes_steps.sum() / (ms_total * 1e-3) / 1e9
    launch_bytes = int((lens0 + last + 1).sum()) * step_bytes_1 / L  # one layer, last step
    kern_gbs = launch_bytes / (kern_us * 1e-6) / 1e9
    p10, p50, p90 = (float(np.percentile(step_us, x)) for x in (10, 50, 90))
    log(f"[bench] per-step (events after each step): median {p50:.2f} us, p10 {p10:.2f}, "
        f"p90 {p90:.2f}")
    log(f"[bench] {K} steps: {ms_per_step * 1e3:.2f} us/step (wall {wall / K * 1e6:.2f} us), "
        f"{gbs:.1f} GB/s over whole steps; decode kernel {kern_us:.2f} us per launch "
        f"({K * L} back to back), {kern_gbs:.1f} GB/s = {kern_gbs / HBM_PEAK_GBS * 100:.1f}% "
        f"of HBM peak")
    final_meta = (staging[last % NBUF] if upload else h_meta[last]).numpy()
    final_tables = final_meta[B:B + B * maxb].reshape(B, maxb).copy()
    final_lens = final_meta[B + B * maxb:2 * B + B * maxb].copy()
    last_r = last % R
    # bytes of the distinct cache slots the last step reads (shared blocks
    # once): below the algorithmic bytes when sequences share blocks
    used = {}
    for b in range(B):
        n = int(final_lens[b])
        for j in range(-(-n // bs)):
            blk = int(final_tables[b, j])
            used[blk] = max(used.get(blk, 0), min(bs, n - j * bs))
    unique_bytes = sum(used.values()) * step_bytes_1 // L
    unique = None
    if unique_bytes < int(launch_bytes):
        ugbs = unique_bytes / (kern_us * 1e-6) / 1e9
        unique = {"bytes": int(unique_bytes), "achieved": round(ugbs, 1),
                  "frac": round(ugbs / HBM_PEAK_GBS, 4),
                  "how": "distinct cache slots of the last step's tables, per launch"}
        log(f"[bench] distinct KV bytes per launch {unique_bytes / 1e6:.1f} MB "
            f"({ugbs:.1f} GB/s, {ugbs / HBM_PEAK_GBS * 100:.1f}% of HBM peak)")

    # The roofline counts the bytes a launch must bring from HBM: with blocks
    # shared between sequences, each distinct cache slot once.
    roof_bytes = unique_bytes if unique is not None else int(launch_bytes)
    roof_gbs = roof_bytes / (kern_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, caches[last_r][0], caches[last_r][1], q, final_tables,
                           final_lens, nblocks, ks, vs, args.cpu_seconds)

    kname = {0: "auto", 1: "valu", 2: "mfma"}[kernel]
    if kernel == pa.KERNEL_AUTO:
        kname = "auto(mfma)" if w.q_dtype in ("bf16", "f16") else "auto(valu)"
    result = {
        "metric": "achieved KV-read HBM GB/s (% of peak) + µs/decode step, "
                  "Llama-3-8B GQA batch 32",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_dist": {"median": round(p50, 2), "p10": round(p10, 2),
                             "p90": round(p90, 2),
                             "how": "second pass of the same K steps, an event after each"},
        "gbs_at_median_step": round(float(bytes_steps.mean()) / (p50 * 1e-6) / 1e9, 1),
        "steps_per_s": round(1e3 / ms_per_step, 1),
        "pct_of_peak": round(gbs / HBM_PEAK_GBS * 100, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype if w.kv_dtype == w.q_dtype else f"{w.q_dtype}+{w.kv_dtype}",
        "data": "synthetic (seeded N(0,1) K/V/q, seeded lengths and block placement)",
        "config": {
            "workload": f"{w.name}: decode step of {L} layer(s), {B} seqs, {Hq} q / {Hkv} kv "
                        f"heads, head_dim {D}, block {bs}, lengths {int(lens0.min()) + 1}.."
                        f"{int(lens0.max()) + 1} at the first timed step",
            "workload_name": w.name,
            "global_batch": B,
            "kv_tokens_first_step": int(tokens[0]),
            "kv_bytes_per_step_avg": int(bytes_steps.mean()),
            "partition": partition,
            "block_size": bs,
            "kernel": kname,
            "cache_replicas": R,
            "metadata": "uploaded per step" if upload else "resident (all steps)",
            "share_plan": not no_hint,
            "step_calls": ("pa_cache_append + pa_decode" if separate else "pa_decode_append"),
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(roof_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
            "probe_gbs": None if probe is None else probe["gbs"],
            "frac_of_probe": None if probe is None else round(roof_gbs / probe["gbs"], 4),
            "probe": probe,
            "traffic": (measured_traffic(w.name, partition, int(roof_bytes), no_hint)
                        if bs == 16 else None),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1)",
            "algorithmic_bytes": int(roof_bytes),
            "logical_bytes": int(launch_bytes),
            "logical_achieved": round(kern_gbs, 1),
            "kernel": ("decode_valu_kernel" if "valu" in kname else
                       "decode_mfma_balanced_kernel" if partition == -1 else
                       "decode_mfma_kernel"),
            "kernel_us_avg": round(kern_us, 2),
            "unique": unique,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def measured_traffic(workload, partition, launch_bytes, no_hint):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs
    (profiles/decode_mfma_balanced_<workload>.traffic.json), if they were
    taken for this launch (same workload, launch mode, hint and algorithmic
    bytes per launch, which fixes every sequence length) and the kernel's
    sources have not changed since; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_mfma_balanced_{workload}.traffic.json")
    try:
        recs = json.load(open(path))
        recs = recs if isinstance(recs, list) else [recs]
        h = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, ValueError):
        return None
    for rec in recs:
        same = (rec.get("kernel_sources") == TRAFFIC_SOURCES and
                rec.get("workload") == workload and rec.get("partition") == partition and
                rec.get("algorithmic_bytes_per_launch") == launch_bytes and
                rec.get("share_plan", False) == (not no_hint) and
                rec.get("kernel_sources_sha256") == h.hexdigest())
        if same:
            return rec["hbm_bytes_per_launch"]
    return None


# The decode kernel's translation unit and what it includes, and the build's
# flags: a traffic record holds only while these are unchanged.
TRAFFIC_SOURCES = [
    "paged_kv_cache_255_amd/csrc/decode_mfma.hip",
    "paged_kv_cache_255_amd/csrc/work.hpp",
    "paged_kv_cache_255_amd/csrc/device.hpp",
    "paged_kv_cache_255_amd/build.py",
]


def _counter_values(path, counter, kernel_substr):
    import csv
    with open(path, newline="") as f:
        return [float(r["Counter_Value"]) for r in csv.DictReader(f)
                if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]]


def write_traffic_record(bench_line, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Turns two rocprofv3 counter runs of one bench command into HBM bytes per
    decode launch.  The counters read KiB per dispatch; each is scaled by
    what it reads for a plain device-to-device copy of known size (bench.py
    --copy-calibration: three copies of 2^30 bytes).  The last `steps`
    dispatches of the decode kernel are the back-to-back launches that the
    roofline times."""
    import hashlib
    line = None
    for ln in open(bench_line):
        if ln.startswith("{") and '"roofline"' in ln:
            line = json.loads(ln)
    if line is None:
        sys.exit(f"no bench JSON line in {bench_line}")
    roof, cfg = line["roofline"], line["config"]
    steps, warmup = line["steps"], line["warmup"]
    if roof["kernel"] != "decode_mfma_balanced_kernel" or cfg.get("block_size", 16) != 16:
        sys.exit("traffic records are kept for the balanced MFMA decode kernel at 16-token "
                 "blocks only")

    def mean_last(path, counter):
        v = _counter_values(path, counter, "decode_mfma_balanced_kernel")
        if len(v) < steps:
            sys.exit(f"{path}: {len(v)} decode dispatches with {counter}, need {steps}")
        return sum(v[-steps:]) / steps

    def copy_mean(path, counter):
        v = _counter_values(path, counter, "copyBuffer")
        if len(v) != 3:
            sys.exit(f"{path}: expected 3 copy dispatches with {counter}, found {len(v)}")
        return sum(v) / 3

    gib_kib = (1 << 30) / 1024
    cf, cw = copy_mean(copy_fetch_csv, "FETCH_SIZE"), copy_mean(copy_write_csv, "WRITE_SIZE")
    fetch_scale, write_scale = round(gib_kib / cf, 2), round(gib_kib / cw, 2)
    fk, wk = mean_last(fetch_csv, "FETCH_SIZE"), mean_last(write_csv, "WRITE_SIZE")
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    rec = {
        "kernel": roof["kernel"],
        "workload": cfg["workload_name"],
        "partition": cfg["partition"],
        "share_plan": cfg.get("share_plan", False),
        "steps": steps,
        "warmup": warmup,
        "launches": f"the last {steps} of the back-to-back decode launches bench.py times "
                    "(last step's metadata)",
        "kernel_sources": TRAFFIC_SOURCES,
        "kernel_sources_sha256": h.hexdigest(),
        "fetch_size_kib_per_launch_raw": round(fk, 2),
        "fetch_scale": fetch_scale,
        "write_size_kib_per_launch_raw": round(wk, 2),
        "write_scale": write_scale,
        "copy_calibration": {"bytes_read_and_written": 1 << 30,
                             "fetch_size_kib": round(cf, 1), "write_size_kib": round(cw, 1)},
        "hbm_bytes_per_launch": int(round(fk * 1024 * fetch_scale + wk * 1024 * write_scale)),
        "algorithmic_bytes_per_launch": roof["algorithmic_bytes"],
    }
    # one record per launch (steps and warmup fix the last step's lengths): a
    # record for the same launch is replaced, others are kept
    path = os.path.join(ROOT, "profiles",
                        f"decode_mfma_balanced_{cfg['workload_name']}.traffic.json")
    try:
        old = json.load(open(path))
        old = old if isinstance(old, list) else [old]
    except (OSError, ValueError):
        old = []
    keep = [r for r in old if not (r.get("steps") == steps and r.get("warmup") == warmup and
                                   r.get("partition") == rec["partition"] and
                                   r.get("share_plan") == rec["share_plan"])]
    with open(path, "w") as f:
        json.dump(keep + [rec], f, indent=1)
        f.write("\n")
    print(f"{path}: {rec['hbm_bytes_per_launch']} HBM bytes per launch, "
          f"{rec['hbm_bytes_per_launch'] / rec['algorithmic_bytes_per_launch']:.4f}x algorithmic")


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _time_launches(torch, fn, reps):
    """Mean ms of fn() over reps back-to-back calls between two events."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _feature_line(name, value, unit, extra):
    line = {"metric": name, "value": value, "unit": unit, "n_gpus": 1,
            "higher_is_better": unit != "us", "data": "synthetic"}
    line.update(extra)
    print(json.dumps(line), flush=True)


def feature_copy(args, torch, pa, workloads, execute_plan):
    """Copy-on-write block copies: 4,096 (source, destination) pairs of config-2
    blocks in one pa_copy_blocks launch.  Bytes = K and V of each block read
    once and written once."""
    w = workloads.config(2)
    NB, npairs = 16384, 4096
    desc = pa.kv_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, NB, w.q_dtype, w.kv_dtype)
    elems = NB * w.num_kv_heads * 16 * w.head_dim
    kc = torch.randn(elems, device="cuda").to(torch.bfloat16)
    vc = torch.randn(elems, device="cuda").to(torch.bfloat16)
    perm = np.random.default_rng(7).permutation(NB)
    pairs = torch.from_numpy(np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1)
                             .astype(np.int32)).cuda()
    ms = _time_launches(torch, lambda: pa.pa_copy_blocks(kc, vc, pairs, desc), args.steps)
    block = 16 * w.num_kv_heads * w.head_dim * 2
    moved = 2 * 2 * npairs * block  # K and V, read and written
    _feature_line("copy-on-write block copies: HBM GB/s (read + write)",
                  round(moved / (ms * 1e-3) / 1e9, 1), "GB/s",
                  {"us_per_launch": round(ms * 1e3, 2), "pairs": npairs,
                   "block_bytes_k_and_v": 2 * block, "peak": HBM_PEAK_GBS,
                   "frac": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "config": {"workload": "config-2 blocks (8 KV heads x 16 x 128 bf16)"}})


def feature_swap(args, torch, pa, workloads, execute_plan):
    """Swapping config 2's 32 sequences out to pinned host memory and back in,
    each direction as one pa_swap_blocks launch over every block of every
    table (pairs from pa_seq_swap_out / pa_seq_swap_in)."""
    w = workloads.config(2)
    Hkv, D = w.num_kv_heads, w.head_dim
    NB = w.num_blocks
    pool = pa.pa_block_pool_init(NB, Hkv, D, w.kv_dtype, shuffle_seed=w.shuffle_seeds[0],
                                 num_host_blocks=NB)
    ids, pre = execute_plan(pool, w.ops)
    dec = [ids[s] for s in w.decode_seqs]
    desc = pa.kv_desc(w.num_q_heads, Hkv, D, NB, w.q_dtype, w.kv_dtype)
    block = pa.pa_block_bytes(pool)
    kc = torch.zeros(NB * block, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    hk = torch.zeros(NB * block, dtype=torch.uint8, pin_memory=True)
    hv = torch.zeros(NB * block, dtype=torch.uint8, pin_memory=True)
    outs, ins = [], []
    for cycle in range(args.warmup + args.steps):
        p_out = np.concatenate([pa.pa_seq_swap_out(pool, s) for s in dec])
        d_out = torch.from_numpy(p_out).cuda()
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        pa.pa_swap_blocks(kc, vc, hk, hv, d_out, desc, to_host=True)
        e1.record()
        p_in = np.concatenate([pa.pa_seq_swap_in(pool, s) for s in dec])
        d_in = torch.from_numpy(p_in).cuda()
        torch.cuda.synchronize()
        e2, e3 = _events(torch)
        e2.record()
        pa.pa_swap_blocks(kc, vc, hk, hv, d_in, desc, to_host=False)
        e3.record()
        torch.cuda.synchronize()
        if cycle >= args.warmup:
            outs.append(e0.elapsed_time(e1))
            ins.append(e2.elapsed_time(e3))
    nbytes = 2 * len(p_out) * block  # K and V
    out_ms, in_ms = float(np.median(outs)), float(np.median(ins))
    _feature_line("swap to pinned host memory and back: GB/s per direction",
                  round(nbytes / (out_ms * 1e-3) / 1e9, 2), "GB/s",
                  {"to_host_gbs": round(nbytes / (out_ms * 1e-3) / 1e9, 2),
                   "to_device_gbs": round(nbytes / (in_ms * 1e-3) / 1e9, 2),
                   "to_host_ms": round(out_ms, 3), "to_device_ms": round(in_ms, 3),
                   "blocks": int(len(p_out)), "bytes_per_direction": int(nbytes),
                   "cycles": args.steps,
                   "config": {"workload": "config 2: 32 sequences, every block of every table"}})


def feature_window(args, torch, pa, workloads, execute_plan):
    """Windowed decode at config 2: every sequence keeps its last 1,024 tokens
    (pa_seq_slide_window releases the blocks before them).  The decode kernel
    alone, back to back over 4 cache replicas; bytes = the window tokens' K
    and V."""
    w = workloads.config(2)
    Hq, Hkv, D, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_seqs
    win = 1024
    NB = w.num_blocks
    pool = pa.pa_block_pool_init(NB, Hkv, D, w.kv_dtype, shuffle_seed=w.shuffle_seeds[0])
    ids, pre = execute_plan(pool, w.ops)
    dec = [ids[s] for s in w.decode_seqs]
    slots = pa.pa_seq_append_slots_batch(pool, dec, 1)
    released = sum(pa.pa_seq_slide_window(pool, s, win) for s in dec)
    maxb = -(-max(w.decode_lengths()) // 16)
    tables, lens, starts = pa.pa_export_block_tables(pool, dec, maxb, with_starts=True)
    desc = pa.kv_desc(Hq, Hkv, D, NB, w.q_dtype, w.kv_dtype)
    k_pre, v_pre = workloads.prefill_tensors(w, 0, "cuda")
    q, k_new, v_new = workloads.step_tensors(w, 0, "cuda")
    R = 4
    caches = []
    for _ in range(R):
        kc = torch.zeros(NB * Hkv * 16 * D, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        pa.pa_cache_append(k_pre, v_pre, kc, vc, torch.from_numpy(pre).cuda(), desc)
        pa.pa_cache_append(k_new, v_new, kc, vc, torch.from_numpy(slots).cuda(), desc)
        caches.append((kc, vc))
    out = torch.empty_like(q)
    dt, dl, ds = (torch.from_numpy(a).cuda() for a in (tables, lens, starts))
    ws = torch.empty(pa.pa_decode_workspace_bytes(desc, B, maxb * 16, pa.PARTITION_BALANCED),
                     dtype=torch.uint8, device="cuda")
    it = [0]

    def launch():
        kc, vc = caches[it[0] % R]
        it[0] += 1
        pa.pa_decode_partials(q, kc, vc, dt, dl, maxb * 16, w.scale, out, desc, ws,
                              pa.PARTITION_BALANCED, seq_starts=ds)

    ms = _time_launches(torch, launch, args.steps)
    tokens = int((lens - starts).sum())
    nbytes = tokens * Hkv * D * 2 * 2
    _feature_line("windowed decode: KV-read HBM GB/s (window tokens)",
                  round(nbytes / (ms * 1e-3) / 1e9, 1), "GB/s",
                  {"kernel_us_avg": round(ms * 1e3, 2), "window": win,
                   "window_tokens": tokens, "blocks_released": int(released),
                   "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "config": {"workload": "config 2, every sequence slid to its last 1024 "
                                          "tokens, balanced split, 4 cache replicas"}})


def feature_prefix(args, torch, pa, workloads, execute_plan):
    """Prefix-cache host work at config 4's shape: 256 requests whose prompts
    start with one 2,048-token system prompt.  Times match + prefill slots +
    register per request (the host side of admitting a request), and counts
    the blocks the cache saves against private copies."""
    import time
    w = workloads.config(4)
    rng = np.random.default_rng(4)
    P = 2048
    system = [int(x) for x in rng.integers(0, 32000, size=P)]
    suffixes = [int(n) for n in np.minimum(rng.geometric(1 / 350, size=256), 2048)]
    prompts = [np.array(system + [int(x) for x in rng.integers(0, 32000, size=n)], np.int32)
               for n in suffixes]
    need = sum(-(-len(p) // 16) for p in prompts)
    pool = pa.pa_block_pool_init(need + 64, w.num_kv_heads, w.head_dim, w.kv_dtype,
                                 shuffle_seed=1)
    t0 = time.perf_counter()
    matched = 0
    for pr in prompts:
        s = pa.pa_seq_create(pool)
        m = pa.pa_prefix_match(pool, s, pr)
        matched += m
        pa.pa_seq_append_slots(pool, s, len(pr) - m)
        pa.pa_prefix_register(pool, s, pr)
    dt = time.perf_counter() - t0
    st = pa.pa_pool_get_stats(pool)
    _feature_line("prefix caching: host time per admitted request", round(dt / 256 * 1e6, 2),
                  "us", {"requests": 256, "tokens_matched": matched,
                         "blocks_used": st["used_blocks"], "blocks_without_cache": need,
                         "blocks_saved_frac": round(1 - st["used_blocks"] / need, 4),
                         "config": {"workload": "config-4 shape: 256 prompts = 2048-token "
                                                "system prompt + Geometric(1/350) suffix"}})


def feature_prefill(args, torch, pa, workloads, execute_plan):
    """The prefill append of one layer of --config (3: 8 x 4,095 tokens, 40 KV
    heads, fp16; 5: 4 x 131,071 tokens, 8 KV heads, bf16 into FP8): one
    pa_cache_append of every prefill token, timed over back-to-back launches.
    Bytes = the K and V rows read (activation dtype) plus those written (cache
    dtype)."""
    w = workloads.config(args.config)
    pool = pa.pa_block_pool_init(w.num_blocks, w.num_kv_heads, w.head_dim, w.kv_dtype,
                                 block_size=w.block_size, shuffle_seed=w.shuffle_seeds[0])
    _, pre = execute_plan(pool, w.ops)
    T = len(pre)
    desc = pa.kv_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_blocks, w.q_dtype,
                      w.kv_dtype, block_size=w.block_size)
    k_pre, v_pre = workloads.prefill_tensors(w, 0, "cuda")
    ks = vs = 1.0
    if w.kv_dtype == "e4m3":
        ks, vs = workloads.fp8_scale(k_pre), workloads.fp8_scale(v_pre)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.uint8}[w.kv_dtype]
    nelem = w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim
    kc = torch.zeros(nelem, dtype=tdt, device="cuda")
    vc = torch.zeros(nelem, dtype=tdt, device="cuda")
    slots = torch.from_numpy(pre).cuda()
    ms = _time_launches(torch, lambda: pa.pa_cache_append(k_pre, v_pre, kc, vc, slots, desc,
                                                          ks, vs), args.steps)
    qb = {"f32": 4, "f16": 2, "bf16": 2}[w.q_dtype]
    kb = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    row = w.num_kv_heads * w.head_dim
    moved = 2 * T * row * (qb + kb)
    gbs = moved / (ms * 1e-3) / 1e9
    log(f"[bench] prefill append {w.name}: {T} tokens, {ms * 1e3:.1f} us per launch, "
        f"{gbs:.1f} GB/s = {gbs / HBM_PEAK_GBS * 100:.1f}% of HBM peak")
    _feature_line("prefill cache append: HBM GB/s (K and V read + written)",
                  round(gbs, 1), "GB/s",
                  {"us_per_launch": round(ms * 1e3, 2), "tokens": T, "bytes_per_launch": moved,
                   "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
                   "kernel": "append_tiles_kernel",
                   "config": {"workload": f"{w.name}: prefill of one layer, {T} tokens, "
                                          f"{w.num_kv_heads} KV heads x {w.head_dim}, "
                                          f"{w.q_dtype} into {w.kv_dtype}"}})


FEATURES = {"copy": feature_copy, "swap": feature_swap, "window": feature_window,
            "prefix": feature_prefix, "prefill": feature_prefill}


def copy_calibration(torch):
    """Three copies of 1 GiB between two device buffers: each reads and writes
    exactly 2^30 bytes, the reference for HBM byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 3
    # also the rate of a plain device copy (read + write), the ceiling a
    # copy-shaped kernel such as the prefill append can be measured against
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3, "us_per_copy": round(us, 1),
                      "gbs_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)}), flush=True)


def cpu_baseline(w, k_cache, v_cache, q, tables, lens, nblocks, ks, vs, target_s):
    """The CPU oracle (fp64 C) on the last timed step's sequences, sized to
    about `target_s` seconds, with one thread per core this process may run
    on (os.sched_getaffinity), then with one thread on about a third of that
    time."""
    import oracle
    import workloads
    kh = workloads.storage(k_cache)
    vh = workloads.storage(v_cache)
    qh = workloads.storage(q)
    eb = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    args = dict(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                block_size=w.block_size, num_blocks=nblocks, q_dtype=w.q_dtype,
                kv_dtype=w.kv_dtype, scale=w.scale, k_scale=ks, v_scale=vs)

    def run(nseq, threads):
        rows = [(b, h) for b in range(nseq) for h in range(w.num_q_heads)]
        t0 = time.perf_counter()
        oracle.decode(qh, kh, vh, tables, lens, rows=rows, nthreads=threads, **args)
        return time.perf_counter() - t0

    def timed(threads, budget):
        # as many sequences as fit in the budget; if the whole batch is faster
        # than that, the whole batch repeated until about the budget has passed
        t1 = run(1, threads)
        nseq = int(max(1, min(len(lens), budget / max(t1, 1e-6))))
        t = run(nseq, threads)
        reps = 1
        while t < 0.8 * budget:
            t += run(nseq, threads)
            reps += 1
        nbytes = reps * int(lens[:nseq].sum()) * w.num_kv_heads * w.head_dim * 2 * eb
        return nbytes / t / 1e9, nseq, reps, t

    cores = len(os.sched_getaffinity(0))
    gbs, nseq, reps, t = timed(cores, target_s)
    gbs1, nseq1, reps1, t_1 = timed(1, target_s / 3)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores,
            "value_1_thread": round(gbs1, 4), "kind": "oracle", "cpu_model": model,
            "sample": f"{nseq} of {len(lens)} sequences ({int(lens[:nseq].sum())} tokens, all "
                      f"{w.num_q_heads} q heads) of the last timed step, {reps} pass(es), fp64 C "
                      f"oracle, {cores} threads, {t:.1f} s; one thread: {nseq1} sequences, "
                      f"{reps1} pass(es), {t_1:.1f} s"}


def read_probe(torch, pa, dev, reps, loads=8, wgs=None, nontemporal=True, one_per_cu=True,
               nbytes=4 << 30):
    """GB/s of pa_read_probe over a buffer of nbytes: `reps` launches back to
    back between two events.  Defaults: the setting that reads fastest on
    MI355X (8 loads in flight per lane, one workgroup per CU, nontemporal)."""
    if wgs is None:
        wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    buf = torch.ones(nbytes // 2, dtype=torch.int16, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    ms = _time_launches(torch, lambda: pa.pa_read_probe(buf, loads, wgs, sink, nontemporal,
                                                         one_per_cu), reps)
    del buf
    return {"gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "loads_in_flight": loads,
            "workgroups": wgs, "nontemporal": nontemporal, "one_wg_per_cu": one_per_cu,
            "bytes": nbytes, "us": round(ms * 1e3, 1)}


def read_ceiling_sweep(torch, pa, args):
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = None
    for nt in (True, False):
        for loads in (4, 8, 16):
            for mult, one in ((1, True), (2, False), (4, False), (16, False)):
                r = read_probe(torch, pa, dev, reps=20, loads=loads, wgs=cus * mult,
                               nontemporal=nt, one_per_cu=one)
                r["frac_of_peak"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
                print(json.dumps({"read_probe": r}), flush=True)
                if best is None or r["gbs"] > best["gbs"]:
                    best = r
    print(json.dumps({"read_ceiling_best": best}), flush=True)


if __name__ == "__main__":
    main()
