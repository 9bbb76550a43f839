"""Benchmark of one MSA decode layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one decode layer over one batch of the chosen synthetic
configuration, inputs resident in HBM: one call of msa_decode_layer_single
(one kernel: indexer + per-block max pool, then top-16 selection + sparse
attention per item) where that path applies and runs the same arithmetic as
the two-kernel path (--layer auto), else of msa_decode_layer (kernel 1:
indexer + pool; kernel 2: selection + attention). Consecutive steps rotate
over R device replicas of the inputs so that no step finds its bytes in the
256 MB Infinity Cache. The K timed steps lie between two HIP events on the
launch stream. A second pass over the same K steps has every kernel's
dispatch record its own start and end events (hipExtLaunchKernel), which
give the per-kernel durations.
Prints one JSON line on stdout (details on stderr):

  value        decode tokens/s per layer = B * T_q / step time
  roofline     the dominant kernel (the single-launch layer kernel, or the
               indexer scan of the two-kernel path): algorithmic bytes per
               launch / its average duration, against the 8 TB/s HBM peak;
               traffic = HBM bytes per launch from rocprofv3 counters, when a
               record for the current kernel source exists (else null)
  cpu_baseline the float64 oracle on a bounded sample of the same workload,
               timed on this host's cores
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
METRIC = "MSA decode tokens/s per layer at 128K ctx; achieved HBM GB/s vs 8 TB/s peak"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_sparse_attention_kv_amd", "csrc")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")
# --layer auto: indexer bytes per step up to which the single launch is
# taken whatever the number of attention items
SINGLE_SCAN_BYTES = 64e6
# the files each kernel's device code is compiled from (a traffic record is
# valid only for the sources it was taken on)
KERNELS = {
    "indexer_pool": dict(symbol="indexer_pool_kernel",
                         sources=("indexer.hip", "indexer_impl.hpp", "fmt.hpp", "indexer_args.hpp")),
    "decode_layer_single": dict(symbol="decode_layer_single_kernel",
                                sources=("layer.hip", "indexer_impl.hpp", "attn_impl.hpp", "topk.hpp", "fmt.hpp",
                                         "indexer_args.hpp", "msa_internal.hpp")),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ byte models

def indexer_bytes(w):
    """Algorithmic bytes of the indexer + pool launch: every visible indexer
    key (64 B codes + 4 B scale for FP8, 32 B codes + 4 B scales for NVFP4,
    128 B for bf16), indexer queries and
    weights, block-table entries read, pooled scores written."""
    prm = w.params
    B, Tq, Hi, maxb = prm["num_seqs"], prm["q_len"], prm["idx_heads"], prm["max_blocks_per_seq"]
    L = np.minimum(w.ctx_lens.astype(np.int64), maxb * 128)
    nblk = (L + 127) // 128
    per_tok = {0: 128, 1: 68, 2: 36}[int(prm["idx_dtype"])]  # bf16, FP8 (+fp32 scale), NVFP4 (+4 E4M3)
    return int(L.sum() * per_tok + B * Tq * Hi * (64 * 2 + 4) + nblk.sum() * 4 + Tq * nblk.sum() * 4)


def attention_bytes(w, sel):
    """Algorithmic bytes of the selection + attention launch: K+V of the
    union of the selected blocks per (sequence, KV head) -- 144 B per token
    per KV head for NVFP4 (codes + scales of K and V), 512 B for bf16 -- plus
    queries, pooled scores read, selections and bf16 outputs."""
    prm = w.params
    B, Tq, Hq, G = prm["num_seqs"], prm["q_len"], prm["num_q_heads"], prm["num_kv_heads"]
    per_tok = 144 if prm["kv_dtype"] == 1 else 512
    blocks = 0
    for b in range(B):
        blocks += len(set(int(x) for x in sel[b].ravel() if x >= 0))
    L = np.minimum(w.ctx_lens.astype(np.int64), prm["max_blocks_per_seq"] * 128)
    pooled = int(((L + 127) // 128).sum()) * Tq * 4
    return int(blocks * G * 128 * per_tok + B * Tq * Hq * 128 * 2 * 2 + B * Tq * prm["top_k"] * 4 + pooled)


def _records():
    try:
        recs = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return []
    return recs if isinstance(recs, list) else []


def traffic_record(kernel, config_id):
    """HBM bytes per launch of `kernel` from the committed counter records, if
    one was taken on the kernel's current sources and this workload."""
    sha = source_sha(KERNELS[kernel]["sources"])
    for rec in _records():
        if rec.get("kernel") == kernel and rec.get("source_sha") == sha and rec.get("config_id") == config_id:
            return rec
    return None


def write_traffic_record(fetch_csv, write_csv, kernel, config_id):
    """HBM bytes per launch of `kernel` from two rocprofv3 --pmc collections of
    a --profile-steps run (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).
    Each counter is scaled by what it reads for the run's 1 GiB device copy
    (1 GiB read, 1 GiB written), so the record is in bytes actually moved.
    Replaces the record of the same kernel and workload."""
    import csv
    symbol = KERNELS[kernel]["symbol"]

    def per_kernel(path, counter):
        vals, copy = [], None
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            if symbol in r["Kernel_Name"]:
                vals.append(v)
            elif "copyBuffer" in r["Kernel_Name"] and (copy is None or v > copy):
                copy = v          # the largest copy: the 1 GiB calibration copy
        return vals, copy

    f, fc = per_kernel(fetch_csv, "FETCH_SIZE")
    w, wc = per_kernel(write_csv, "WRITE_SIZE")
    if not f or not w:
        raise SystemExit("no %s dispatches in the counter files" % symbol)
    gib = float(1 << 30)
    f_scale, w_scale = gib / fc, gib / wc
    fetch = float(np.mean(f)) * f_scale
    write = float(np.mean(w)) * w_scale
    rec = {"kernel": kernel, "config_id": config_id, "source_sha": source_sha(KERNELS[kernel]["sources"]),
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write, "fetch_scale": f_scale, "write_scale": w_scale,
           "launches": [len(f), len(w)]}
    recs = [r for r in _records() if not (r.get("kernel") == kernel and r.get("config_id") == config_id)]
    recs.append(rec)
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(recs, fh, indent=1)
    print(json.dumps(rec))


# ------------------------------------------------------------ cpu baseline

def cpu_baseline(w, gpu_res, budget_s=20.0):
    """Time the oracle (as it stands) on whole sequences of the workload until
    about budget_s seconds of CPU work; also compare its results with the GPU
    step's on those sequences."""
    from oracle import msa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    prm = w.params
    t0 = time.perf_counter()
    done_tok, seqs, other_sel, max_err = 0, [], 0, 0.0
    for b in range(prm["num_seqs"]):
        res = O.decode_sequence(w, b)
        done_tok += len(res)
        seqs.append(b)
        for t, r in enumerate(res):
            if r["p"] < 0:
                continue
            g = sorted(int(x) for x in gpu_res["sel"][b, t] if x >= 0)
            if g != list(r["sel"]):
                other_sel += 1
            else:
                err = np.abs(gpu_res["out"][b, t] - r["out"])
                small = np.abs(r["out"]) < 0.5
                if small.any():
                    max_err = max(max_err, float(err[small].max()))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_tok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d of %d sequences (%d query tokens), float64 numpy, %.1f s" % (
                len(seqs), prm["num_seqs"], done_tok, dt),
            "sample_check": {"tokens_with_other_selection": other_sel, "max_abs_where_o_below_0.5": max_err}}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--idx-dtype", choices=("fp8", "nvfp4"), default="fp8",
                    help="indexer-key format (the measured configurations use fp8)")
    ap.add_argument("--replicas", type=int, default=0, help="input copies rotated per step (0: auto)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many steps and a 1 GiB calibration copy (for rocprofv3 runs)")
    ap.add_argument("--layer", choices=("auto", "single", "two"), default="auto",
                    help="single: msa_decode_layer_single; two: msa_decode_layer; auto: single where it applies "
                         "and has at least two (sequence, token, KV head) items per compute unit or a short "
                         "indexer scan (<= 64 MB)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write a record of profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "counter collections of a --profile-steps run, and exit")
    ap.add_argument("--traffic-kernel", choices=sorted(KERNELS), default="decode_layer_single",
                    help="the kernel whose counters --traffic-from records")
    args = ap.parse_args()
    wkey = str(args.config) if args.idx_dtype == "fp8" else "%d/%s" % (args.config, args.idx_dtype)
    if args.traffic_from:
        write_traffic_record(args.traffic_from[0], args.traffic_from[1], args.traffic_kernel, wkey)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (one GPU's share of the decode "
              "batch is the unit of work). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, ROOT)
    import block_sparse_attention_kv_amd as msa
    from workloads import make_config, CONFIG_NAMES, IDX_NVFP4

    t0 = time.perf_counter()
    w = make_config(args.config, idx_dtype=IDX_NVFP4 if args.idx_dtype == "nvfp4" else None)
    log("generated %s in %.1f s (%.2f GB host)" % (w.name, time.perf_counter() - t0, w.nbytes() / 1e9))
    prm = w.params
    B, Tq, Hq = prm["num_seqs"], prm["q_len"], prm["num_q_heads"]
    step_guess = indexer_bytes(w) + B * prm["num_kv_heads"] * 64 * 128 * 144
    R = args.replicas or max(2, min(4, int(math.ceil(3 * 256e6 / max(step_guess, 1)))))
    dev = "cuda"
    reps = [msa.to_device(w, dev) for _ in range(R)]
    torch.cuda.synchronize()
    log("uploaded %d replica(s) in %.1f s" % (R, time.perf_counter() - t0))
    out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device=dev)
    lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Tq, prm["top_k"]), dtype=torch.int32, device=dev)
    ws = msa.alloc_workspace(reps[0][0], dev)

    # Every C argument is built once, so that a timed step is one C-ABI call:
    # the host then stays ahead of the GPU and the queue never drains.
    import ctypes
    L = msa.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws_bytes = ws.numel() * ws.element_size()
    keep = []

    def vp(t):
        return ctypes.c_void_p(t.data_ptr())

    call_args = []
    for params, cache, qs in reps:
        c = cache.c()
        keep.append(c)
        call_args.append([ctypes.byref(params), ctypes.byref(c), vp(qs["q"]), vp(qs["idx_q"]), vp(qs["idx_w"]),
                          vp(out), vp(lse), vp(sel), vp(ws), ctypes.c_size_t(ws_bytes), stream])

    items = B * Tq * prm["num_kv_heads"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    single_ok = prm["kv_dtype"] == 1 and prm["idx_dtype"] in (1, 2) and Tq <= 4
    if args.layer == "auto":
        # the single launch wins from two items per CU up, and wherever the
        # scan is short enough that the gap between two kernels weighs more
        # than 4 instead of 8 waves per item (measured: 32K x 8 sequences)
        single = single_ok and (items >= 2 * cus or indexer_bytes(w) <= SINGLE_SCAN_BYTES)
    else:
        single = args.layer == "single"
        if single and not single_ok:
            raise SystemExit("--layer single: this configuration needs the two-kernel path")
    kernel = "decode_layer_single" if single else "indexer_pool"
    plain = L.msa_decode_layer_single if single else L.msa_decode_layer
    traced = L.msa_decode_layer_single_traced if single else L.msa_decode_layer_traced
    entry = "msa_decode_layer_single" if single else "msa_decode_layer"
    log("layer path: %s (%d items, %d compute units)" % (entry, items, cus))

    def step(i, events=None):
        if events is None:
            st = plain(*call_args[i % R])
        else:
            st = traced(*call_args[i % R], events)
        if st != 0:
            raise RuntimeError("%s: %s" % (entry, L.msa_last_error().decode()))

    if args.profile_steps:
        for i in range(args.profile_steps):
            step(i)
        torch.cuda.synchronize()
        log("profile run: %d steps done" % args.profile_steps)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    gpu_res = {"sel": sel.cpu().numpy(),
               "out": (out.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.uint32) << 16)
               .view(np.float32).astype(np.float64)}

    # ---- timed region: K steps between two HIP events on the launch stream
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    log("timed %d steps: %.4f ms/step (events), %.4f ms/step (wall)" % (args.steps, ms_step,
                                                                       wall * 1e3 / args.steps))

    # ---- per-kernel durations: the same K steps again, each kernel's dispatch
    # recording its own start and end event (hipExtLaunchKernel); the events
    # lengthen the step a little, so the step time above comes from the
    # uninstrumented pass
    n_st = 1 if single else msa.NUM_STAGES
    stage_names = ["decode_layer_single"] if single else list(msa.STAGE_NAMES)
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_st)] for _ in range(args.steps)]
    for row in kev:          # create the HIP events before the timed pass
        for e in row:
            e.record()
    torch.cuda.synchronize()
    ev_arrays = [(ctypes.c_void_p * (2 * n_st))(*[e.cuda_event for e in row]) for row in kev]
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for i in range(args.steps):
        step(i, ev_arrays[i])
    k1.record()
    torch.cuda.synchronize()
    ms_step_traced = k0.elapsed_time(k1) / args.steps
    stage_all = [np.array([kev[i][2 * s].elapsed_time(kev[i][2 * s + 1]) for i in range(args.steps)])
                 for s in range(n_st)]
    stage_ms = [float(np.mean(d)) for d in stage_all]
    # spread of the per-step kernel durations (ms): p10, median, p90
    stage_pct = {n: [float(x) for x in np.percentile(d, [10, 50, 90])] for n, d in zip(stage_names, stage_all)}
    log("kernels (ms): " + ", ".join("%s %.4f" % (n, v) for n, v in zip(stage_names, stage_ms)) +
        "; step with kernel events %.4f ms" % ms_step_traced)
    log("kernel durations p10 / median / p90 (ms): " +
        ", ".join("%s %.4f / %.4f / %.4f" % (n, *stage_pct[n]) for n in stage_names))

    # ---- attainable copy bandwidth on this machine (context)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    # ---- attainable read bandwidth: the library's streaming read kernel
    chk = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        msa.msa_debug_read_bandwidth(src, chk)
    c0.record()
    for _ in range(10):
        msa.msa_debug_read_bandwidth(src, chk)
    c1.record()
    torch.cuda.synchronize()
    read_gbps = (1 << 30) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    log("attainable on this box: read %.0f GB/s (1 GiB stream), device copy %.0f GB/s (read + write)"
        % (read_gbps, copy_gbps))
    del src, dst

    idx_b = indexer_bytes(w)
    att_b = attention_bytes(w, gpu_res["sel"])
    step_b = idx_b + att_b
    step_gbps = step_b / (ms_step * 1e-3) / 1e9
    if single:   # one kernel moves the step's bytes
        kern_b, kern_ms = step_b, stage_ms[0]
        stage_detail = {}
    else:        # the indexer kernel dominates
        kern_b, kern_ms = idx_b, stage_ms[0]
        stage_detail = {"attention_gbps": att_b / (stage_ms[1] * 1e-3) / 1e9}
    kern_gbps = kern_b / (kern_ms * 1e-3) / 1e9
    rec = traffic_record(kernel, wkey)
    tokens = B * Tq
    res = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/bf16 mfma, f32 accumulate (nvfp4 K/V, %s idx keys in)" % args.idx_dtype,
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[args.config] + ("" if args.idx_dtype == "fp8" else
                                                             ", NVFP4 idx keys instead of FP8"),
                   "config_id": wkey, "batch": B, "q_len": Tq,
                   "ctx_len": int(w.ctx_lens.max()), "q_heads": Hq, "kv_heads": prm["num_kv_heads"],
                   "idx_heads": prm["idx_heads"], "top_k": prm["top_k"], "block": 128,
                   "input_replicas": R},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": kern_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": kern_gbps / HBM_PEAK_GBPS,
                     "traffic": None if rec is None else rec["traffic_bytes_per_launch"],
                     "algorithmic_bytes": kern_b, "avg_ms": kern_ms},
        "step": dict({"entry": entry, "algorithmic_bytes": step_b, "gbps": step_gbps,
                      "frac": step_gbps / HBM_PEAK_GBPS, "stage_ms": dict(zip(stage_names, stage_ms)),
                      "stage_ms_p10_p50_p90": stage_pct,
                      "ms_per_step_with_kernel_events": ms_step_traced, "indexer_bytes": idx_b,
                      "attention_bytes": att_b, "copy_gbps_attainable": copy_gbps,
                      "read_gbps_attainable": read_gbps}, **stage_detail),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, gpu_res, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
