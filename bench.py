"""Benchmark of one MSA decode layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one decode layer over one batch of the chosen synthetic
configuration, inputs resident in HBM: one call of msa_decode_layer_single
(one kernel: indexer + per-block max pool, then top-16 selection + sparse
attention) where that path applies (--layer auto: NVFP4 K/V, FP8 or NVFP4
indexer keys, q_len <= 4), else of msa_decode_layer (kernel 1: indexer +
pool; kernel 2: selection + attention). Consecutive
steps rotate over R device replicas of the inputs so that no step finds its
bytes in the 256 MB Infinity Cache. Order: the device's attainable read and
copy bandwidth (about 10 ms of streaming), W untimed steps, max(K, 500)
steps whose kernels' dispatches record their own start and end events
(hipExtLaunchKernel: the per-kernel durations), then the timed region: K
steps between two HIP events on the launch stream, with a device
synchronisation on both sides. The step time reaches its steady state only
after some 50 ms of sustained load (passes in the first ~50 ms ran up to 20%
slower), so the measurements before the timed region also bring the GPU to
that state.
Prints one JSON line on stdout (details on stderr):

  value        decode tokens/s per layer = B * T_q / step time
  roofline     the dominant kernel: the single-launch layer kernel (its time
               per launch is the timed region's time per step) or the
               indexer scan of the two-kernel path (from the traced pass):
               algorithmic bytes per launch / its average duration, against
               the 8 TB/s HBM peak; traffic = HBM bytes per launch from
               rocprofv3 counters, when a record for the current kernel
               source exists (else null)
  step         the step's algorithmic bytes term by term, rate and fraction
  cpu_baseline the float64 oracle on a bounded sample of the same workload,
               timed on this host's cores, and its comparison with the GPU
  other_workloads  (default run) the 32K, 512K and ragged decode workloads
               and the 128K one with NVFP4 indexer keys: step time, rate,
               fraction, and every query token's selection checked against
               the oracle
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
# steps of the event-traced pass at least (before the timed region): on the
# MI355X the step time reaches its steady state only after some 50 ms of
# sustained load (20-step passes in the first ~50 ms ran 77-92 us, later ones
# 75.5-77.8 us on the 128K workload)
TRACED_MIN_STEPS = 500
METRIC = "MSA decode tokens/s per layer at 128K ctx; achieved HBM GB/s vs 8 TB/s peak"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_sparse_attention_kv_amd", "csrc")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")
# the files each kernel's device code is compiled from (a traffic record is
# valid only for the sources it was taken on)
KERNELS = {
    "indexer_pool": dict(symbol="indexer_pool_kernel",
                         sources=("indexer.hip", "indexer_impl.hpp", "fmt.hpp", "indexer_args.hpp")),
    "decode_layer_single": dict(symbol="decode_layer_single_kernel",
                                sources=("layer.hip", "indexer_impl.hpp", "attn_impl.hpp", "topk.hpp", "fmt.hpp",
                                         "indexer_args.hpp", "msa_internal.hpp", "msa_api.hip")),
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
#
# Algorithmic bytes of one decode step: what the path has to read and write
# at least once, nothing it re-reads, over-fetches or keeps as intermediates
# (pooled scores, selections, partial softmax states are not counted).

IDX_KEY_BYTES = {0: 128, 1: 68, 2: 36}   # per token: bf16 row; FP8 row + fp32 scale; NVFP4 codes + 4 E4M3
KV_BYTES = {0: 512, 1: 144}              # per token and KV head, K + V: bf16; NVFP4 codes + E4M3 scales


def step_byte_terms(params, ctx_lens, union_blocks):
    """Algorithmic bytes of one step, term by term. ctx_lens: int array [B];
    union_blocks: the number of distinct blocks selected per sequence (the
    union over its query tokens), summed over the batch. Terms:
      idx_keys    every visible indexer key (codes + scales)
      kv          K and V of the union of the selected blocks per sequence,
                  for every KV head (codes + scales)
      q, out      bf16 attention queries and outputs
      idx_q, idx_w  bf16 indexer queries, fp32 head weights
      table       the block-table entries of every visible block
      ctx_lens    one int32 per sequence"""
    B, Tq = int(params["num_seqs"]), int(params["q_len"])
    Hq, G, Hi = int(params["num_q_heads"]), int(params["num_kv_heads"]), int(params["idx_heads"])
    L = np.minimum(np.asarray(ctx_lens, dtype=np.int64), int(params["max_blocks_per_seq"]) * 128)
    nblk = (L + 127) // 128
    return {
        "idx_keys": int(L.sum()) * IDX_KEY_BYTES[int(params["idx_dtype"])],
        "kv": int(union_blocks) * G * 128 * KV_BYTES[int(params["kv_dtype"])],
        "q": B * Tq * Hq * 128 * 2,
        "out": B * Tq * Hq * 128 * 2,
        "idx_q": B * Tq * Hi * 64 * 2,
        "idx_w": B * Tq * Hi * 4,
        "table": int(nblk.sum()) * 4,
        "ctx_lens": B * 4,
    }


def union_blocks(sel):
    """Distinct selected blocks per sequence, summed: sel int [B][Tq][top_k],
    -1 padded."""
    return sum(len(set(int(x) for x in sel[b].ravel() if x >= 0)) for b in range(sel.shape[0]))


def indexer_bytes(params, ctx_lens):
    """Bytes of the indexer + pool stage: indexer keys, indexer queries and
    weights, block-table entries, context lengths."""
    t = step_byte_terms(params, ctx_lens, 0)
    return t["idx_keys"] + t["idx_q"] + t["idx_w"] + t["table"] + t["ctx_lens"]


def attention_bytes(params, ctx_lens, sel):
    """Bytes of the selection + attention stage: K/V of the union of the
    selected blocks per sequence, queries and outputs."""
    t = step_byte_terms(params, ctx_lens, union_blocks(sel))
    return t["kv"] + t["q"] + t["out"]


def dense_kv_bytes(params, ctx_lens):
    """K/V bytes that dense attention over every visible key would read."""
    L = np.minimum(np.asarray(ctx_lens, dtype=np.int64), int(params["max_blocks_per_seq"]) * 128)
    return int(L.sum()) * int(params["num_kv_heads"]) * KV_BYTES[int(params["kv_dtype"])]


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


# ------------------------------------------------------------ oracle checks

TIE_REL = 1e-4   # selections may differ only where the k-th ranked pooled score is this close


def selection_verdict(gpu_row, r, top_k, keep_last):
    """0: the GPU selected the oracle's blocks; 1: the two sets differ only
    in blocks whose oracle pooled score lies within TIE_REL (relative) of
    the k-th ranked (keep-last adjusted) oracle pooled score; 2: otherwise."""
    from oracle import msa_oracle as O
    g = sorted(int(x) for x in gpu_row if x >= 0)
    o = [int(x) for x in r["sel"]]
    if g == o:
        return 0
    kth, _ = O.boundary_values(r["pooled"], top_k, keep_last)
    if kth is None or not np.isfinite(kth) or len(g) != len(o):
        return 2
    for blk in set(g) ^ set(o):
        if blk >= len(r["pooled"]) or abs(r["pooled"][blk] - kth) > TIE_REL * max(abs(kth), 1e-30):
            return 2
    return 1


def compare_tokens(w, b, res, gpu_res, acc):
    """Accumulate the comparison of sequence b's oracle results `res` with the
    GPU step's selections and outputs into the dict `acc`."""
    prm = w.params
    for t, r in enumerate(res):
        if r["p"] < 0:
            continue
        v = selection_verdict(gpu_res["sel"][b, t], r, prm["top_k"], prm["keep_last"])
        acc["tokens"] += 1
        acc["tie_band_tokens"] += v == 1
        acc["other_selection_tokens"] += v == 2
        if v == 0 and "out" in gpu_res:
            err = np.abs(gpu_res["out"][b, t] - r["out"])
            small = np.abs(r["out"]) < 0.5
            if small.any():
                acc["max_abs"] = max(acc["max_abs"], float(err[small].max()))
            if (~small).any():  # in bf16 ulps of the oracle value (2^(e-7) for |o| in [2^e, 2^(e+1)))
                ulp = 2.0 ** (np.floor(np.log2(np.abs(r["out"][~small]))) - 7)
                acc["max_ulp"] = max(acc["max_ulp"], float((err[~small] / ulp).max()))
            acc["sum_abs"] += float(err.sum())
            acc["n_elems"] += err.size


def new_acc():
    return dict(tokens=0, tie_band_tokens=0, other_selection_tokens=0, max_abs=0.0, max_ulp=0.0, sum_abs=0.0,
                n_elems=0)


def acc_summary(acc):
    return {"tokens_compared": acc["tokens"], "tie_band_tokens": acc["tie_band_tokens"],
            "other_selection_tokens": acc["other_selection_tokens"], "out_max_abs_where_o_below_0_5": acc["max_abs"],
            "out_max_bf16_ulps_where_o_at_least_0_5": acc["max_ulp"],
            "out_mean_abs": acc["sum_abs"] / max(acc["n_elems"], 1)}


def cpu_baseline(w, gpu_res, budget_s=20.0):
    """Time the oracle (as it stands) on whole sequences of the workload until
    about budget_s seconds of CPU work; also compare its results with the GPU
    step's on those sequences."""
    from oracle import msa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas = None
    prm = w.params
    acc = new_acc()
    t0 = time.perf_counter()
    done_tok, seqs = 0, 0
    for b in range(prm["num_seqs"]):
        res = O.decode_sequence(w, b)
        done_tok += len(res)
        seqs += 1
        compare_tokens(w, b, res, gpu_res, acc)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_tok / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "blas_threads": blas, "kind": "oracle",
            "sample": "%d of %d sequences (%d query tokens) of the same workload, float64 numpy, %.1f s" % (
                seqs, prm["num_seqs"], done_tok, dt),
            "sample_check": acc_summary(acc)}


# ------------------------------------------------------------ GPU runs

class Runner:
    """Device replicas of one workload and the prebuilt C arguments of its
    decode-layer call, so that a timed step is one C-ABI call."""

    def __init__(self, w, layer="auto", replicas=0):
        import ctypes
        import torch
        import block_sparse_attention_kv_amd as msa
        self.w, self.torch, self.msa = w, torch, msa
        prm = w.params
        B, Tq, Hq = prm["num_seqs"], prm["q_len"], prm["num_q_heads"]
        step_guess = indexer_bytes(prm, w.ctx_lens) + B * prm["num_kv_heads"] * 64 * 128 * 144
        self.R = replicas or max(2, min(4, int(math.ceil(3 * 256e6 / max(step_guess, 1)))))
        dev = "cuda"
        self.reps = [msa.to_device(w, dev) for _ in range(self.R)]
        self.out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device=dev)
        self.lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, Tq, prm["top_k"]), dtype=torch.int32, device=dev)
        self.ws = msa.alloc_workspace(self.reps[0][0], dev)
        L = self.L = msa.load()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        ws_bytes = self.ws.numel() * self.ws.element_size()
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        self.keep, self.call_args = [], []
        for params, cache, qs in self.reps:
            c = cache.c()
            self.keep.append(c)
            self.call_args.append([ctypes.byref(params), ctypes.byref(c), vp(qs["q"]), vp(qs["idx_q"]),
                                   vp(qs["idx_w"]), vp(self.out), vp(self.lse), vp(self.sel), vp(self.ws),
                                   ctypes.c_size_t(ws_bytes), stream])
        self.items = B * Tq * prm["num_kv_heads"]
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count
        single_ok = prm["kv_dtype"] == 1 and prm["idx_dtype"] in (1, 2) and Tq <= 4
        if layer == "auto":
            # the single launch wherever it applies: it matches or beats the
            # two-kernel layer on every measured workload
            self.single = single_ok
        else:
            self.single = layer == "single"
            if self.single and not single_ok:
                raise SystemExit("--layer single: this configuration needs the two-kernel path")
        self.kernel = "decode_layer_single" if self.single else "indexer_pool"
        self.entry = "msa_decode_layer_single" if self.single else "msa_decode_layer"
        self.plain = L.msa_decode_layer_single if self.single else L.msa_decode_layer
        self.traced_fn = L.msa_decode_layer_single_traced if self.single else L.msa_decode_layer_traced
        self.stage_names = ["decode_layer_single"] if self.single else list(msa.STAGE_NAMES)
        torch.cuda.synchronize()

    def step(self, i, events=None):
        st = self.plain(*self.call_args[i % self.R]) if events is None else \
            self.traced_fn(*self.call_args[i % self.R], events)
        if st != 0:
            raise RuntimeError("%s: %s" % (self.entry, self.L.msa_last_error().decode()))

    def results(self):
        torch = self.torch
        torch.cuda.synchronize()
        return {"sel": self.sel.cpu().numpy(),
                "out": (self.out.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.uint32) << 16)
                .view(np.float32).astype(np.float64)}

    def timed(self, steps):
        """K steps between two HIP events on the launch stream: ms per step."""
        torch = self.torch
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            self.step(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def traced(self, steps):
        """K steps whose kernels record their own start and end events
        (hipExtLaunchKernel): per-kernel durations (ms) of every step."""
        import ctypes
        torch = self.torch
        n = len(self.stage_names)
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n)] for _ in range(steps)]
        for row in kev:          # create the HIP events before the pass
            for e in row:
                e.record()
        torch.cuda.synchronize()
        arrays = [(ctypes.c_void_p * (2 * n))(*[e.cuda_event for e in row]) for row in kev]
        for i in range(steps):
            self.step(i, arrays[i])
        torch.cuda.synchronize()
        return [np.array([kev[i][2 * s].elapsed_time(kev[i][2 * s + 1]) for i in range(steps)]) for s in range(n)]

    def release(self):
        self.reps = self.call_args = self.keep = None
        self.out = self.lse = self.sel = self.ws = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def step_report(w, ms_step, sel):
    prm = w.params
    terms = step_byte_terms(prm, w.ctx_lens, union_blocks(sel))
    step_b = sum(terms.values())
    gbps = step_b / (ms_step * 1e-3) / 1e9
    return terms, step_b, gbps


def other_workload(cfg, steps, warmup, layer, nvfp4_idx=False):
    """Compact measurement of another decode workload (with nvfp4_idx, the
    same configuration with NVFP4 indexer keys): step time, rate, fraction of
    the HBM peak, and the selection of every query token checked against the
    oracle (tie-band and other differences counted)."""
    from oracle import msa_oracle as O
    from workloads import make_config, CONFIG_NAMES, IDX_NVFP4
    t0 = time.perf_counter()
    w = make_config(cfg, idx_dtype=IDX_NVFP4 if nvfp4_idx else None)
    run = Runner(w, layer)
    for i in range(warmup):
        run.step(i)
    ms = run.timed(steps)
    gpu_res = run.results()
    entry = run.entry
    run.release()
    terms, step_b, gbps = step_report(w, ms, gpu_res["sel"])
    acc = new_acc()
    for b in range(w.B):
        compare_tokens(w, b, O.decode_sequence(w, b), gpu_res, acc)
    prm = w.params
    rep = {"config_id": str(cfg) + ("/nvfp4" if nvfp4_idx else ""),
           "workload": CONFIG_NAMES[cfg] + (", NVFP4 idx keys instead of FP8" if nvfp4_idx else ""),
           "entry": entry, "steps": steps,
           "warmup": warmup, "ms_per_step": ms, "tokens_per_s": prm["num_seqs"] * prm["q_len"] / (ms * 1e-3),
           "algorithmic_bytes": step_b, "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
           "oracle_check": acc_summary(acc)}
    log("%s: %s %.4f ms/step, %.0f GB/s (%.3f), ties %d, other %d (%.1f s)" % (
        w.name, entry, ms, gbps, gbps / HBM_PEAK_GBPS, acc["tie_band_tokens"], acc["other_selection_tokens"],
        time.perf_counter() - t0))
    del w
    return rep


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
    ap.add_argument("--no-others", action="store_true",
                    help="skip the compact measurements of the other decode workloads")
    ap.add_argument("--other-steps", type=int, default=50)
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many steps and a 1 GiB calibration copy (for rocprofv3 runs)")
    ap.add_argument("--layer", choices=("auto", "single", "two"), default="auto",
                    help="single: msa_decode_layer_single; two: msa_decode_layer; auto: single where it applies "
                         "(NVFP4 K/V, FP8 or NVFP4 indexer keys, q_len <= 4)")
    ap.add_argument("--layer-splits", type=int, default=0, choices=(0, 1, 2, 4),
                    help="workgroups per attention item of the single launch (0: the library's choice)")
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

    if args.layer_splits:
        msa.msa_debug_layer_splits(args.layer_splits)
    t0 = time.perf_counter()
    w = make_config(args.config, idx_dtype=IDX_NVFP4 if args.idx_dtype == "nvfp4" else None)
    log("generated %s in %.1f s (%.2f GB host)" % (w.name, time.perf_counter() - t0, w.nbytes() / 1e9))
    prm = w.params
    B, Tq = prm["num_seqs"], prm["q_len"]
    run = Runner(w, args.layer, args.replicas)
    log("uploaded %d replica(s) in %.1f s; layer path: %s (%d items, %d compute units)" % (
        run.R, time.perf_counter() - t0, run.entry, run.items, run.cus))

    if args.profile_steps:
        for i in range(args.profile_steps):
            run.step(i)
        torch.cuda.synchronize()
        log("profile run: %d steps done" % args.profile_steps)
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        return

    # ---- attainable bandwidth on this machine (context), measured first: the
    # GPU's clocks settle only after some milliseconds of load, and this
    # measurement and the event-traced pass below provide that load before
    # the timed region
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
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
    chk = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        msa.msa_debug_read_bandwidth(src, chk)
    c0.record()
    for _ in range(30):
        msa.msa_debug_read_bandwidth(src, chk)
    c1.record()
    torch.cuda.synchronize()
    read_gbps = (1 << 30) * 30 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    log("attainable on this box: read %.0f GB/s (1 GiB stream), device copy %.0f GB/s (read + write)"
        % (read_gbps, copy_gbps))
    del src, dst

    for i in range(args.warmup):
        run.step(i)
    # ---- per-kernel durations: K steps whose kernels' dispatches record
    # their own start and end (these events lengthen the step a little, so
    # the step time comes from the plain pass below)
    stage_all = run.traced(max(args.steps, TRACED_MIN_STEPS))
    stage_ms = [float(np.mean(d)) for d in stage_all]
    stage_pct = {n: [float(x) for x in np.percentile(d, [10, 50, 90])] for n, d in zip(run.stage_names, stage_all)}
    log("kernels (ms, event-traced pass): " + ", ".join("%s %.4f" % (n, v) for n, v in zip(run.stage_names, stage_ms)))

    # ---- timed region: K steps between two HIP events on the launch stream
    ms_step = run.timed(args.steps)
    gpu_res = run.results()
    log("timed %d steps: %.4f ms/step" % (args.steps, ms_step))

    kernel, entry, single, stage_names = run.kernel, run.entry, run.single, run.stage_names
    run.release()

    terms, step_b, step_gbps = step_report(w, ms_step, gpu_res["sel"])
    idx_b = indexer_bytes(prm, w.ctx_lens)
    att_b = attention_bytes(prm, w.ctx_lens, gpu_res["sel"])
    stages = {}
    if single:
        # one kernel is the whole step: its duration per launch is the timed
        # region's time per step (back-to-back launches on one stream)
        kern_b, kern_ms = step_b, ms_step
    else:
        kern_b, kern_ms = idx_b, stage_ms[0]
        for n, b_, ms in zip(stage_names, (idx_b, att_b), stage_ms):
            stages[n] = {"algorithmic_bytes": b_, "avg_ms": ms, "gbps": b_ / (ms * 1e-3) / 1e9,
                         "frac": b_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    kern_gbps = kern_b / (kern_ms * 1e-3) / 1e9
    rec = traffic_record(kernel, wkey)
    res = {
        "metric": METRIC,
        "value": B * Tq / (ms_step * 1e-3),
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
                   "ctx_len": int(w.ctx_lens.max()), "q_heads": prm["num_q_heads"],
                   "kv_heads": prm["num_kv_heads"], "idx_heads": prm["idx_heads"], "top_k": prm["top_k"],
                   "block": 128, "input_replicas": run.R},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": kern_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": kern_gbps / HBM_PEAK_GBPS,
                     "traffic": None if rec is None else rec["traffic_bytes_per_launch"],
                     "algorithmic_bytes": kern_b, "avg_ms": kern_ms,
                     "avg_ms_from": "timed region, one kernel per step" if single else "event-traced pass"},
        "step": {"entry": entry, "algorithmic_bytes": step_b, "byte_terms": terms, "gbps": step_gbps,
                 "frac": step_gbps / HBM_PEAK_GBPS, "dense_kv_bytes": dense_kv_bytes(prm, w.ctx_lens),
                 "msa_over_dense": (terms["idx_keys"] + terms["kv"]) / dense_kv_bytes(prm, w.ctx_lens),
                 "traced_stage_ms": dict(zip(stage_names, stage_ms)),
                 "traced_stage_ms_p10_p50_p90": stage_pct, "stages": stages,
                 "indexer_bytes": idx_b, "attention_bytes": att_b,
                 "copy_gbps_attainable": copy_gbps, "read_gbps_attainable": read_gbps},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, gpu_res, args.cpu_budget)
    del w
    if not args.no_others and args.config == 3 and args.idx_dtype == "fp8":
        # 300 untimed steps each (at most ~21 ms), so that these compact
        # measurements are of the steady state too
        res["other_workloads"] = [other_workload(c, args.other_steps, max(args.warmup, 300), args.layer, nv)
                                  for c, nv in ((2, False), (4, False), (5, False), (3, True))]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
