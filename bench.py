#!/usr/bin/env python3
"""Benchmark of position-free paged prefill attention on one MI355X.

One step is one pass of the whole hot path over one synthetic batch that is
already resident in HBM:
  1. minipic_write_kv     - scatter this step's unrotated K and V into the paged cache
  2. minipic_prefill_attn - paged gather, in-kernel RoPE on K tiles, block mask
                            from span descriptors, online-softmax flash loop on
                            bf16 MFMA, split-KV combine

Default workload (c4): Llama-3.1-8B attention shape (32 query heads, 8 KV
heads, head dim 128, bf16, RoPE base 5e5), one request of 120 SSep spans of
256 tokens (a seeded half cached, half computed in the step) and a 512-token
PDep suffix: 15,872 query tokens over a 31,232-token context.

Prints ONE JSON line. `value` is query tokens per second of the whole step;
the `roofline` object prices the attention kernel (its average launch
duration over a second pass of the same timed steps, from the HIP events the
library records around its launches on the launch stream, read once after the
last step)
against the bf16 MFMA peak using the exact count of visible (query, key)
pairs: FLOPs = 4 * d * Hq * pairs. Its `traffic` is the kernel's HBM bytes per
launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by what the
same counters read for a plain copy of known size), read from the record in
profiles/ while the kernel sources still hash to the values it names, else
null. The `cpu_baseline` object times the float64 CPU oracle on a bounded
random sample of the same workload's query rows.

Two helper modes serve the counter record:
  --calibrate-copy           run a plain device-to-device copy of known size
                             (profile it with --pmc FETCH_SIZE / WRITE_SIZE)
  --summarize-counters DIRS  turn rocprofv3 counter CSVs of this script (the
                             bench runs and the copy runs) into the record
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attention tokens/s and TFLOP/s (% of MFMA bf16 peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 4096 flop/clk x 2.4 GHz
PEAK_F32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["position_independent_paged_amd/csrc/attn_bf16.hip", "position_independent_paged_amd/csrc/common.h"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_bf16_c4_traffic.json")
COPY_BYTES = 1 << 30

WORKLOADS = {
    "c1": "tiny fp32: 1 request, 2 SSep spans of 32 + 16-token PDep query; Hq 4, Hkv 2, d 64, RoPE base 1e4",
    "c2": "8B shape: 1 request, system prompt 512 + 10 SSep spans of 192 + 64-token PDep question, all fresh; "
          "Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c3": "8B shape: 16 requests, each 10 of 40 shared cached 192-token spans in random order + 64-token PDep "
          "question; Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c3w": "8B shape, retrieval batch: 64 requests, each 10 of 160 shared cached documents of 100 tokens padded "
           "to 112, in random order, + 64-token PDep question; Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c4": "8B shape long context: 1 request, 120 SSep spans of 256 (60 cached, 60 fresh) + 512-token PDep suffix; "
          "Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c5": "70B shape: 8 requests, shared cached 256-token GLOBAL prefix + 20 fresh SSep spans of U{128..512} "
          "padded to 16 + 128-token PDep question; Hq 64, Hkv 8, d 128, bf16, RoPE base 5e5",
    "e2": "C2 with each span's first block recomputed against all earlier context (EPIC / LegoLink) and the "
          "rest of the span an SSep span that sees it",
    "e4": "C4's context, every span cached except its first block, recomputed against all earlier context "
          "(EPIC / LegoLink), + the 512-token PDep suffix",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c4", choices=sorted(k for k in WORKLOADS if k.startswith("c")))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--suite", default="c2,c3,c3w,c5,e2,e4,d2,d3,d4,d5",
                    help="other workloads whose attention is timed beside the main one (empty: none)")
    ap.add_argument("--sweeps", action="store_true",
                    help="only run the kernel sweeps that mirror the pages' preload / TTFT figure and print "
                         "one JSON line per point")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                              "COPY_WRITE_DIR"),
                    help="write the traffic record from rocprofv3 --pmc output directories")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_means(d, counter, name_filter):
    """Mean per-dispatch value of `counter` over the dispatches whose kernel name contains `name_filter`."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or name_filter not in r["Kernel_Name"]:
                continue
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {name_filter!r} under {d}")
    return sum(per.values()) / len(per), len(per)


def summarize_counters(dirs):
    fetch_d, write_d, cfetch_d, cwrite_d = dirs
    kname = "attn_bf16_kernel<128, 4, true"
    fetch_kib, nf = counter_means(fetch_d, "FETCH_SIZE", kname)
    write_kib, nw = counter_means(write_d, "WRITE_SIZE", kname)
    copy_name = "copyBuffer"
    cfetch_kib, _ = counter_means(cfetch_d, "FETCH_SIZE", copy_name)
    cwrite_kib, _ = counter_means(cwrite_d, "WRITE_SIZE", copy_name)
    sf = COPY_BYTES / (cfetch_kib * 1024.0)
    sw = COPY_BYTES / (cwrite_kib * 1024.0)
    rec = {
        "kernel": kname + ", 1>",
        "workload": "c4",
        "kernel_sources_sha256": kernel_source_hash(),
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "fetch_dispatches": nf,
        "write_kib_per_dispatch": round(write_kib, 1), "write_dispatches": nw,
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib": round(cfetch_kib, 1), "copy_write_kib": round(cwrite_kib, 1),
        "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
        "hbm_bytes_per_launch": int(round((fetch_kib * sf + write_kib * sw) * 1024.0)),
    }
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def recorded_traffic():
    """HBM bytes per launch of the attention kernel from the counter record, if it matches the sources."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy():
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, target_s, seed=0):
    """Time the float64 oracle on a random sample of query rows (rank 0, N=1 only)."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default is one thread per core
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(seed)
    counts = np.diff(w.q_indptr).astype(np.int64)
    reqs = np.nonzero(counts)[0]

    def run(n):
        # rows drawn uniformly over all query rows, grouped per request
        flat = np.sort(rng.choice(int(counts.sum()), size=min(n, int(counts.sum())), replace=False))
        owner = np.searchsorted(w.q_indptr[1:], flat, side="right")
        t0 = time.perf_counter()
        done = 0
        for r in reqs:
            rows = flat[owner == r] - int(w.q_indptr[r])
            if len(rows):
                oracle.workload_reference(w, int(r), rows=rows)
                done += len(rows)
        return done, time.perf_counter() - t0

    n, t = run(8)
    # rescale the sample until it takes at least 60% of the target time (the
    # first rows of a request pay its one-off setup, so small samples mislead)
    for _ in range(3):
        if t >= 0.6 * target_s or n >= int(counts.sum()):
            break
        n = int(max(8, min(int(counts.sum()), n * target_s / max(t, 1e-6))))
        n, t = run(n)
    return {"value": n / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly from the {int(counts.sum())} of workload {w.name}, "
                      f"float64 numpy oracle, {t:.1f} s",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_model():
    """Model name of the host CPU (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def algorithmic_bytes(w):
    """Q + out + unique K/V + the cos/sin rows of the distinct positions read (one pass each)."""
    import numpy as np
    elem = 2 if w.dtype == "bf16" else 4
    qo = 2 * int(w.total_q) * w.num_q_heads * w.head_dim * elem
    blocks, positions = set(), set()
    for r in range(int(w.num_reqs)):
        L = int(w.ctx_len[r])
        nb = (L + w.block_size - 1) // w.block_size
        blocks.update(int(b) for b in w.block_table[r, :nb])
        positions.update(int(p) for p in np.unique(w.logical_pos[r, :L]))
    kv = 2 * len(blocks) * w.block_size * w.num_kv_heads * w.head_dim * elem
    cs = len(positions) * w.head_dim * 4
    return qo + kv + cs


def graph_steps(step, ms_step, reps=5):
    """ms per step of `step` replayed from one captured HIP graph of N steps
    (N so that one replay takes >= 50 ms), median over `reps` replays."""
    import statistics
    import torch
    n = max(10, min(2000, int(50.0 / max(ms_step, 1e-3)) + 1))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(n):
            step()
    g.replay()                            # first replay uploads the graph
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n)
    del g
    return {"ms_per_step_median": round(statistics.median(times), 5), "reps": reps, "steps_per_replay": n,
            "ms_per_step_all": [round(t, 5) for t in times]}


def shader_clock_mhz(workspace):
    """Shader clock over the attention kernel's last launch, from the clock stamps
    its first work-group leaves at bytes 128..159 of the workspace (shader clock
    counter and 100 MHz real-time counter at start and end), or None."""
    import torch
    torch.cuda.synchronize()
    c0, r0, c1, r1 = (int(v) for v in workspace[128:160].view(torch.int64).cpu().tolist())
    if r1 <= r0 or c1 <= c0:
        return None
    return round(100.0 * (c1 - c0) / (r1 - r0), 1)


def steps_kernel_ms(step, n):
    """Average (plan, attention, merge) kernel durations over n back-to-back calls of `step` (each making one
    attention call), from the HIP events the library records around its launches, read after the last step."""
    import torch
    from position_independent_paged_amd import minipic_kernel_times_all, minipic_set_kernel_timing
    torch.cuda.synchronize()
    minipic_set_kernel_timing(True)
    try:
        for _ in range(n):
            step()
        times = minipic_kernel_times_all(n)
    finally:
        minipic_set_kernel_timing(False)
    if len(times) != n:
        raise RuntimeError(f"{len(times)} timed calls, expected {n}")
    return [sum(t[i] for t in times) / n for i in range(3)]


def paired_kernel_ms(step_a, step_b, n, blocks=4):
    """Attention kernel ms of `step_a` and of `step_b` (each one attention call), timed in `blocks` alternating
    runs of n / blocks calls each, so that both see the same clock and cache conditions; returns (a, b)."""
    per = max(1, n // blocks)
    ta = tb = 0.0
    for _ in range(blocks):
        ta += steps_kernel_ms(step_a, per)[1]
        tb += steps_kernel_ms(step_b, per)[1]
    return ta / blocks, tb / blocks


def calls_ms(call, n):
    """Average time of n back-to-back calls on the current stream, one event pair around all of them."""
    import torch
    call()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def private_copy_prerotated(dw, w, reps):
    """Attention kernel time of the pre-rotated reference when every request owns private copies of
    its blocks (a shared span at different positions needs one rotated copy per position)."""
    import numpy as np
    import torch
    from position_independent_paged_amd import minipic_reference_prerotated
    from position_independent_paged_amd.staging import DeviceBatch
    R, MB = w.block_table.shape
    bt = np.full((R, MB), -1, np.int32)
    src = []
    for r in range(R):
        nb = (int(w.ctx_len[r]) + w.block_size - 1) // w.block_size
        bt[r, :nb] = np.arange(len(src), len(src) + nb, dtype=np.int32)
        src.extend(int(b) for b in w.block_table[r, :nb])
    idx = torch.tensor(src, dtype=torch.int64, device=dw.k_cache.device)
    k_priv = dw.k_cache.index_select(0, idx)
    v_priv = dw.v_cache.index_select(0, idx)
    batch = DeviceBatch(q_indptr=w.q_indptr, q_ctx_idx=w.q_ctx_idx, ctx_len=w.ctx_len, block_table=bt,
                        logical_pos=w.logical_pos, span_id=w.span_id, blk_flags=w.blk_flags,
                        num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                        block_size=w.block_size, device=dw.k_cache.device)

    def call():
        minipic_reference_prerotated(dw.q, k_priv, v_priv, len(src), batch.struct, dw.out, dw.workspace,
                                     cos_sin=dw.cos_sin, max_pos=dw.max_pos)
    call()
    ms = steps_kernel_ms(call, reps)[1]
    unique = 2 * len(src) * w.block_size * w.num_kv_heads * w.head_dim * (2 if w.dtype == "bf16" else 4)
    del k_priv, v_priv
    return ms, unique


def decode_entry(name, reps):
    """Decode attention of the decode view of a workload: time against the HBM roofline, RoPE overhead."""
    import torch
    import workload
    from position_independent_paged_amd import metrics
    from position_independent_paged_amd.staging import DeviceWorkload
    w = workload.make_config(name)
    dw = DeviceWorkload(w, device="cuda:0")
    dw.write_new()
    for _ in range(3):
        dw.decode()
        dw.decode_prerotated()
    torch.cuda.synchronize()
    if dw.decode_error_word() != 0:
        raise RuntimeError(f"{name}: kernel error word {dw.decode_error_word():#x}")
    nbytes = metrics.decode_bytes(w)
    _, attn, merge = steps_kernel_ms(dw.decode, reps)
    # RoPE overhead: the two kernels in alternating runs of calls
    attn_p, prerot = paired_kernel_ms(dw.decode, dw.decode_prerotated, reps)
    gbs = nbytes / (attn * 1e-3) / 1e9
    # whole calls (decode kernel + merge) back to back between one pair of events: free of
    # the few microseconds that events around every launch add to such short kernels
    call_ms = calls_ms(dw.decode, 10 * reps)
    call_ms_prerot = calls_ms(dw.decode_prerotated, 10 * reps)
    # whole calls replayed from a captured HIP graph: the GPU's time per call, free of the host's launch rate
    graph = graph_steps(dw.decode, call_ms, reps=5)["ms_per_step_median"]
    graph_prerot = graph_steps(dw.decode_prerotated, call_ms_prerot, reps=5)["ms_per_step_median"]
    e = {"workload": f"decode step after {name.replace('d', 'c', 1)}: one query row per request (its last "
                     f"context token)", "requests": int(w.num_reqs), "context_tokens": int(w.ctx_len.sum()),
         "algorithmic_MB": round(nbytes / 1e6, 2), "decode_kernel_ms": round(attn, 5),
         "merge_kernel_ms": round(merge, 5), "GBps_kernel": round(gbs, 1),
         "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "prerotated_kernel_ms": round(prerot, 5),
         "rope_overhead_pct": round(100 * (attn_p / prerot - 1), 2),
         "call_ms_back_to_back": round(call_ms, 5), "prerotated_call_ms_back_to_back": round(call_ms_prerot, 5),
         "GBps_call_back_to_back": round(nbytes / (call_ms * 1e-3) / 1e9, 1),
         "rope_overhead_call_pct": round(100 * (call_ms / call_ms_prerot - 1), 2),
         "call_ms_graph_replay": graph, "prerotated_call_ms_graph_replay": graph_prerot,
         "GBps_call_graph_replay": round(nbytes / (graph * 1e-3) / 1e9, 1),
         "rope_overhead_graph_pct": round(100 * (graph / graph_prerot - 1), 2)}
    del dw
    torch.cuda.empty_cache()
    return e


def suite_entry(name, reps):
    """Attention kernel of one more workload: time, MFMA and HBM fractions, RoPE overhead."""
    if name.startswith("d"):
        return decode_entry(name, reps)
    import torch
    import workload
    from position_independent_paged_amd import metrics
    from position_independent_paged_amd.staging import DeviceWorkload
    w = workload.make_config(name)
    dw = DeviceWorkload(w, device="cuda:0")
    dw.write_new()
    for _ in range(3):
        dw.attend()
        dw.attend_prerotated()
    torch.cuda.synchronize()
    if dw.error_word() != 0:
        raise RuntimeError(f"{name}: kernel error word {dw.error_word():#x}")
    pairs = metrics.workload_pairs(w)
    flops = metrics.attention_flops(pairs, w.num_q_heads, w.head_dim)
    nbytes = algorithmic_bytes(w)
    # the step sequence of the main measurement: write_kv, then the call
    def step():
        dw.write_new()
        dw.attend()

    def step_prerotated():
        dw.write_new()
        dw.attend_prerotated()
    plan, attn, merge = steps_kernel_ms(step, reps)
    # RoPE overhead: the two kernels in alternating runs of steps
    attn_p, prerot = paired_kernel_ms(step, step_prerotated, reps)
    tf = flops / (attn * 1e-3) / 1e12
    e = {"workload": WORKLOADS[name], "query_tokens": int(w.total_q), "gflop": round(flops / 1e9, 3),
         "algorithmic_MB": round(nbytes / 1e6, 1),
         "attention_kernel_ms": round(attn, 5), "plan_kernels_ms": round(plan, 5), "merge_kernel_ms": round(merge, 5),
         "tflops_kernel": round(tf, 2), "pct_mfma_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
         "pct_hbm_peak": round(100 * nbytes / (attn * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
         "prerotated_kernel_ms": round(prerot, 5), "rope_overhead_pct": round(100 * (attn_p / prerot - 1), 2)}
    if name in ("c3", "c3w"):   # shared documents at different offsets
        ms, unique = private_copy_prerotated(dw, w, reps)
        e["prerotated_private_copies_kernel_ms"] = round(ms, 5)
        e["prerotated_private_copies_unique_kv_MB"] = round(unique / 1e6, 1)
        e["rope_overhead_vs_private_copies_pct"] = round(100 * (attn / ms - 1), 2)
    del dw
    torch.cuda.empty_cache()
    return e


def sweeps(reps=10):
    """Kernel-level mirror of the pages' preload / time-to-first-token figure (one
    attention layer, 8B shape): (a) one causal prompt of N tokens, no spans;
    (b) n documents of 1000 tokens (padded to 1008) prefilled together as SSep
    spans of one request; (c) n such documents cached and a 64-token PDep
    question computed, against the same with every document fresh."""
    import torch
    import workload
    from workload import Segment
    from position_independent_paged_amd import metrics
    from position_independent_paged_amd.staging import DeviceWorkload
    shape = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", rope_theta=5e5)

    def point(sweep, x, segs, **extra):
        L = sum(sg.length for sg in segs)
        w = workload.custom(f"{sweep}{x}", [segs], max_pos=max(32768, L), seed=x, **shape)
        dw = DeviceWorkload(w, device="cuda:0")
        dw.write_new()
        for _ in range(20):   # warm-up: the GPU settles under a few tens of ms of load
            dw.attend()
            dw.attend_prerotated()
        torch.cuda.synchronize()
        plan, attn, merge = steps_kernel_ms(dw.attend, reps)
        attn_p, prerot = paired_kernel_ms(dw.attend, dw.attend_prerotated, reps)
        flops = metrics.attention_flops(metrics.workload_pairs(w), w.num_q_heads, w.head_dim)
        rec = {"sweep": sweep, "x": x, "context_tokens": int(L), "query_tokens": int(w.total_q),
               "call_ms": round(plan + attn + merge, 5), "attention_kernel_ms": round(attn, 5),
               "prerotated_kernel_ms": round(prerot, 5), "rope_overhead_pct": round(100 * (attn_p / prerot - 1), 2),
               "tflops_kernel": round(flops / (attn * 1e-3) / 1e12, 1), **extra}
        print(json.dumps(rec), flush=True)
        del dw
        torch.cuda.empty_cache()

    for n in [1024, 2048, 4096, 8192, 16384, 32768]:
        point("prompt_length", n, [Segment("pdep", n)])
    for n in [1, 2, 4, 8, 16, 32]:
        point("doc_count_preload", n, [Segment("span", 1008) for _ in range(n)])
    for n in [1, 2, 4, 8, 16, 32]:
        point("doc_count_question_cached", n, [Segment("span", 1008, fresh=False) for _ in range(n)] +
              [Segment("pdep", 64)])
        point("doc_count_question_fresh", n, [Segment("span", 1008) for _ in range(n)] + [Segment("pdep", 64)])


def main():
    a = parse()
    if a.summarize_counters:
        summarize_counters(a.summarize_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {a.gpus} / WORLD_SIZE {world} is not supported "
              f"(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workload
    from position_independent_paged_amd import metrics
    from position_independent_paged_amd.staging import DeviceWorkload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.sweeps:
        sweeps()
        return
    log(f"[bench] generating {a.config}")
    w = workload.make_config(a.config)
    pairs = metrics.workload_pairs(w)
    flops = metrics.attention_flops(pairs, w.num_q_heads, w.head_dim)
    dw = DeviceWorkload(w, device="cuda:0")
    info = dw.launch_info()
    log(f"[bench] total_q={w.total_q} ctx={w.max_ctx_len} pairs/head={pairs} GFLOP={flops / 1e9:.2f} plan={info}")
    elem = 2 if w.dtype == "bf16" else 4
    kv_bytes = 2 * len(w.new_tok) * w.num_kv_heads * w.head_dim * elem * 2   # read + write, K and V

    def sync():
        torch.cuda.synchronize()

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        sync()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        sync()
        return e0.elapsed_time(e1) / n

    # warm-up (also checks the error word once)
    for _ in range(a.warmup):
        dw.step()
    sync()
    if dw.error_word() != 0:
        raise RuntimeError(f"kernel error word {dw.error_word():#x}")

    # ---- timed steps: the whole hot path
    log(f"[bench] timing {a.steps} steps")
    sync()
    t0 = time.perf_counter()
    ms_step = timed(dw.step, a.steps)
    wall = time.perf_counter() - t0
    log(f"[bench] {ms_step:.4f} ms/step (wall {wall:.3f} s)")

    # ---- the same steps replayed from a captured HIP graph (no launch gaps):
    # one graph of enough steps for >= 50 ms, replayed 5 times, median
    graph = graph_steps(dw.step, ms_step, reps=5)
    log(f"[bench] graph replay: {graph['ms_per_step_median']:.4f} ms/step (median of {graph['reps']} replays of "
        f"{graph['steps_per_replay']} steps)")


    # ---- the same timed steps again, with the HIP events the library records
    # around each of its launches on the launch stream (no wait between
    # steps): the kernels' durations inside the step sequence
    ms_plan, ms_kernel, ms_merge = steps_kernel_ms(dw.step, a.steps)
    ms_attn = ms_plan + ms_kernel + ms_merge
    sclk = shader_clock_mhz(dw.workspace)
    # the pre-rotated reference kernel in the same sequence (write_kv, then the call)
    def step_prerotated():
        dw.write_new()
        dw.attend_prerotated()
    # RoPE overhead: the kernel with and without the rotation in alternating runs of
    # steps (same clock and cache conditions for both)
    ms_kernel_paired, ms_kernel_prerot = paired_kernel_ms(dw.step, step_prerotated, a.steps)
    # ---- cold caches: the same steps, each after writing a 512 MB buffer on the
    # stream (more than L2 and the 256 MB Infinity Cache together), so every
    # K/V block, q row and table row comes from HBM; the library's events time
    # only its own kernels
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")

    def step_cold():
        # this step's K/V are written first, then the caches are flushed, so the
        # attention kernel reads every K/V block, q row and table row from HBM
        dw.write_new()
        scratch.fill_(1)
        dw.attend()
    ms_plan_cold, ms_kernel_cold, ms_merge_cold = steps_kernel_ms(step_cold, a.steps)
    del scratch

    # ---- a model's later layers (after the passes above): the batch's plan made
    # once (minipic_prefill_plan), each layer's step = write_kv +
    # minipic_prefill_run, replayed from a graph (a figure beside `value`,
    # which times whole steps)
    dw.plan()
    def layer_step():
        dw.write_new()
        dw.run()
    graph_layer = graph_steps(layer_step, ms_step, reps=5)
    log(f"[bench] graph replay, plan reused: {graph_layer['ms_per_step_median']:.4f} ms/step")
    reps = max(a.steps, 20)
    ms_wkv = timed(dw.write_new, reps)
    log(f"[bench] kernels in the timed steps: plan {ms_plan:.4f} ms, attention {ms_kernel:.4f} ms, "
        f"merge {ms_merge:.4f} ms; attention without RoPE {ms_kernel_prerot:.4f} ms; write_kv {ms_wkv:.4f} ms; "
        f"cold caches: attention {ms_kernel_cold:.4f} ms; shader clock {sclk} MHz")

    tflops = flops / (ms_kernel * 1e-3) / 1e12
    call_tflops = flops / (ms_attn * 1e-3) / 1e12
    step_tflops = flops / (ms_step * 1e-3) / 1e12
    value = w.total_q / (ms_step * 1e-3)
    if w.dtype == "bf16":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic() if a.config == "c4" else None}
    else:
        roof = {"bound": "alu", "achieved": round(tflops, 4), "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_F32_VALU_TFLOPS, 6), "traffic": None}

    suite = {}
    for name in [n for n in a.suite.split(",") if n and n != a.config]:
        log(f"[bench] suite: {name}")
        suite[name] = suite_entry(name, reps)
        e = suite[name]
        if "decode_kernel_ms" in e:
            log(f"[bench] suite {name}: decode {e['decode_kernel_ms']:.4f} ms, {e['GBps_kernel']:.0f} GB/s, "
                f"RoPE +{e['rope_overhead_pct']:.1f}%; back-to-back calls {e['call_ms_back_to_back']:.4f} ms "
                f"(with merge), RoPE +{e['rope_overhead_call_pct']:.1f}%; graph-replayed calls "
                f"{e['call_ms_graph_replay']:.4f} ms ({e['GBps_call_graph_replay']:.0f} GB/s), "
                f"RoPE +{e['rope_overhead_graph_pct']:.1f}%")
        else:
            log(f"[bench] suite {name}: {e['attention_kernel_ms']:.4f} ms, {e['tflops_kernel']:.1f} TFLOP/s, "
                f"RoPE +{e['rope_overhead_pct']:.1f}%")

    cpu = None
    if a.cpu_seconds > 0:
        log(f"[bench] cpu baseline (~{a.cpu_seconds:.0f} s of oracle work)")
        cpu = cpu_baseline(w, a.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{a.config}: {WORKLOADS[a.config]}",
            "query_tokens": int(w.total_q),
            "context_tokens": int(w.max_ctx_len),
            "requests": int(w.num_reqs),
            "visible_pairs_per_head": int(pairs),
            "gflop_per_step": round(flops / 1e9, 3),
        },
        "tflops_step": round(step_tflops, 2),
        "graph_replay": graph,
        "graph_replay_plan_reused": {"ms_per_step_median": graph_layer["ms_per_step_median"],
                                     "query_tokens_per_s": round(int(w.total_q) / (graph_layer["ms_per_step_median"] * 1e-3), 1),
                                     "note": "write_kv + minipic_prefill_run on a plan made once (a model's later "
                                             "layers); not the headline value"},
        "tflops_attention_call": round(call_tflops, 2),
        "tflops_attention_kernel": round(tflops, 2),
        "pct_mfma_bf16_peak_attention_kernel": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "kernels": {
            "prefill_attn_kernels_ms": round(ms_attn, 5),
            "plan_kernels_ms": round(ms_plan, 5),
            "attention_kernel_ms": round(ms_kernel, 5),
            "merge_kernel_ms": round(ms_merge, 5),
            "prerotated_attention_kernel_ms": round(ms_kernel_prerot, 5),
            "cold_cache": {"attention_kernel_ms": round(ms_kernel_cold, 5), "plan_kernels_ms": round(ms_plan_cold, 5),
                           "merge_kernel_ms": round(ms_merge_cold, 5),
                           "tflops_attention_kernel": round(flops / (ms_kernel_cold * 1e-3) / 1e12, 2)},
            "rope_overhead_pct": round(100 * (ms_kernel_paired / ms_kernel_prerot - 1), 2),
            "rope_overhead_note": "in-kernel RoPE against the pre-rotated kernel, both timed in 4 alternating runs of steps",
            "shader_clock_mhz": sclk,
            "pct_hbm_peak_attention_kernel": round(100 * algorithmic_bytes(w) / (ms_kernel * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
            "write_kv_ms": round(ms_wkv, 5),
            "write_kv_GBps": round(kv_bytes / (ms_wkv * 1e-3) / 1e9, 1),
            "plan": info,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "other_workloads": suite,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
