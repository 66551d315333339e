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
the `roofline` object prices the attention call (its average duration from
HIP events on the launch stream) against the bf16 MFMA peak using the exact
count of visible (query, key) pairs: FLOPs = 4 * d * Hq * pairs. The
`cpu_baseline` object times the float64 CPU oracle on a bounded random sample
of the same workload's query rows.
"""
import argparse
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

WORKLOADS = {
    "c1": "tiny fp32: 1 request, 2 SSep spans of 32 + 16-token PDep query; Hq 4, Hkv 2, d 64, RoPE base 1e4",
    "c2": "8B shape: 1 request, system prompt 512 + 10 SSep spans of 192 + 64-token PDep question, all fresh; "
          "Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c3": "8B shape: 16 requests, each 10 of 40 shared cached 192-token spans in random order + 64-token PDep "
          "question; Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c4": "8B shape long context: 1 request, 120 SSep spans of 256 (60 cached, 60 fresh) + 512-token PDep suffix; "
          "Hq 32, Hkv 8, d 128, bf16, RoPE base 5e5",
    "c5": "70B shape: 8 requests, shared cached 256-token GLOBAL prefix + 20 fresh SSep spans of U{128..512} "
          "padded to 16 + 128-token PDep question; Hq 64, Hkv 8, d 128, bf16, RoPE base 5e5",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables the cpu_baseline leg)")
    return ap.parse_args()


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

    n0, t0 = run(8)
    per_row = t0 / max(n0, 1)
    n = int(max(8, min(int(counts.sum()), target_s / max(per_row, 1e-6))))
    n, t = run(n)
    return {"value": n / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly from the {int(counts.sum())} of workload {w.name}, "
                      f"float64 numpy oracle, {t:.1f} s"}


def main():
    a = parse()
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

    # ---- per-call durations on the launch stream (HIP events)
    reps = max(a.steps, 20)
    ms_attn = timed(dw.attend, reps)
    ms_prerot = timed(dw.attend_prerotated, reps)
    ms_wkv = timed(dw.write_new, reps)
    log(f"[bench] attn {ms_attn:.4f} ms, prerotated {ms_prerot:.4f} ms, write_kv {ms_wkv:.4f} ms")

    tflops = flops / (ms_attn * 1e-3) / 1e12
    step_tflops = flops / (ms_step * 1e-3) / 1e12
    value = w.total_q / (ms_step * 1e-3)
    if w.dtype == "bf16":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        roof = {"bound": "alu", "achieved": round(tflops, 4), "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_F32_VALU_TFLOPS, 6), "traffic": None}

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
        "tflops_attention": round(tflops, 2),
        "pct_mfma_bf16_peak_attention": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "kernels": {
            "prefill_attn_ms": round(ms_attn, 5),
            "reference_prerotated_ms": round(ms_prerot, 5),
            "rope_overhead_pct": round(100 * (ms_attn / ms_prerot - 1), 2),
            "write_kv_ms": round(ms_wkv, 5),
            "write_kv_GBps": round(kv_bytes / (ms_wkv * 1e-3) / 1e9, 1),
            "plan": info,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
