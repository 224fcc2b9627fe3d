#!/usr/bin/env python3
"""Benchmark of the MoBA prefill forward on one MI355X.

One step = one moba_attn_fwd call (block means, gate + top-k, dispatch,
past-block attention, own-block attention + merge) over the whole workload,
inputs resident in HBM.  Prints one JSON line.

Headline workload: 1M tokens, Llama-3.1-8B-shaped grouped-query attention
(32 query / 8 KV heads, head dim 128), block 4096, top-12, bf16.  The 32K
workload (32 heads, block 512, top-3, planted needles) is measured in the same
run and reported under "secondary".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (datasheet)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (datasheet)
METRIC = "MoBA prefill fwd useful TFLOP/s + tokens/s at 32K and 1M; MFMA util %"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_past_gqa32x8_1m.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_40_amd", "csrc", "attn_bf16.hip")


def useful_flops(w) -> float:
    """4 * head_dim * attended keys, summed over every query row: a row in
    block j attends min(k-1, j) full past blocks plus its own block up to
    itself (causal); every row attends min(k, n) full blocks (non-causal)."""
    B, n, D = w.block_size, w.num_blocks, w.head_dim
    k = min(w.topk, n)
    keys = 0
    for j in range(n):
        if w.causal:
            keys += B * min(k - 1, j) * B + B * (B + 1) // 2
        else:
            keys += B * k * B
    return 4.0 * D * keys * w.batch * w.num_q_heads


def measure(M, W, w, steps, warmup, log):
    import torch
    dev = "cuda"
    t0 = time.perf_counter()
    q, k, v, _ = W.make_inputs(w, device=dev)
    out = torch.empty_like(q)
    sel = torch.empty((w.batch, w.num_q_heads, w.seqlen, w.topk), dtype=torch.int32, device=dev)
    nbytes = M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim,
                               M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32, w.block_size, w.topk, w.causal)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs ready in {time.perf_counter() - t0:.1f}s, workspace {nbytes / 2**30:.2f} GiB")
    for i in range(warmup):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws)
        torch.cuda.synchronize()
        log(f"[bench] {w.name}: warmup {i + 1}/{warmup} done")
    M.profile_read()  # drop anything recorded earlier
    M.profile_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    M.profile_enable(False)
    stages = M.profile_read()
    log(f"[bench] {w.name}: {steps} steps in {elapsed:.3f}s")
    ms = elapsed / steps * 1e3
    fl = useful_flops(w)
    attn_ms = (stages["attn_past"]["ms"] + stages["attn_own"]["ms"] + stages["attn_f32"]["ms"]) / steps
    attn_fl = (stages["attn_past"]["work"] + stages["attn_own"]["work"] + stages["attn_f32"]["work"]) / steps
    res = {
        "workload": w.name,
        "ms_per_step": ms,
        "useful_tflops": fl / (ms * 1e-3) / 1e12,
        "tokens_per_s": w.batch * w.seqlen / (ms * 1e-3),
        "attention_ms": attn_ms,
        "attention_tflops": attn_fl / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None,
        "mfma_util_attention": attn_fl / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if attn_ms > 0 else None,
        "stages": {name: {"ms_per_step": s["ms"] / steps, "launches_per_step": s["launches"] / steps,
                          "work_per_step": s["work"] / steps,
                          ("tflops" if name.startswith("attn") else "gbs"):
                              (s["work"] / (s["ms"] * 1e-3) / (1e12 if name.startswith("attn") else 1e9)
                               if s["ms"] > 0 else None)}
                   for name, s in stages.items() if s["launches"]},
        "useful_flops_per_step": fl,
    }
    # the library's own work accounting must agree with the closed form
    if abs(attn_fl - fl) > 1e-6 * fl:
        raise RuntimeError(f"useful FLOP accounting mismatch: library {attn_fl:.6e} vs closed form {fl:.6e}")
    inputs = (q, k, v, out, sel)
    return res, inputs, stages


def roofline(stages, steps):
    past = stages["attn_past"]
    if not past["launches"]:
        return None
    avg_ms = past["ms"] / past["launches"]
    flops_per_launch = past["work"] / past["launches"]
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        src_hash = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") == src_hash:
            traffic = rec.get("hbm_bytes_per_launch")
    return {"kernel": "attn_past_kernel", "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
            "avg_launch_ms": avg_ms, "launches_per_step": past["launches"] / steps,
            "flops_per_launch": flops_per_launch}


def cpu_baseline(W, w, inputs, budget_s, log):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    block means over all of K, then seeded query rows until the budget is used."""
    import numpy as np
    import torch
    import oracle.moba_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    q, k, v, _, _ = inputs
    t0 = time.perf_counter()
    k32 = k.detach().cpu().to(torch.float32).numpy()
    v32 = v.detach().cpu().to(torch.float32).numpy()
    qh = q.detach().cpu()
    t_copy = time.perf_counter() - t0
    log(f"[cpu] host copies {t_copy:.1f}s")
    t0 = time.perf_counter()
    mu = O.block_means(k32, w.block_size)
    t_mu = time.perf_counter() - t0
    log(f"[cpu] block means {t_mu:.1f}s")

    class Rows:
        shape, ndim = tuple(qh.shape), qh.ndim

        def __getitem__(self, idx):
            return qh[idx].to(torch.float64).numpy()

    rows = W.sample_rows(w, 256, seed=99)
    rng = np.random.default_rng(99)
    rng.shuffle(rows)
    done, keys, t_rows = 0, 0, 0.0
    D, B = w.head_dim, w.block_size
    # rows grouped per KV head inside moba_rows: feed small batches
    batch = 16
    while done < len(rows) and t_rows < budget_s:
        chunk = rows[done:done + batch]
        t0 = time.perf_counter()
        O.moba_rows(Rows(), k32, v32, B, w.topk, w.causal, chunk, mu=mu)
        t_rows += time.perf_counter() - t0
        for (_, t, _) in chunk:
            j = t // B
            keys += min(w.topk - 1, j) * B + (t - j * B + 1)
        done += len(chunk)
    fl = 4.0 * D * keys
    total_rows = w.batch * w.seqlen * w.num_q_heads
    log(f"[cpu] {done} rows in {t_rows:.1f}s")
    return {"value": fl / t_rows / 1e12, "unit": "TFLOP/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle: block means over all of K ({t_mu:.1f}s) plus {done} seeded query rows "
                      f"of the {w.name} workload ({t_rows:.1f}s); value = useful FLOPs of those rows / their time",
            "host_cpus_available": cores, "rows": done, "rows_seconds": t_rows, "block_means_seconds": t_mu,
            "tokens_per_s_equiv": done / w.num_q_heads / t_rows,
            "extrapolated_full_seconds": t_mu + t_rows / done * total_rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="gqa32x8_1m")
    ap.add_argument("--secondary", default="mha32_32k_needle", help="second workload ('' to skip)")
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: this build has no multi-GPU path "
                  "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import block_sparse_attention_40_amd as M
    import moba_workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w = W.WORKLOADS[args.workload]
    res, inputs, stages = measure(M, W, w, args.steps, args.warmup, log)
    line = {
        "metric": METRIC,
        "value": res["useful_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), bf16-rounded; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "topk": w.topk, "causal": w.causal, "parallelism": "none (1 GPU)"},
        "tokens_per_s": res["tokens_per_s"],
        "attention_tflops": res["attention_tflops"],
        "mfma_util_attention": res["mfma_util_attention"],
        "stages": res["stages"],
        "roofline": roofline(stages, args.steps),
    }
    if args.secondary:
        w2 = W.WORKLOADS[args.secondary]
        res2, inputs2, _ = measure(M, W, w2, args.secondary_steps, max(args.warmup, 3), log)
        del inputs2
        line["secondary"] = res2
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W, w, inputs, args.cpu_seconds, log)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
