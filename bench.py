#!/usr/bin/env python3
"""Benchmark of the MoBA prefill forward on one MI355X.

One step = one moba_attn_fwd call (block means, gate + top-k, dispatch,
past-block attention, own-block attention + merge) over the whole workload,
inputs resident in HBM.  Prints one JSON line.

Headline workload: 1M tokens, Llama-3.1-8B-shaped grouped-query attention
(32 query / 8 KV heads, head dim 128), block 4096, top-12, bf16.  The 32K
workload (32 heads, block 512, top-3, planted needles) is measured in the same
run and reported under "secondary", launched eagerly and, under "graph", as
replays of the same call captured once into a HIP graph.
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
# the past-block attention kernel the 1M workload runs (384-row tiles fed from the K/V slice images)
PAST_KERNEL = "moba::attn_past_img_kernel<12>"
PAST_TAG = "attn_past"


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


def graph_replay(M, w, q, k, v, out, sel, ws, steps, gate, log):
    """The same forward captured once into a HIP graph (torch.cuda.CUDAGraph)
    and replayed `steps` times: the step time without the host's per-kernel
    launch cost.  The first replay's output must equal the eager output bit
    for bit (the kernels are deterministic)."""
    import torch
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws, gate=gate)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws, gate=gate)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("graph replay output differs from the eager forward")
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    log(f"[bench] {w.name}: {steps} graph replays, {ms:.3f} ms each")
    del g
    return ms


def measure(M, W, w, steps, warmup, log, gate="mean", graph=False, max_chunk_blocks=0):
    import torch
    dev = "cuda"
    t0 = time.perf_counter()
    q, k, v, _ = W.make_inputs(w, device=dev)
    out = torch.empty_like(q)
    sel = torch.empty((w.batch, w.num_q_heads, w.seqlen, w.topk), dtype=torch.int32, device=dev)
    nbytes = M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim,
                               M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32, w.block_size, w.topk, w.causal,
                               max_chunk_blocks=max_chunk_blocks)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs ready in {time.perf_counter() - t0:.1f}s, workspace {nbytes / 2**30:.2f} GiB")
    for i in range(warmup):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws, gate=gate)
        torch.cuda.synchronize()
        log(f"[bench] {w.name}: warmup {i + 1}/{warmup} done")
    M.profile_read()  # drop anything recorded earlier
    M.profile_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws, gate=gate)
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
        "gate": gate,
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
    if graph:
        gms = graph_replay(M, w, q, k, v, out, sel, ws, steps, gate, log)
        res["graph"] = {"ms_per_step": gms, "useful_tflops": fl / (gms * 1e-3) / 1e12,
                        "tokens_per_s": w.batch * w.seqlen / (gms * 1e-3)}
    inputs = (q, k, v, out, sel)
    return res, inputs, stages


def past_kernel_name(M, w):
    """The past-block kernel the forward launches on workload w, from its
    plan: 384-row tiles over the slice images, 256-row tiles through
    registers, or 128-row tiles (straight from K and V rows when the block is
    a multiple of 32 keys)."""
    dt = M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32
    nbytes = M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt, w.block_size,
                               w.topk, w.causal)
    plan = M.plan_info(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt, w.block_size, w.topk,
                       w.causal, nbytes)
    if plan["tile_rows"] == 384:
        return PAST_KERNEL
    if plan["tile_rows"] == 256:
        return "moba::attn_past_kernel<8>"
    return "moba::attn_past_rows_kernel<4, 3, 1>" if w.block_size % 32 == 0 else "moba::attn_past_kernel<4>"


def roofline(stages, steps, kernel=PAST_KERNEL, workload="gqa32x8_1m"):
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
        if (rec.get("kernel_source_sha256") == src_hash and rec.get("kernel") == kernel
                and rec.get("workload") == workload):
            traffic = rec.get("hbm_bytes_per_launch")
    return {"kernel": kernel, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
            "avg_launch_ms": avg_ms, "launches_per_step": past["launches"] / steps,
            "flops_per_launch": flops_per_launch}


def cpu_baseline(W, w, inputs, budget_s, log, per_call=64, gate="mean"):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    block summaries (means, or min / max) over all of K, then seeded query rows
    until the budget is used."""
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
    mu = O.block_means(k32, w.block_size) if gate == "mean" else None
    mm = O.block_minmax(k32, w.block_size) if gate == "minmax" else None
    t_mu = time.perf_counter() - t0
    log(f"[cpu] block summaries ({gate}) {t_mu:.1f}s")

    class Rows:
        shape, ndim = tuple(qh.shape), qh.ndim

        def __getitem__(self, idx):
            return qh[idx].to(torch.float64).numpy()

    # the oracle converts one KV head's K and V to fp64 per call: feed it
    # batches of rows that share a KV head, heads in turn
    rows = W.sample_rows(w, 256, seed=99)
    g = w.num_q_heads // w.num_kv_heads
    rng = np.random.default_rng(99)
    groups = {}
    for r in rows:
        groups.setdefault((r[0], r[2] // g), []).append(r)
    per_head = []
    for key in sorted(groups):
        grp = groups[key]
        rng.shuffle(grp)
        per_head.append([grp[i:i + per_call] for i in range(0, len(grp), per_call)])
    batches = [hb[i] for i in range(max(len(hb) for hb in per_head)) for hb in per_head if i < len(hb)]
    done, keys, t_rows, calls = 0, 0, 0.0, 0
    D, B = w.head_dim, w.block_size
    for chunk in batches:
        if t_rows >= budget_s:
            break
        t0 = time.perf_counter()
        O.moba_rows(Rows(), k32, v32, B, w.topk, w.causal, chunk, mu=mu, gate=gate, minmax=mm)
        t_rows += time.perf_counter() - t0
        calls += 1
        for (_, t, _) in chunk:
            j = t // B
            keys += min(w.topk - 1, j) * B + (t - j * B + 1)
        done += len(chunk)
        log(f"[cpu] {done} rows, {t_rows:.1f}s")
    fl = 4.0 * D * keys
    total_rows = w.batch * w.seqlen * w.num_q_heads
    log(f"[cpu] {done} rows in {t_rows:.1f}s")
    return {"value": fl / t_rows / 1e12, "unit": "TFLOP/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle: block {'means' if gate == 'mean' else 'min / max'} over all of K "
                      f"({t_mu:.1f}s) plus {done} seeded query rows "
                      f"of the {w.name} workload in {calls} calls of up to {per_call} rows sharing a KV head "
                      f"({t_rows:.1f}s, per-head fp64 conversion included); value = useful FLOPs of those rows "
                      f"/ their time",
            "host_cpus_available": cores, "rows": done, "rows_seconds": t_rows, "block_means_seconds": t_mu,
            "tokens_per_s_equiv": done / w.num_q_heads / t_rows,
            "extrapolated_full_seconds": t_mu + t_rows / done * total_rows}


# ---------------------------------------------------------------------------
# Profile evidence: the commands whose output the committed summaries under
# profiles/ come from, and the converters that write those summaries.
# ---------------------------------------------------------------------------
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace_1m -o run -- "
             "python3 -u bench.py --steps 3 --warmup 1 --secondary '' --no-cpu-baseline > gpurun_out/trace_1m.json")
PMC_CMD = ("rocprofv3 --pmc {counter} --output-format csv -d gpurun_out/pmc_{counter} -o run -- "
           "python3 -u bench.py --steps 1 --warmup 0 --secondary '' --no-cpu-baseline --copy-calibration 1024 "
           "> gpurun_out/pmc_{counter}.json")
COPY_KERNEL_TAG = "neg_kernel"   # torch.neg(src, out=dst): reads and writes the buffer once


def copy_calibration(mib, log):
    """A plain elementwise copy (negation) of `mib` MiB, three times: the
    reference dispatch that scales the HBM byte counters."""
    import torch
    n = mib * 2 ** 20 // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 x {mib} MiB")
    del src, dst


def _per_dispatch(d, counter):
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    key = (r["Kernel_Name"], r["Dispatch_Id"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (name, _), v in vals.items():
        by_kernel.setdefault(name, []).append(v)
    return by_kernel


def summarize_traffic(fetch_dir, write_dir, calib_mib, out_path):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the past-block kernel,
    each scaled by what the same counter reads for the calibration copy."""
    calib_kib = calib_mib * 1024.0
    res = {"kernel": PAST_KERNEL, "workload": "gqa32x8_1m",
           "kernel_source_sha256": hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest(),
           "commands": [PMC_CMD.format(counter="FETCH_SIZE"), PMC_CMD.format(counter="WRITE_SIZE")],
           "calibration": {"kernel": "torch.neg (elementwise copy)", "bytes_read": calib_kib * 1024,
                           "bytes_written": calib_kib * 1024}}
    total = 0.0
    for counter, d, field in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        per = _per_dispatch(d, counter)
        cal = [v for name, vs in per.items() if COPY_KERNEL_TAG in name for v in vs]
        past = [v for name, vs in per.items() if PAST_TAG in name for v in vs]
        if not cal or not past:
            raise RuntimeError(f"{counter}: calibration or past-kernel dispatches missing in {d}")
        cal_kib = sum(cal) / len(cal)
        factor = calib_kib / cal_kib
        kib = sum(past) / len(past)
        res["calibration"][f"{counter}_kib"] = cal_kib
        res["calibration"][f"{field}_factor"] = factor
        res[f"{field}_kib_per_launch_raw"] = kib
        res[f"{field}_bytes_per_launch"] = kib * factor * 1024
        res["launches"] = len(past)
        total += kib * factor * 1024
    res["hbm_bytes_per_launch"] = total
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    return res


MFMA_CMD = ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
            "-d gpurun_out/pmc_mfma -o run -- python3 -u bench.py --steps 1 --warmup 0 --secondary '' "
            "--no-cpu-baseline --no-gemm-reference > gpurun_out/pmc_mfma.json")
# the same three counter runs on the 32K workload (two untimed calls first)
PMC32_CMD = ("rocprofv3 --pmc {counters} --output-format csv -d gpurun_out/pmc32k_{tag} -o run -- "
             "python3 -u bench.py --workload mha32_32k_needle --steps 1 --warmup 2 --secondary '' "
             "--no-cpu-baseline --no-gemm-reference --copy-calibration 1024 > gpurun_out/pmc32k_{tag}.json")
# VALU counters (the gate's bound, the attention kernels' co-issue)
VALU_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES "
                 "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_LDS SQ_WAIT_INST_ANY SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
VALU_CMD = ("rocprofv3 --pmc " + VALU_COUNTERS + " --output-format csv -d gpurun_out/pmc_valu -o run -- "
            "python3 -u bench.py --steps 1 --warmup 0 --secondary '' --no-cpu-baseline --no-gemm-reference "
            "> gpurun_out/pmc_valu.json")
# the backward on its benchmark configuration (a training step: the forward
# with lse, then the backward)
BWD_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace_bwd -o run -- "
                 "python3 -u bench.py --backward gqa32x8_128k --steps 3 --warmup 1 > gpurun_out/trace_bwd.json")
BWD_PMC_CMD = ("rocprofv3 --pmc {counters} --output-format csv -d gpurun_out/pmcbwd_{tag} -o run -- "
               "python3 -u bench.py --backward gqa32x8_128k --steps 1 --warmup 0 > gpurun_out/pmcbwd_{tag}.json")
PROFILE_CMDS = {
    "gqa32x8_1m": {"title": "gqa32x8_1m workload (1M tokens, 32/8 heads, D 128, block 4096, top-12)",
                   "fetch": PMC_CMD.format(counter="FETCH_SIZE"), "write": PMC_CMD.format(counter="WRITE_SIZE"),
                   "mfma": MFMA_CMD, "valu": VALU_CMD},
    "mha32_32k_needle": {"title": "mha32_32k_needle workload (32K tokens, 32 heads, D 128, block 512, top-3)",
                         "fetch": PMC32_CMD.format(counters="FETCH_SIZE", tag="FETCH_SIZE"),
                         "write": PMC32_CMD.format(counters="WRITE_SIZE", tag="WRITE_SIZE"),
                         "mfma": PMC32_CMD.format(counters="SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
                                                  tag="mfma"),
                         "valu": PMC32_CMD.format(counters=VALU_COUNTERS, tag="valu")},
    "bwd_gqa32x8_128k": {"title": "gqa32x8_128k workload (128K tokens, 32/8 heads, D 128, block 4096, top-12)",
                         "pass": "training step (forward with lse, then backward)",
                         "calls": "forward-with-lse and backward calls",
                         "mfma": BWD_PMC_CMD.format(counters="SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
                                                    tag="mfma"),
                         "valu": BWD_PMC_CMD.format(counters=VALU_COUNTERS, tag="valu")},
}


def _workload_of(bench_json):
    """The profile key of a bench.py run: its workload, prefixed with bwd_ for
    a --backward run."""
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    wl = line["config"]["workload"]
    return "bwd_" + wl if "backward" in line["metric"] else wl


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _agent_info(d):
    import csv
    import glob
    for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Name", "").startswith("gfx"):
                    return r
    raise RuntimeError(f"no GPU agent in {d}")


def _short(name):
    n = name.replace("void ", "")
    return n.split("(")[0]


def summarize_mfma(pmc_dir, bench_json):
    """MFMA-busy fraction per kernel from SQ_VALU_MFMA_BUSY_CYCLES (summed over
    every SIMD) against GRBM_GUI_ACTIVE (summed over the XCDs): busy =
    MFMA cycles / (GPU cycles per XCD x SIMDs); the clock the kernels ran at =
    GPU cycles per XCD / kernel time."""
    info = _agent_info(pmc_dir)
    simds, xcc = int(info["Simd_Count"]), int(info["Num_Xcc"])
    wl = _workload_of(bench_json)
    cmds = PROFILE_CMDS[wl]
    out_path = os.path.join(ROOT, "profiles", f"mfma_busy_{wl}.md")
    per = {}
    for r in _counter_rows(pmc_dir):
        k = _short(r["Kernel_Name"])
        if not k.startswith("moba::"):
            continue
        d = per.setdefault(k, {"disp": set(), "t": {}})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["disp"].add(r["Dispatch_Id"])
        d["t"][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = [f"# MFMA busy: MoBA {cmds.get('pass', 'forward')}, {cmds['title']}",
           "", "Command (run from the repository root on one MI355X):", "", "```", cmds["mfma"], "```", "",
           f"Counters summed over the dispatches of the run's {cmds.get('calls', 'forward calls')}; {simds} SIMDs, "
           f"{xcc} XCDs. "
           "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs); clock = "
           "(GRBM_GUI_ACTIVE / XCDs) / kernel time.", "",
           "| Kernel | Dispatches | Kernel ms (sum) | MFMA busy | Clock GHz |", "|---|---|---|---|---|"]
    res = {}
    for k, d in sorted(per.items(), key=lambda x: -sum(x[1]["t"].values())):
        if d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) <= 0:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / xcc
        t = sum(d["t"].values())
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)
        res[k] = {"busy": busy, "clock_ghz": cyc / t / 1e9, "ms": t * 1e3}
        out.append(f"| {k} | {len(d['disp'])} | {t * 1e3:.2f} | {100 * busy:.1f} % | {cyc / t / 1e9:.2f} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    return res


def summarize_valu(pmc_dir, bench_json):
    """Per kernel, from one counter run: VALU and MFMA instructions per wave-
    instruction slot, the VALU issue fraction (VALU instructions x 4 cycles,
    a wave64 VALU instruction's issue time, over the SIMD cycles), the MFMA-
    busy fraction, the fraction of MFMA-busy cycles in which a VALU
    instruction was issued beside it (co-issue), and the wave-cycles spent
    waiting to issue."""
    info = _agent_info(pmc_dir)
    simds, xcc = int(info["Simd_Count"]), int(info["Num_Xcc"])
    wl = _workload_of(bench_json)
    cmds = PROFILE_CMDS[wl]
    out_path = os.path.join(ROOT, "profiles", f"valu_{wl}.md")
    per = {}
    for r in _counter_rows(pmc_dir):
        k = _short(r["Kernel_Name"])
        if not k.startswith("moba::"):
            continue
        d = per.setdefault(k, {"disp": set(), "t": {}})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["disp"].add(r["Dispatch_Id"])
        d["t"][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = [f"# VALU and MFMA issue: MoBA {cmds.get('pass', 'forward')}, {cmds['title']}",
           "", "Command (run from the repository root on one MI355X):", "", "```", cmds["valu"], "```", "",
           f"Counters summed over the dispatches of the run's {cmds.get('calls', 'forward calls')}; {simds} SIMDs, "
           f"{xcc} XCDs; SIMD cycles "
           "= GRBM_GUI_ACTIVE / XCDs x SIMDs.  VALU issue = SQ_INSTS_VALU x 4 / SIMD cycles (a wave64 VALU "
           "instruction issues over 4 cycles); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD cycles; co-issue = "
           "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; VALU per MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) "
           "/ SQ_INSTS_MFMA (SQ_INSTS_VALU counts the MFMA instructions too).", "",
           "| Kernel | Dispatches | Kernel ms (sum) | VALU issue | MFMA busy | co-issue | VALU per MFMA | "
           "LDS per MFMA |", "|---|---|---|---|---|---|---|---|"]
    res = {}
    for k, d in sorted(per.items(), key=lambda x: -sum(x[1]["t"].values())):
        if d.get("GRBM_GUI_ACTIVE", 0.0) <= 0:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / xcc * simds
        t = sum(d["t"].values())
        valu = d.get("SQ_INSTS_VALU", 0.0)
        mfma = d.get("SQ_INSTS_MFMA", 0.0)
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        r = {"valu_issue": valu * 4 / cyc, "mfma_busy": busy / cyc,
             "coissue": d.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / busy if busy else None,
             "valu_per_mfma": (valu - mfma) / mfma if mfma else None,
             "lds_per_mfma": d.get("SQ_INSTS_LDS", 0.0) / mfma if mfma else None, "ms": t * 1e3}
        res[k] = r
        f = lambda x, pct=True: "-" if x is None else (f"{100 * x:.1f} %" if pct else f"{x:.2f}")
        out.append(f"| {k} | {len(d['disp'])} | {t * 1e3:.2f} | {f(r['valu_issue'])} | {f(r['mfma_busy'])} | "
                   f"{f(r['coissue'])} | {f(r['valu_per_mfma'], False)} | {f(r['lds_per_mfma'], False)} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    return res


def summarize_stage_hbm(fetch_dir, write_dir, calib_mib, bench_json):
    """HBM bytes per dispatch of every MoBA kernel from FETCH_SIZE and
    WRITE_SIZE (scaled by the calibration copy, as for the past-block kernel),
    over the dispatch time in the same counter run, beside the bytes the stage
    must move (bench.py's own accounting, HIP-event time)."""
    calib_kib = calib_mib * 1024.0
    wl = _workload_of(bench_json)
    cmds = PROFILE_CMDS[wl]
    out_path = os.path.join(ROOT, "profiles", f"hbm_stages_{wl}.md")
    byk = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        cal = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL_TAG in r["Kernel_Name"]]
        if not cal:
            raise RuntimeError(f"{counter}: calibration dispatch missing in {d}")
        factor = calib_kib / (sum(cal) / len(cal))
        for r in rows:
            k = _short(r["Kernel_Name"])
            if not k.startswith("moba::"):
                continue
            e = byk.setdefault(k, {"FETCH_SIZE": [], "WRITE_SIZE": [], "t": []})
            e[counter].append(float(r["Counter_Value"]) * factor * 1024)
            if counter == "FETCH_SIZE":
                e["t"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    st = line["stages"]
    out = [f"# HBM traffic per kernel: MoBA forward, {cmds['title']}",
           "", "Commands (run from the repository root on one MI355X):", "", "```",
           cmds["fetch"], cmds["write"], "```", "",
           f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what each reads for a {calib_mib} MiB "
           "elementwise copy in the same run; time = dispatch time in the FETCH_SIZE run. Peak 8000 GB/s.", "",
           "| Kernel | Dispatches | HBM read GB | HBM write GB | ms | GB/s | % of peak |",
           "|---|---|---|---|---|---|---|"]
    res = {}
    for k, e in sorted(byk.items(), key=lambda x: -sum(x[1]["t"])):
        n = len(e["t"])
        rd = sum(e["FETCH_SIZE"]) / max(1, len(e["FETCH_SIZE"]))
        wr = sum(e["WRITE_SIZE"]) / max(1, len(e["WRITE_SIZE"]))
        t = sum(e["t"]) / n
        gbs = (rd + wr) / t / 1e9
        res[k] = {"read": rd, "write": wr, "ms": t * 1e3, "gbs": gbs}
        out.append(f"| {k} | {n} | {rd / 1e9:.3f} | {wr / 1e9:.3f} | {t * 1e3:.3f} | {gbs:.0f} | "
                   f"{100 * gbs / PEAK_HBM_GBS:.1f} % |")
    # the bytes each stage must move (bench.py's accounting of the same call)
    # over its kernels' time in this run
    kernels_of = {"meanpool": ("moba::meanpool_kernel", "moba::mu_split_kernel"),
                  "gate": ("moba::gate_mfma_kernel",),
                  "dispatch": ("moba::scatter_kernel", "moba::tile_plan_kernel", "moba::list_scan_kernel"),
                  "kv_layout": ("moba::kv_image_kernel",)}
    out += ["", "Per stage, the bytes it must move (bench.py's accounting of the same call) over its kernels' time "
            "in this run:", "",
            "| Stage | kernels | algorithmic GB per call | ms per call | GB/s | % of peak |", "|---|---|---|---|---|---|"]
    line_w = json.loads(open(bench_json).read().strip().splitlines()[-1])
    calls = line_w["steps"] + line_w["warmup"]
    for name, ks in kernels_of.items():
        if name not in st:
            continue
        t = sum(sum(e["t"]) for k, e in byk.items() if k.startswith(ks)) / calls
        if t <= 0:
            continue
        gb = st[name]["work_per_step"]
        out.append(f"| {name} | {', '.join(k.split('::')[1] for k in ks)} | {gb / 1e9:.3f} | {t * 1e3:.3f} | "
                   f"{gb / t / 1e9:.0f} | {100 * gb / t / 1e9 / PEAK_HBM_GBS:.1f} % |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    return res


DECODE_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace_decode -o run -- "
                    "python3 -u bench.py --decode --decode-skip-dense --steps 20 --warmup 3 --no-cpu-baseline "
                    "> gpurun_out/trace_decode.json")


def summarize_decode_trace(trace_dir, bench_json, out_path):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of
    bench.py --decode, with bench.py's own HIP-event average for the decode
    attention kernel."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    m = line["moba"]
    cfg = line["config"]
    out = [f"# Kernel trace: MoBA decode, {cfg['workload']} workload ({cfg['batch']} sequences of up to "
           f"{cfg['max_len']} cached positions, {cfg['num_q_heads']}/{cfg['num_kv_heads']} heads, D {cfg['head_dim']}, "
           f"block {cfg['block_size']}, top-{cfg['topk']})",
           "", "Command (run from the repository root on one MI355X):", "", "```", DECODE_TRACE_CMD, "```", "",
           f"{line['warmup'] + line['steps']} decode calls ({line['warmup']} untimed + {line['steps']} timed).",
           "", "| Kernel | Calls | Total ns | Average ns | % | Min ns | Max ns |", "|---|---|---|---|---|---|---|"]
    for r in rows[:12]:
        name = r["Name"] if len(r["Name"]) < 72 else r["Name"][:69] + "..."
        out.append(f"| {name} | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
                   f"{float(r['Percentage']):.2f} | {r['MinNs']} | {r['MaxNs']} |")
    att = [r for r in rows if "decode_attn_kernel" in r["Name"]][0]
    by = m["bytes_per_step"]
    out += ["", f"bench.py in the same run, HIP events around each decode attention launch on its stream: average "
                f"{m['attn_kernel_ms']:.3f} ms (rocprofv3: {float(att['AverageNs']) / 1e6:.3f} ms); algorithmic bytes "
                f"{by['attn_kernel'] / 1e9:.3f} GB per launch (the chosen blocks' K and V, each block read once per "
                f"KV-head group, plus queries and partials) = {m['attn_kernel_gbs']:.0f} GB/s, "
                f"{100 * line['roofline']['frac']:.1f}% of the 8000 GB/s HBM peak.",
            f"Step: {line['ms_per_step']:.3f} ms, {line['value']:.0f} sequences decoded per second."]
    with open(out_path, "w") as fh:
        fh.write("\n".join(out) + "\n")


def summarize_trace(trace_dir, bench_json, out_path):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of bench.py,
    with bench.py's own HIP-event average for the past-block kernel."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    rf = line["roofline"]
    out = ["# Kernel trace: MoBA forward, gqa32x8_1m workload (1M tokens, 32/8 heads, D 128, block 4096, top-12)",
           "", "Command (run from the repository root on one MI355X):", "", "```", TRACE_CMD, "```", "",
           f"{line['warmup'] + line['steps']} forward calls ({line['warmup']} warm-up + {line['steps']} timed); "
           f"{rf['launches_per_step']:.0f} query chunks per call.", "",
           "| Kernel | Calls | Total ns | Average ns | % | Min ns | Max ns |", "|---|---|---|---|---|---|---|"]
    for r in rows[:12]:
        name = r["Name"] if len(r["Name"]) < 72 else r["Name"][:69] + "..."
        out.append(f"| {name} | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
                   f"{float(r['Percentage']):.2f} | {r['MinNs']} | {r['MaxNs']} |")
    past = [r for r in rows if PAST_TAG in r["Name"]][0]
    out += ["", f"bench.py in the same run, HIP events around each {PAST_KERNEL} launch on its stream: "
                f"average {rf['avg_launch_ms']:.2f} ms per launch (rocprofv3: {float(past['AverageNs']) / 1e6:.2f} ms); "
                f"{rf['achieved']:.1f} TFLOP/s = {100 * rf['frac']:.1f}% of the {rf['peak']:.0f} TFLOP/s bf16 peak.",
            f"Step: {line['ms_per_step']:.1f} ms, {line['value']:.1f} useful TFLOP/s."]
    with open(out_path, "w") as fh:
        fh.write("\n".join(out) + "\n")


def summarize_bwd_trace(trace_dir, bench_json, out_path):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of
    bench.py --backward, with bench.py's own HIP-event averages for the two
    gradient kernels."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    cmds = PROFILE_CMDS[_workload_of(bench_json)]
    out = [f"# Kernel trace: MoBA {cmds['pass']}, {cmds['title']}",
           "", "Command (run from the repository root on one MI355X):", "", "```", BWD_TRACE_CMD, "```", "",
           f"One untimed forward-with-lse and {line['warmup']} untimed backward calls, then {line['steps']} timed "
           f"forward-with-lse and {line['steps']} timed backward calls.", "",
           "| Kernel | Calls | Total ns | Average ns | % | Min ns | Max ns |", "|---|---|---|---|---|---|---|"]
    for r in rows[:14]:
        name = r["Name"] if len(r["Name"]) < 72 else r["Name"][:69] + "..."
        out.append(f"| {name} | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
                   f"{float(r['Percentage']):.2f} | {r['MinNs']} | {r['MaxNs']} |")
    out.append("")
    # the stages bench.py times and the kernels each one launches (the dq
    # stage of a query chunk: its past-block and own-block tiles, then the
    # merge of a row's contributions)
    stages = (("bwd_dkdv", ("bwd_dkdv_kernel",), 8),
              ("bwd_dq", ("bwd_dq_kernel<false>", "bwd_dq_kernel<true>", "bwd_dq_merge_kernel"), 6))
    for stage, tags, per_key in stages:
        st = line["stages"][stage]
        prof = [r for r in rows if any(t in r["Name"] for t in tags)]
        per_launch = sum(float(r["TotalDurationNs"]) for r in prof) / int(prof[0]["Calls"]) / 1e6
        out.append(f"bench.py in the same run, HIP events around each {stage} stage ({', '.join(tags)}): average "
                   f"{st['ms'] / st['launches']:.2f} ms per launch (rocprofv3, the same kernels: {per_launch:.2f} "
                   f"ms); {st['tflops']:.0f} TFLOP/s ({per_key}·D FLOP per attended key) = "
                   f"{100 * st['tflops'] / PEAK_BF16_TFLOPS:.1f}% of the {PEAK_BF16_TFLOPS:.0f} TFLOP/s bf16 peak.")
    out.append(f"Backward: {line['ms_per_step']:.1f} ms, {line['value']:.0f} useful TFLOP/s (10·D per attended key); "
               f"training step (forward with lse + backward): {line['train_step_ms']:.1f} ms.")
    with open(out_path, "w") as fh:
        fh.write("\n".join(out) + "\n")


def curve(M, W, lengths, log, budget_s=4.0, moba_only=False):
    """Speedup of MoBA over dense causal attention, both from this library
    (report §4.5: the attention layer forward only, MoBA with the block count
    and top-k fixed, n = 256 blocks and top-12, so the block size grows with
    the sequence; dense = block_size = seqlen, topk = 1: one causal block).
    One JSON line per length; steps adapt to about budget_s of GPU time.
    moba_only: skip the dense side (10M positions: about 13 minutes of dense
    attention), and when one call exceeds the budget, time a single call
    after one untimed call."""
    import torch
    out_lines = []
    for S in lengths:
        res = {"seqlen": S}
        sides = (("moba", W.Workload(f"gqa32x8_{S}_moba", "bf16", 1, 32, 8, S, 128, S // 256, 12, seed=1100)),
                 ("dense", W.Workload(f"gqa32x8_{S}_dense", "bf16", 1, 32, 8, S, 128, S, 1, seed=1100)))
        for tag, w in sides[:1 if moba_only else 2]:
            t_in = time.perf_counter()
            q, k, v, _ = W.make_inputs(w, device="cuda")
            log(f"[curve] S={S} {tag}: inputs in {time.perf_counter() - t_in:.1f}s")
            out = torch.empty_like(q)
            nbytes = M.workspace_bytes(1, S, 32, 8, 128, M.DTYPE_BF16, w.block_size, w.topk, True)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            call = lambda: M.moba_attn_fwd(q, k, v, w.block_size, w.topk, True, out=out, workspace=ws,
                                           return_sel=False)
            t0 = time.perf_counter()
            call()
            torch.cuda.synchronize()
            log(f"[curve] S={S} {tag}: untimed call {time.perf_counter() - t0:.1f}s")
            one = 0.0
            if not moba_only:
                t0 = time.perf_counter()
                call()
                torch.cuda.synchronize()
                one = time.perf_counter() - t0
            steps = max(1, min(20, int(budget_s / max(one, 1e-6)))) if one > 0 else 1
            M.profile_read()
            M.profile_enable(True)
            t0 = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) / steps * 1e3
            M.profile_enable(False)
            st = M.profile_read()
            fl = useful_flops(w)
            res[tag] = {"block_size": w.block_size, "topk": w.topk, "ms": ms, "steps": steps,
                        "useful_tflops": fl / (ms * 1e-3) / 1e12,
                        "stages_ms": {n: x["ms"] / steps for n, x in st.items() if x["launches"]}}
            log(f"[curve] S={S} {tag}: {ms:.3f} ms ({steps} steps)")
            del q, k, v, out, ws
            torch.cuda.empty_cache()
        if not moba_only:
            res["speedup"] = res["dense"]["ms"] / res["moba"]["ms"]
        print(json.dumps(res), flush=True)
        out_lines.append(res)
    return out_lines


def granularity(M, W, log, budget_s=2.0):
    """Kernel speed across the block granularities of the report's ablation
    (§4.2, Figure 4): 32K positions at 75 % sparsity, n blocks choosing n / 4
    (8/2, 16/4, 32/8, 64/16, 128/32), on the 32K scaling-law layout (32 query
    heads = KV heads, D = 128, bf16).  One JSON line per shape.  The report
    compares model loss here; only speed is measured."""
    import torch
    S = 32768
    lines = []
    for n in (8, 16, 32, 64, 128):
        w = W.Workload(f"mha32_32k_n{n}_k{n // 4}", "bf16", 1, 32, 32, S, 128, S // n, n // 4, seed=1200 + n)
        q, k, v, _ = W.make_inputs(w, device="cuda")
        out = torch.empty_like(q)
        ws = torch.empty(M.workspace_bytes(1, S, 32, 32, 128, M.DTYPE_BF16, w.block_size, w.topk, True),
                         dtype=torch.uint8, device="cuda")
        call = lambda: M.moba_attn_fwd(q, k, v, w.block_size, w.topk, True, out=out, workspace=ws,
                                       return_sel=False)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        steps = max(3, min(200, int(budget_s / max(time.perf_counter() - t0, 1e-6))))
        M.profile_read()
        M.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        M.profile_enable(False)
        st = M.profile_read()
        fl = useful_flops(w)
        res = {"seqlen": S, "blocks": n, "topk": n // 4, "block_size": w.block_size, "ms": ms, "steps": steps,
               "useful_tflops": fl / (ms * 1e-3) / 1e12, "tokens_per_s": S / (ms * 1e-3),
               "stages_ms": {k_: x["ms"] / steps for k_, x in st.items() if x["launches"]}}
        log(f"[granularity] {n}/{n // 4}: {ms:.3f} ms")
        print(json.dumps(res), flush=True)
        lines.append(res)
        del q, k, v, out, ws
        torch.cuda.empty_cache()
    return lines


def gemm_peak(log, sizes=(4096, 8192, 16384), emit=True):
    """The attainable dense bf16 rate on this GPU: torch.matmul (hipBLASLt)
    on square bf16 products."""
    import torch
    best = {}
    for n in sizes:
        a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
        b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        reps = max(3, int(2e14 / (2.0 * n ** 3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        tf = 2.0 * n ** 3 * reps / (time.perf_counter() - t0) / 1e12
        best[str(n)] = round(tf, 1)
        log(f"[gemm] {n}^3 bf16: {tf:.1f} TFLOP/s")
        del a, b
    if emit:
        print(json.dumps({"gemm_bf16_tflops": best, "peak_datasheet": PEAK_BF16_TFLOPS}), flush=True)
    return best


def decode_bytes(w, sel, lens, chunk):
    """Algorithmic HBM bytes of one decode step, from the step's own selection:
    per (sequence, KV head) the union of the group's chosen blocks is read once
    (K and V; the own block up to the new token), plus the queries, the gate's
    cached means of the complete past blocks, the output, and the attention
    kernel's partials (written once, read once by the merge)."""
    import numpy as np
    elt = 2 if w.dtype == "bf16" else 4
    B, D, g = w.block_size, w.head_dim, w.num_q_heads // w.num_kv_heads
    nchunk = -(-B // chunk)
    kv = gate = partial = 0
    for bb, L in enumerate(lens):
        j = (L - 1) // B
        for hk in range(w.num_kv_heads):
            blocks = set(int(i) for i in np.unique(sel[bb, hk * g:(hk + 1) * g]) if i >= 0)
            for i in blocks:
                keys = B if i < j else L - j * B
                kv += keys * D * elt * 2
            gate += j * D * 4
        for h in range(w.num_q_heads):
            for i in sel[bb, h]:
                if i < 0:
                    continue
                keys = B if i < j else L - j * B
                partial += -(-keys // chunk) * (D + 2) * 4
    qo = w.batch * w.num_q_heads * D * elt * 2
    return {"kv": kv, "gate": gate, "partials": partial, "q_out": qo,
            "attn_kernel": kv + partial + w.batch * w.num_q_heads * D * elt,
            "total": kv + gate + 2 * partial + qo, "nchunk": nchunk}


def measure_decode(M, W, w, steps, warmup, log, cpu_seconds=0.0, dense=True):
    """One decode step per call for every sequence of the batch (cache
    lengths fixed across steps), then the same caches decoded densely by this
    library (block_size = max_len, topk = 1: one causal block of L keys)."""
    import numpy as np
    import torch
    t0 = time.perf_counter()
    q, kc, vc, lens = W.make_decode_inputs(w, device="cuda")
    dt = M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32
    res = {"workload": w.name}
    for tag, B, k in (("moba", w.block_size, w.topk), ("dense", w.max_len, 1))[:2 if dense else 1]:
        mu = M.moba_decode_means(kc, lens, B)
        out = torch.empty_like(q)
        sel = torch.empty((w.batch, w.num_q_heads, k), dtype=torch.int32, device="cuda")
        ws = torch.empty(M.decode_workspace_bytes(w.batch, w.max_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                  dt, B, k), dtype=torch.uint8, device="cuda")
        call = lambda: M.moba_decode_fwd(q, kc, vc, mu, lens, B, k, out=out, sel_idx=sel, workspace=ws)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        log(f"[decode] {tag}: inputs and warmup in {time.perf_counter() - t0:.1f}s")
        M.profile_read()
        M.profile_enable(True)
        torch.cuda.synchronize()
        ts = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        el = time.perf_counter() - ts
        M.profile_enable(False)
        st = M.profile_read()
        ms = el / steps * 1e3
        wb = W.DecodeWorkload(w.name, w.dtype, w.num_q_heads, w.num_kv_heads, w.max_len, w.head_dim, B, k, w.lens)
        by = decode_bytes(wb, sel.cpu().numpy(), list(w.lens), M.DECODE_CHUNK)
        attn = st["decode_attn"]
        attn_ms = attn["ms"] / max(attn["launches"], 1)
        res[tag] = {"block_size": B, "topk": k, "ms_per_step": ms, "steps": steps,
                    "tokens_per_s": w.batch / (ms * 1e-3), "bytes_per_step": by,
                    "hbm_gbs_step": by["total"] / (ms * 1e-3) / 1e9,
                    "attn_kernel_ms": attn_ms, "attn_kernel_gbs": by["attn_kernel"] / (attn_ms * 1e-3) / 1e9,
                    "stages_ms": {n: x["ms"] / steps for n, x in st.items() if x["launches"]}}
        log(f"[decode] {tag}: {ms:.3f} ms/step, attention kernel {attn_ms:.3f} ms "
            f"({res[tag]['attn_kernel_gbs']:.0f} GB/s)")
        del out, sel, ws, mu
        torch.cuda.empty_cache()
    moba = res["moba"]
    line = {
        "metric": "MoBA decode step: sequences decoded per second (one new token each)",
        "value": moba["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": moba["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1), bf16-rounded caches; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "max_len": w.max_len, "cache_lens": list(w.lens),
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "topk": w.topk},
        "moba": moba, "dense": res.get("dense"),
        "speedup_vs_dense": res["dense"]["ms_per_step"] / moba["ms_per_step"] if dense else None,
        "roofline": {"bound": "hbm", "kernel": "moba::decode_attn_kernel<unsigned short, 128>",
                     "achieved": moba["attn_kernel_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": moba["attn_kernel_gbs"] / PEAK_HBM_GBS, "traffic": None},
    }
    if cpu_seconds > 0:
        import oracle.moba_oracle as O
        qh = q.cpu()
        kh, vh = kc[0].cpu(), vc[0].cpu()  # sequence 0 only

        class Src:
            def __init__(self, t):
                self.t, self.shape = t, (1,) + tuple(t.shape)

            def __getitem__(self, idx):
                return self.t[idx[1:]].to(torch.float64).numpy()

        g = w.num_q_heads // w.num_kv_heads
        done, tsum = 0, 0.0
        for hk in range(w.num_kv_heads):
            if tsum >= cpu_seconds:
                break
            rows = [(0, h) for h in range(hk * g, (hk + 1) * g)]
            ts = time.perf_counter()
            O.decode_rows(qh[:1].to(torch.float64).numpy(), Src(kh), Src(vh), [w.lens[0]], w.block_size,
                          w.topk, rows=rows)
            tsum += time.perf_counter() - ts
            done += len(rows)
        line["cpu_baseline"] = {"value": done / w.num_q_heads / tsum, "unit": "tokens/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"fp64 numpy oracle decode_rows on sequence 0: {done} of its "
                                          f"{w.num_q_heads} heads in {tsum:.1f}s (per-KV-head fp64 conversion "
                                          f"of the cached prefix and its block means included); value = "
                                          f"sequences per second at that rate"}
    return line


def measure_backward(M, W, w, steps, warmup, log):
    """Training step of the attention: moba_attn_fwd_train, then
    moba_attn_bwd with the forward's selection (dout seeded N(0,1)).  Useful
    FLOPs: the forward's 4 D per attended key, the backward's 10 D (five
    products: S and dP recomputed once, dV, dK, dQ)."""
    import torch
    t0 = time.perf_counter()
    q, k, v, _ = W.make_inputs(w, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype)
    dt = M.DTYPE_BF16
    wsf = torch.empty(M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt,
                                        w.block_size, w.topk, w.causal), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(M.bwd_workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt,
                                            w.block_size, w.topk, w.causal), dtype=torch.uint8, device="cuda")
    log(f"[bwd] {w.name}: inputs in {time.perf_counter() - t0:.1f}s, workspaces {wsf.numel() / 2**30:.2f} + "
        f"{wsb.numel() / 2**30:.2f} GiB")
    fwd = lambda: M.moba_attn_fwd_train(q, k, v, w.block_size, w.topk, w.causal, workspace=wsf)
    out, sel, lse = fwd()
    bwd = lambda: M.moba_attn_bwd(q, k, v, out, dout, lse, sel, w.block_size, w.topk, w.causal, workspace=wsb)
    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    res = {"workload": w.name}
    for tag, fn in (("forward_train", fwd), ("backward", bwd)):
        M.profile_read()
        M.profile_enable(True)
        torch.cuda.synchronize()
        ts = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - ts) / steps * 1e3
        M.profile_enable(False)
        st = M.profile_read()
        res[tag] = {"ms": ms, "stages": {n: {"ms": x["ms"] / steps, "launches": x["launches"] / steps,
                                             "tflops": x["work"] / (x["ms"] * 1e-3) / 1e12
                                             if x["ms"] > 0 and n.startswith(("attn", "bwd_d")) else None}
                                         for n, x in st.items() if x["launches"]}}
        if tag == "backward":
            res["dkdv"] = st["bwd_dkdv"]
            res["dq"] = st["bwd_dq"]
        log(f"[bwd] {w.name} {tag}: {ms:.2f} ms")
    fl = useful_flops(w)
    bw = res["backward"]["ms"]
    dkdv = res.pop("dkdv")
    dq = res.pop("dq")
    dk_ms = dkdv["ms"] / steps / max(dkdv["launches"] / steps, 1)
    line = {
        "metric": "MoBA attention backward useful TFLOP/s (10 D per attended key)",
        "value": 2.5 * fl / (bw * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": bw, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), bf16-rounded; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "topk": w.topk, "causal": w.causal},
        "forward_train_ms": res["forward_train"]["ms"],
        "train_step_ms": res["forward_train"]["ms"] + bw,
        "train_step_useful_tflops": 3.5 * fl / ((res["forward_train"]["ms"] + bw) * 1e-3) / 1e12,
        "stages": res["backward"]["stages"],
        "roofline": {"bound": "mfma", "kernel": "moba::bwd_dkdv_kernel", "achieved": dkdv["work"] / steps /
                     (dkdv["ms"] / steps * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "avg_launch_ms": dk_ms, "traffic": None},
    }
    line["roofline"]["frac"] = line["roofline"]["achieved"] / PEAK_BF16_TFLOPS
    return line


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
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the bf16 GEMM reference rate measured after the run")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--gate", choices=("mean", "minmax"), default="mean",
                    help="block gate: block means (the method's) or element-wise key min / max")
    ap.add_argument("--decode", nargs="?", const="decode_gqa32x8_1m_b8", default=None, metavar="WORKLOAD",
                    help="measure decode-time MoBA on a decode workload instead, then exit")
    ap.add_argument("--backward", nargs="?", const="gqa32x8_128k", default=None, metavar="WORKLOAD",
                    help="measure the attention training step (forward with lse, backward) instead, then exit")
    ap.add_argument("--decode-skip-dense", action="store_true",
                    help="with --decode: skip the dense-decode comparison")
    ap.add_argument("--summarize-decode-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="write the decode kernel-trace summary from a rocprofv3 --stats run, then exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain copy of MIB MiB first (reference dispatch for HBM byte counters)")
    ap.add_argument("--chunk-sweep", nargs="+", default=None, metavar="WORKLOAD [CHUNK_BLOCKS ...]",
                    help="time a workload with workspaces that hold at most these many query blocks per chunk "
                         "(one JSON line each; default 0 = the library's default chunk)")
    ap.add_argument("--granularity", action="store_true",
                    help="time the 32K forward at the report's five block granularities (75 %% sparsity), then exit")
    ap.add_argument("--gemm-peak", action="store_true",
                    help="measure the attainable dense bf16 GEMM rate (torch.matmul), then exit")
    ap.add_argument("--curve-moba-only", action="store_true",
                    help="with --curve: MoBA side only (for lengths where dense attention takes minutes)")
    ap.add_argument("--curve", nargs="*", type=int, metavar="SEQLEN",
                    help="MoBA (256 blocks, top-12) vs dense causal attention at these lengths, one JSON line each")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc runs, then exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="write the kernel-trace summary from a rocprofv3 --stats run, then exit")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "BENCH_JSON"),
                    help="write the MFMA-busy summary from a rocprofv3 --pmc run, then exit")
    ap.add_argument("--summarize-valu", nargs=2, metavar=("PMC_DIR", "BENCH_JSON"),
                    help="write profiles/valu_<workload>.md from a VALU counter run")
    ap.add_argument("--summarize-bwd-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="write profiles/kernel_trace_bwd_gqa32x8_128k.md from a kernel-trace run of --backward")
    ap.add_argument("--summarize-hbm", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="write the per-kernel HBM summary from the two traffic runs, then exit")
    args = ap.parse_args()
    if args.summarize_mfma:
        print(json.dumps(summarize_mfma(*args.summarize_mfma), indent=1))
        return
    if args.summarize_hbm:
        print(json.dumps(summarize_stage_hbm(args.summarize_hbm[0], args.summarize_hbm[1], 1024,
                                             args.summarize_hbm[2]), indent=1))
        return
    if args.summarize_valu:
        print(json.dumps(summarize_valu(*args.summarize_valu), indent=1))
        return
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(*args.summarize_traffic, 1024, TRAFFIC_FILE), indent=1))
        return
    if args.summarize_decode_trace:
        summarize_decode_trace(*args.summarize_decode_trace,
                               os.path.join(ROOT, "profiles", "kernel_trace_decode_gqa32x8_1m_b8.md"))
        return
    if args.summarize_bwd_trace:
        summarize_bwd_trace(*args.summarize_bwd_trace,
                            os.path.join(ROOT, "profiles", "kernel_trace_bwd_gqa32x8_128k.md"))
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, os.path.join(ROOT, "profiles", "kernel_trace_gqa32x8_1m.md"))
        return

    def log(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: there is no multi-GPU path "
                  "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import block_sparse_attention_40_amd as M
    import moba_workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.granularity:
        granularity(M, W, log)
        return
    if args.chunk_sweep:
        wc = W.WORKLOADS[args.chunk_sweep[0]]
        for cap in [int(x) for x in args.chunk_sweep[1:]] or [0]:
            dt = M.DTYPE_BF16 if wc.dtype == "bf16" else M.DTYPE_F32
            nbytes = M.workspace_bytes(wc.batch, wc.seqlen, wc.num_q_heads, wc.num_kv_heads, wc.head_dim, dt,
                                       wc.block_size, wc.topk, wc.causal, max_chunk_blocks=cap)
            plan = M.plan_info(wc.batch, wc.seqlen, wc.num_q_heads, wc.num_kv_heads, wc.head_dim, dt,
                               wc.block_size, wc.topk, wc.causal, nbytes)
            r, inp, _ = measure(M, W, wc, args.steps, args.warmup, log, gate=args.gate, max_chunk_blocks=cap)
            del inp
            print(json.dumps({"workload": wc.name, "max_chunk_blocks": cap, "plan": plan,
                              "workspace_bytes": nbytes, **r}), flush=True)
        return
    if args.gemm_peak:
        gemm_peak(log)
        return
    if args.backward:
        print(json.dumps(measure_backward(M, W, W.WORKLOADS[args.backward], args.steps, args.warmup, log)),
              flush=True)
        return
    if args.decode:
        print(json.dumps(measure_decode(M, W, W.DECODE_WORKLOADS[args.decode], args.steps, args.warmup, log,
                                        0.0 if args.no_cpu_baseline else min(args.cpu_seconds, 10.0),
                                        dense=not args.decode_skip_dense)),
              flush=True)
        return
    if args.curve is not None:
        curve(M, W, args.curve or [32768, 65536, 131072, 262144, 524288, 1048576], log,
              moba_only=args.curve_moba_only)
        return
    w = W.WORKLOADS[args.workload]
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, log)
    res, inputs, stages = measure(M, W, w, args.steps, args.warmup, log, gate=args.gate)
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
                   "topk": w.topk, "causal": w.causal, "gate": args.gate, "parallelism": "none (1 GPU)"},
        "tokens_per_s": res["tokens_per_s"],
        "attention_tflops": res["attention_tflops"],
        "mfma_util_attention": res["mfma_util_attention"],
        "stages": res["stages"],
        "roofline": roofline(stages, args.steps, past_kernel_name(M, w), w.name),
    }
    if args.secondary:
        w2 = W.WORKLOADS[args.secondary]
        res2, inputs2, _ = measure(M, W, w2, args.secondary_steps, max(args.warmup, 3), log, gate=args.gate,
                                   graph=True)
        del inputs2
        line["secondary"] = res2
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W, w, inputs, args.cpu_seconds, log, gate=args.gate)
    if not args.no_gemm_reference and line["roofline"]:
        # context for the roofline: what a library GEMM attains on this GPU now
        del inputs
        torch.cuda.empty_cache()
        g = gemm_peak(log, sizes=(8192,), emit=False)
        line["gemm_reference"] = {"kernel": "torch.matmul bf16 8192^3 (hipBLASLt)", "tflops": g["8192"],
                                  "past_kernel_frac_of_gemm": line["roofline"]["achieved"] / g["8192"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
