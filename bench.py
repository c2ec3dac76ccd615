"""Throughput of the SageBwd INT8 attention path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM:  sage_quantize -> sage_fwd -> sage_bwd_pre ->
sage_bwd, through the C ABI, on the workload with d = 128 and N = 8192
(B = 2, H = 16, causal, bf16, QK-normed Q/K with a per-channel K offset).

Throughput is attention operations per second in the FlashAttention
convention (forward 4*B*H*N^2*d, backward 10*B*H*N^2*d, halved for causal).
Besides the one JSON line the driver reads, the line carries per-call times
(HIP events on the launch stream), the roofline of the dominant kernel and a
CPU baseline: the oracle timed on this machine's host cores on a bounded
sample (ten whole heads of the same workload).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SageBwd fwd+bwd TOPS at d=128,N=8K (1 GPU) + % of INT8 MFMA peak"
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense BF16 MFMA, published
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the HIP sources: traffic counters are only valid for this code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_trainable_attention_block_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(call: str):
    """HBM bytes per launch of C-ABI call `call` from the committed counter
    summary (profiles/traffic.json), or None when absent or taken on
    different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("source_hash") != kernel_source_hash():
            return None
        return t["calls"][call]["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


SQ_FILE = os.path.join(ROOT, "profiles", "sq_utilisation.json")
SQ_KERNELS = ("fwd_kernel", "bwd_kernel", "dq_kernel")
# VALU instruction classes counted separately on gfx950 (a third counter run)
SQ_VALU_CLASSES = ("SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_FMA_F32",
                   "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_INT32", "SQ_INSTS_VALU_INT64")
HEADLINE_WORKLOAD = "d128_n8k_causal_qknorm"


def full_size_workloads():
    """The full-size workloads of the sweep, by name."""
    from bit_trainable_attention_block_amd import workloads as wl
    return {c.name: c for c in (wl.C2, wl.C2_CAUSAL, wl.C3, *wl.C4, wl.C5, wl.C5_QSMOOTH)}


def sq_file(workload):
    return SQ_FILE if workload == HEADLINE_WORKLOAD else os.path.join(ROOT, "profiles", f"sq_utilisation_{workload}.json")


def sq_from(directory, workload=HEADLINE_WORKLOAD, out_path=None):
    """Write profiles/sq_utilisation.json (or out_path; and print its table rows) from
    rocprofv3 --pmc runs of one bench step under `directory` holding the SQ
    counters below.  Derived per kernel, with T = GRBM_GUI_ACTIVE / 8 (the
    counter is summed over the eight XCDs), 1024 SIMDs and 256 CUs: VALU issue
    busy = 4 cycles x SQ_INSTS_VALU (MFMA included) per SIMD over T; MFMA busy
    = SQ_VALU_MFMA_BUSY_CYCLES per SIMD over T; LDS busy = SQ_LDS_IDX_ACTIVE
    per CU over T; resident waves per SIMD = 4 SQ_WAVE_CYCLES / (1024 T)
    (the counter advances once per four cycles of each resident wave: the
    backward's two-wave workgroups read 1.84, its launch limit being 2);
    instructions per 64 unmasked (query, key) pairs of `workload` (one
    bench step of it), with the VALU classes of SQ_VALU_CLASSES when a run
    holds them ("other" = VALU minus MFMA minus those classes)."""
    import csv
    import glob
    sums = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].replace("sage::(anonymous namespace)::", "").replace("void ", "")
            name = name.split("(")[0].split("<")[0].strip()
            if name in SQ_KERNELS:
                d = sums.setdefault(name, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    cfg = full_size_workloads()[workload]
    out_path = out_path or sq_file(workload)
    pairs64 = cfg.attention_ops()[0] / (4 * cfg.D) / 64
    out = {}
    for k in SQ_KERNELS:
        v = sums[k]
        T = v["GRBM_GUI_ACTIVE"] / 8
        out[k] = {
            "cycles": T,
            "valu_issue_busy": 4 * v["SQ_INSTS_VALU"] / (1024 * T),
            "mfma_busy": v["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * T),
            "mfma_valu_coexec": v["SQ_VALU_MFMA_COEXEC_CYCLES"] / (1024 * T),
            "lds_busy": v["SQ_LDS_IDX_ACTIVE"] / (256 * T),
            "waves_waiting_on_dependency": v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"],
            "waves_issuing": v["SQ_ACTIVE_INST_ANY"] / v["SQ_WAVE_CYCLES"],
            "valu_per_64_pairs": (v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"]) / pairs64,
            "mfma_per_64_pairs": v["SQ_INSTS_MFMA"] / pairs64,
            "exp_per_64_pairs": v["SQ_INSTS_VALU_TRANS_F32"] / pairs64,
            "salu_per_64_pairs": v["SQ_INSTS_SALU"] / pairs64,
            "resident_waves_per_simd": 4 * v["SQ_WAVE_CYCLES"] / (1024 * T),
        }
        if all(c in v for c in SQ_VALU_CLASSES):
            cls = {c[len("SQ_INSTS_VALU_"):]: v[c] / pairs64 for c in SQ_VALU_CLASSES}
            cls["other"] = out[k]["valu_per_64_pairs"] - sum(cls.values())
            out[k]["valu_classes_per_64_pairs"] = cls
    doc = {"source_hash": kernel_source_hash(), "workload": workload, "kernels": out}
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
    for k, d in out.items():
        print(f"| `{k}` | {d['cycles']/1e6:.3f} | {d['valu_issue_busy']:.0%} | {d['mfma_busy']:.1%} | "
              f"{d['mfma_valu_coexec']:.1%} | {d['lds_busy']:.1%} | {d['waves_waiting_on_dependency']:.0%} | "
              f"{d['waves_issuing']:.0%} | {d['valu_per_64_pairs']:.1f} | {d['mfma_per_64_pairs']:.2f} | "
              f"{d['exp_per_64_pairs']:.2f} | {d['salu_per_64_pairs']:.1f} | {d['resident_waves_per_simd']:.2f} |")
    for k, d in out.items():
        if "valu_classes_per_64_pairs" in d:
            print(f"| `{k}` | " + " | ".join(f"{n} {x:.2f}" for n, x in d["valu_classes_per_64_pairs"].items()) + " |")
    return doc


def measured_sq(kernel: str):
    """The committed shader-pipe figures of `kernel` (profiles/sq_utilisation.json),
    or None when absent or taken on different kernel sources."""
    try:
        with open(SQ_FILE) as f:
            t = json.load(f)
        if t.get("source_hash") != kernel_source_hash():
            return None
        d = t["kernels"][kernel]
        return {"valu_issue_busy": round(d["valu_issue_busy"], 3), "mfma_busy": round(d["mfma_busy"], 3)}
    except (OSError, KeyError, ValueError):
        return None


# kernels of each C-ABI call (by name prefix in the counter output)
CALL_KERNELS = {
    "sage_quantize": ("quant_v_ksum_kernel", "kmean_kernel", "quant_q_kernel", "quant_k_kernel"),
    "sage_fwd": ("fwd_kernel",),
    "sage_bwd_pre": ("bwd_pre_kernel",),
    "sage_bwd": ("bwd_kernel", "dq_kernel"),
}


def _counter_means(directory):
    """{short kernel name: {counter: mean value per dispatch}} from the
    rocprofv3 counter_collection.csv files under `directory`."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].replace("sage::(anonymous namespace)::", "").replace("void ", "")
            name = name.split("(")[0].split("<")[0].strip()
            key = (name, r["Counter_Name"])
            sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
            counts.setdefault(key, set()).add(r["Dispatch_Id"])
    out = {}
    for (name, ctr), v in sums.items():
        out.setdefault(name, {})[ctr] = v / len(counts[(name, ctr)])
    return out


def traffic_from(directory, copy_bytes):
    """Write profiles/traffic.json (and print it) from four rocprofv3 --pmc
    runs under `directory`: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE over one
    bench step) and copy_fetch/, copy_write/ (the same counters over a plain
    device copy of `copy_bytes` bytes, which calibrates both counters)."""
    fetch = _counter_means(os.path.join(directory, "fetch"))
    write = _counter_means(os.path.join(directory, "write"))
    cf = _counter_means(os.path.join(directory, "copy_fetch"))
    cw = _counter_means(os.path.join(directory, "copy_write"))
    copy_kernel = max(cf, key=lambda k: cf[k].get("FETCH_SIZE", 0.0))
    k_fetch = copy_bytes / (cf[copy_kernel]["FETCH_SIZE"] * 1024.0)
    k_write = copy_bytes / (cw[copy_kernel]["WRITE_SIZE"] * 1024.0)
    kernels, calls = {}, {}
    for name in sorted(set(fetch) | set(write)):
        fb = fetch.get(name, {}).get("FETCH_SIZE", 0.0) * 1024.0 * k_fetch
        wb = write.get(name, {}).get("WRITE_SIZE", 0.0) * 1024.0 * k_write
        kernels[name] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    for call, names in CALL_KERNELS.items():
        fb = sum(kernels[n]["fetch_bytes"] for n in names if n in kernels)
        wb = sum(kernels[n]["write_bytes"] for n in names if n in kernels)
        calls[call] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    out = {"source_hash": kernel_source_hash(), "workload": "d128_n8k_causal_qknorm",
           "copy_probe": {"kernel": copy_kernel, "bytes": copy_bytes, "fetch_factor": k_fetch,
                          "write_factor": k_write},
           "calls": calls, "kernels": kernels}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


# whole heads timed for the CPU baseline, one per worker process
CPU_HEADS = ((0, 0), (0, 5), (0, 10), (0, 15), (1, 0), (1, 3), (1, 7), (1, 9), (1, 12), (1, 15), (1, 2),
             (0, 8), (1, 5), (0, 3), (1, 11), (0, 13))
CPU_WORKERS_MAX = 16  # at most 16 heads of 1.5-6 s of CPU work each: a bounded sample


def _cpu_head(args):
    """One whole head through the oracle as it stands (single BLAS thread);
    returns (forward seconds, backward seconds, start, end): quantize + fwd,
    then bwd_pre + bwd, and the wall-clock span of that work."""
    cfg, head = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    from bit_trainable_attention_block_amd import workloads as wl
    from oracle import sage

    sh = sage.Shape.of(cfg)
    x = wl.generate(cfg, heads=head)
    Q, K, V, dO = (x[n]["f32"][0, 0].astype(np.float64) for n in ("q", "k", "v", "do"))
    with threadpool_limits(1):
        start = time.time()
        t0 = time.perf_counter()
        qz = sage.quantize(Q, K, V, sh)
        O, L = sage.forward(qz, sh)
        t1 = time.perf_counter()
        delta, dOc, sdO = sage.backward_pre(O, dO, sh)
        sage.backward(qz, V, dO, dOc, sdO, L, delta, sh)
        t2 = time.perf_counter()
        end = time.time()
    return t1 - t0, t2 - t1, start, end


def sample_heads(cfg, n):
    """n (batch, head) pairs spread evenly over the workload's B*H heads."""
    total = cfg.B * cfg.H
    n = min(n, total)
    return [divmod(k * total // n, cfg.H) for k in range(n)]


def cpu_baseline(cfg, heads=None):
    """The oracle as it stands on whole heads of the workload, one head per
    worker process (single BLAS thread each), the workers started before
    anything touches the GPU.  value = attention ops of the sampled heads
    over the wall-clock span from the first worker's start to the last
    worker's end of that work (input generation and imports excluded).
    heads: the (batch, head) pairs to time; by default the fixed sample of
    the d=128 N=8192 causal workload, as many as there are workers."""
    import multiprocessing as mp

    cpus = len(os.sched_getaffinity(0))
    workers = max(1, min(CPU_WORKERS_MAX, cpus))
    heads = CPU_HEADS[:workers] if heads is None else heads[:workers]
    fwd_ops, bwd_ops = (v / (cfg.B * cfg.H) for v in cfg.attention_ops())
    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map(abs, range(workers))          # interpreters up
        times = pool.map(_cpu_head, [(cfg, h) for h in heads], chunksize=1)
    wall = max(t[3] for t in times) - min(t[2] for t in times)
    tf = sum(t[0] for t in times)
    tb = sum(t[1] for t in times)
    n = len(heads)
    return {"value": (fwd_ops + bwd_ops) * n / wall / 1e12, "unit": "TOPS", "cores": workers, "kind": "oracle",
            "sample": f"{n} of {cfg.B * cfg.H} heads of the same workload, whole chain (quantize, fwd, bwd_pre, "
                      f"bwd), one head per process, {wall:.1f} s wall, {tf + tb:.1f} s of CPU work",
            "fwd_tops_per_core": fwd_ops * n / tf / 1e12, "bwd_tops_per_core": bwd_ops * n / tb / 1e12,
            "fwd_cpu_s": round(tf, 2), "bwd_cpu_s": round(tb, 2),
            "host_cpus": os.cpu_count(), "affinity_cpus": cpus, "blas_threads": 1}


def cpu_sweep():
    """One JSON line per workload configuration (tiny, d=64 N=2048, d=128
    N=8192 causal, the sigma=1 member of the sigma sweep, N=32768 causal):
    the oracle's whole chain on up to CPU_WORKERS_MAX heads spread over the
    workload, fwd (quantize + fwd) and bwd (bwd_pre + bwd) CPU seconds and
    TOPS in the same convention as the GPU figures."""
    from bit_trainable_attention_block_amd import workloads as wl
    for cfg in (wl.C1, wl.C2, wl.C3, wl.C4[0], wl.C5):
        r = cpu_baseline(cfg, sample_heads(cfg, CPU_WORKERS_MAX))
        print(json.dumps({"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "D": cfg.D,
                          "causal": cfg.causal, **r}), flush=True)


def mfma_probe(kind="i8", iters=4000):
    """Achieved rate of v_mfma_i32_16x16x64_i8 (kind "i8") or
    v_mfma_f32_16x16x32_bf16 ("bf16") on this device (two 8-wave workgroups
    per CU, register operands) and the shader clock under it."""
    import torch

    from bit_trainable_attention_block_amd import binding as bd
    probe, ops_each, name, spec = {
        "i8": (bd.probe_mfma_i8, 32768, "v_mfma_i32_16x16x64_i8", INT8_PEAK_TOPS),
        "bf16": (bd.probe_mfma_bf16, 16384, "v_mfma_f32_16x16x32_bf16", BF16_PEAK_TFLOPS)}[kind]
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    clk = torch.zeros(3, dtype=torch.int64, device="cuda")
    probe(blocks, 200, clk)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    probe(blocks, iters, clk)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ops = blocks * 8 * iters * 8 * ops_each
    c = [int(v) for v in clk.cpu().tolist()]
    tops = ops / (ms * 1e-3) / 1e12
    return {"kernel": name, "tops": round(tops, 1),
            "clock_ghz": round(c[0] / (c[1] / 100e6) / 1e9, 3) if c[1] else None,
            "frac_of_spec": round(tops / spec, 4)}


def bwd_work(cfg):
    """Algorithmic work of one sage_bwd launch, by dtype: per unmasked
    (query, key) pair 2*D operations for each of the four INT8 products (S
    recompute, dV, dK, dQ) and 2*D for the BF16 dP product."""
    pairs = float(cfg.B * cfg.H) * cfg.N * cfg.N * (0.5 if cfg.causal else 1.0)
    return {"int8_ops": 8.0 * cfg.D * pairs, "bf16_flops": 2.0 * cfg.D * pairs}


def mixed_ceiling_tops(work):
    """Rate (TOP/s) at which that work would run with each product at its own
    dtype's published dense peak: INT8 at 5.0 POP/s, BF16 at 2.5 PFLOP/s."""
    ideal_s = work["int8_ops"] / (INT8_PEAK_TOPS * 1e12) + work["bf16_flops"] / (BF16_PEAK_TFLOPS * 1e12)
    return (work["int8_ops"] + work["bf16_flops"]) / ideal_s / 1e12


# Algorithmic HBM bytes per (token, channel) element of the HBM-bound calls,
# what the method itself must move: sage_quantize reads Q once and K twice
# (the token mean, then the codes) and V once in 16 bits, and writes one code
# byte each of Q, K and V (11 B); sage_bwd_pre reads O and dO in 16 bits and
# writes dO's codes (5 B) plus delta (4 B per row).
QUANT_ALGO_BYTES = 11.0


def bwd_pre_algo_bytes(D):
    return 5.0 + 4.0 / D


def copy_gbps(mib=512, reps=5):
    """Plain device copy bandwidth (bytes read + written per second)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def sweep(steps, warmup, only=None):
    """One JSON line per full-size workload (not the default headline line):
    the four calls' mean times (HIP events on the launch stream) and the
    forward, backward and whole-step TOPS in the FlashAttention convention."""
    import numpy as np
    import torch
    from bit_trainable_attention_block_amd import binding as bd
    from bit_trainable_attention_block_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bd.load()
    stream = torch.cuda.current_stream()
    for name, cfg in full_size_workloads().items():
        if only and name != only:
            continue
        sh = bd.Shape.of(cfg)
        x = wl.generate(cfg)
        Q, K, V, dO = (torch.from_numpy(x[n]["bits"].view(np.int16)).to("cuda").view(sh.torch_dtype)
                       for n in ("q", "k", "v", "do"))
        del x
        qt, dot, bws = bd.alloc_qtensors(sh), bd.alloc_dotensors(sh), bd.bwd_workspace(sh)
        O = torch.empty(Q.shape, dtype=sh.torch_dtype, device="cuda")
        L = torch.empty(Q.shape[:3], dtype=torch.float32, device="cuda")
        dQ, dK, dV = (torch.empty(Q.shape, dtype=torch.float32, device="cuda") for _ in range(3))
        calls = (lambda: bd.quantize(sh, Q, K, V, out=qt), lambda: bd.fwd(sh, qt, O, L),
                 lambda: bd.bwd_pre(sh, O, dO, out=dot), lambda: bd.bwd(sh, qt, dot, V, dO, L, dQ, dK, dV, ws=bws))
        for _ in range(warmup):
            for c in calls:
                c()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        for k in range(steps):
            for i, c in enumerate(calls):
                ev[k][i].record(stream)
                c()
            ev[k][4].record(stream)
        torch.cuda.synchronize()
        ms = np.mean([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in ev], axis=0)
        fwd_ops, bwd_ops = cfg.attention_ops()
        print(json.dumps({"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "D": cfg.D,
                          "causal": cfg.causal, "q_smooth": cfg.q_smooth,
                          "call_ms": dict(zip(("sage_quantize", "sage_fwd", "sage_bwd_pre", "sage_bwd"),
                                              (round(float(v), 4) for v in ms))),
                          "fwd_kernel_tops": round(fwd_ops / (ms[1] * 1e-3) / 1e12, 1),
                          "bwd_kernel_tops": round(bwd_ops / (ms[3] * 1e-3) / 1e12, 1),
                          "step_tops": round((fwd_ops + bwd_ops) / (float(ms.sum()) * 1e-3) / 1e12, 1)}),
              flush=True)
        del Q, K, V, dO, qt, dot, bws, O, L, dQ, dK, dV
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the INT8-dP and E4M3 legs (profiler runs: only the method's kernels launch)")
    ap.add_argument("--traffic-from", default="",
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs in this directory into "
                         "profiles/traffic.json (no GPU needed) and exit")
    ap.add_argument("--sq-from", default="",
                    help="summarise rocprofv3 SQ counter runs in this directory into "
                         "profiles/sq_utilisation.json (no GPU needed) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line of call times and TOPS per full-size workload, then exit")
    ap.add_argument("--cpu-sweep", action="store_true",
                    help="the oracle's CPU baseline on a bounded sample of heads of each of the five "
                         "workload configurations (one JSON line each; no GPU needed), then exit")
    ap.add_argument("--workload", default="",
                    help="with --sweep: only this full-size workload (a profiler run of its kernels); "
                         "with --sq-from: the workload the counter runs were taken on")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run one plain device-to-device copy of this many MiB (the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from, 1024 << 20)
        return
    if args.sq_from:
        sq_from(args.sq_from, args.workload or HEADLINE_WORKLOAD)
        return
    if args.cpu_sweep:
        cpu_sweep()
        return
    if args.sweep and args.gpus == 1:
        if args.workload and args.workload not in full_size_workloads():
            print(f"bench.py: unknown workload {args.workload}", file=sys.stderr)
            sys.exit(2)
        sweep(args.steps, args.warmup, args.workload or None)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_trainable_attention_block_amd import binding as bd
    from bit_trainable_attention_block_amd import workloads as wl

    # the oracle's timing runs first, in worker processes started while
    # nothing in this process has touched the GPU
    cpu = None
    if not args.no_cpu_baseline and not args.copy_probe_mib:
        cpu = cpu_baseline(wl.C3)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}), flush=True)
        return
    bd.load()
    cfg = wl.C3
    sh = bd.Shape.of(cfg)
    x = wl.generate(cfg)
    dt = sh.torch_dtype
    Q, K, V, dO = (torch.from_numpy(x[n]["bits"].view(np.int16)).to("cuda").view(dt) for n in ("q", "k", "v", "do"))
    del x
    qt = bd.alloc_qtensors(sh)
    dot = bd.alloc_dotensors(sh)
    O = torch.empty(Q.shape, dtype=dt, device="cuda")
    L = torch.empty(Q.shape[:3], dtype=torch.float32, device="cuda")
    dQ, dK, dV = (torch.empty(Q.shape, dtype=torch.float32, device="cuda") for _ in range(3))
    bws = bd.bwd_workspace(sh)
    stream = torch.cuda.current_stream()

    calls = ("sage_quantize", "sage_fwd", "sage_bwd_pre", "sage_bwd")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        bd.quantize(sh, Q, K, V, out=qt)
        if ev is not None:
            ev[1].record(stream)
        bd.fwd(sh, qt, O, L)
        if ev is not None:
            ev[2].record(stream)
        bd.bwd_pre(sh, O, dO, out=dot)
        if ev is not None:
            ev[3].record(stream)
        bd.bwd(sh, qt, dot, V, dO, L, dQ, dK, dV, ws=bws)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_call = {c: [] for c in calls}
    for ev in events:
        for i, c in enumerate(calls):
            per_call[c].append(ev[i].elapsed_time(ev[i + 1]))
    call_ms = {c: float(np.mean(v)) for c, v in per_call.items()}
    step_ms = np.array([ev[0].elapsed_time(ev[4]) for ev in events])
    ms_per_step = wall * 1e3 / args.steps
    fwd_ops, bwd_ops = cfg.attention_ops()
    total_ops = fwd_ops + bwd_ops
    tops = total_ops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the backward (MFMA-bound).  Algorithmic work per launch:
    # 8*D INT8 operations (S, dV, dK, dQ) and 2*D BF16 flops (dP) per unmasked
    # (query, key) pair of the B*H heads.  The peak prices each product at its
    # own dtype's published dense rate (INT8 5.0 POP/s, BF16 2.5 PFLOP/s), so
    # `frac` is the fraction of the time the matrix cores would need.
    bwd_ms = call_ms["sage_bwd"]
    bwd_tops = bwd_ops / (bwd_ms * 1e-3) / 1e12
    work = bwd_work(cfg)
    peak = mixed_ceiling_tops(work)
    traffic = measured_traffic("sage_bwd")
    roofline = {"bound": "mfma", "kernel": "sage_bwd", "achieved": round(bwd_tops, 2), "peak": round(peak, 1),
                "unit": "TOP/s", "frac": round(bwd_tops / peak, 4),
                "traffic": traffic,
                "peak_basis": "INT8 ops at 5.0 POP/s plus BF16 flops at 2.5 PFLOP/s (published dense)",
                "work_per_launch": {k: v for k, v in work.items()},
                # the same achieved rate priced wholly at the INT8 peak
                "frac_of_int8_peak": round(bwd_tops / INT8_PEAK_TOPS, 4),
                # bwd_kernel's shader-pipe use from the committed SQ counter summary
                # (null once the kernels have changed since it was taken)
                "counters": measured_sq("bwd_kernel")}

    fwd_path_ms = call_ms["sage_quantize"] + call_ms["sage_fwd"]
    bwd_path_ms = call_ms["sage_bwd_pre"] + call_ms["sage_bwd"]
    breakdown = {
        "call_ms": {c: round(v, 4) for c, v in call_ms.items()},
        "call_ms_min": {c: round(float(np.min(v)), 4) for c, v in per_call.items()},
        "step_ms_median": round(float(np.median(step_ms)), 4), "step_ms_min": round(float(np.min(step_ms)), 4),
        "fwd_kernel_tops": round(fwd_ops / (call_ms["sage_fwd"] * 1e-3) / 1e12, 1),
        "bwd_kernel_tops": round(bwd_tops, 1),
        "fwd_path_tops": round(fwd_ops / (fwd_path_ms * 1e-3) / 1e12, 1),
        "bwd_path_tops": round(bwd_ops / (bwd_path_ms * 1e-3) / 1e12, 1),
        "pct_int8_peak_fwd_bwd": round(100 * tops / INT8_PEAK_TOPS, 2),
        "pct_int8_peak_fwd_kernel": round(100 * fwd_ops / (call_ms["sage_fwd"] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
        # the backward against its mixed ceiling (4 INT8 products + 1 BF16 one)
        "pct_mixed_ceiling_bwd_kernel": round(100 * bwd_tops / peak, 2),
    }
    # second denominators: the INT8 and BF16 product rates this device
    # achieves (the backward's measured mixed ceiling prices each product at
    # its probed rate), and the HBM-bound calls' algorithmic bytes per second
    # against the 8 TB/s figure and a plain copy timed here
    probe = mfma_probe("i8")
    probe_bf16 = mfma_probe("bf16")
    breakdown["mfma_probe"] = probe
    breakdown["mfma_probe_bf16"] = probe_bf16
    breakdown["pct_measured_i8_fwd_bwd"] = round(100 * tops / probe["tops"], 2)
    measured_mixed = (work["int8_ops"] + work["bf16_flops"]) / (
        work["int8_ops"] / probe["tops"] + work["bf16_flops"] / probe_bf16["tops"])
    breakdown["bwd_kernel_pct_measured_mixed"] = round(100 * bwd_tops / measured_mixed, 2)
    elems = cfg.B * cfg.H * cfg.N * cfg.D
    cp = copy_gbps()
    q_gbps = QUANT_ALGO_BYTES * elems / (call_ms["sage_quantize"] * 1e-3) / 1e9
    p_gbps = bwd_pre_algo_bytes(cfg.D) * elems / (call_ms["sage_bwd_pre"] * 1e-3) / 1e9
    breakdown["hbm"] = {"algo_bytes_per_elem": {"sage_quantize": QUANT_ALGO_BYTES,
                                                "sage_bwd_pre": round(bwd_pre_algo_bytes(cfg.D), 4)},
                        "copy_gbps": round(cp, 1),
                        "sage_quantize_gbps": round(q_gbps, 1),
                        "sage_quantize_pct_hbm_peak": round(100 * q_gbps / HBM_PEAK_GBS, 1),
                        "sage_quantize_pct_copy": round(100 * q_gbps / cp, 1),
                        "sage_bwd_pre_gbps": round(p_gbps, 1),
                        "sage_bwd_pre_pct_hbm_peak": round(100 * p_gbps / HBM_PEAK_GBS, 1),
                        "sage_bwd_pre_pct_copy": round(100 * p_gbps / cp, 1)}

    out = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8+bf16",
        "data": "synthetic (seeded Gaussian, QK-normed Q/K, per-channel K offset), resident in HBM",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "D": cfg.D, "causal": cfg.causal,
                   "io_dtype": "bf16", "bq": cfg.bq, "bkv": cfg.bkv, "k_smooth": cfg.k_smooth,
                   "q_smooth": cfg.q_smooth, "parallelism": "single GPU"},
        "roofline": roofline,
        "breakdown": breakdown,
    }
    # Variants (not the method), the same step with one switch flipped;
    # reported beside the headline, never as it: the INT8-dP ablation (dP
    # from the INT8 codes of dO and V) and the E4M3 variant (E4M3 codes and
    # float32 products in place of INT8)
    variants = () if args.no_variants else (("ablation_dp_int8", {"dp_int8": True}), ("variant_fp8", {"fp8": True}))
    for key, sw in variants:
        sha = dataclasses.replace(sh, **sw)
        # the INT8-dP ablation also writes and reads row-tile copies of V's and
        # dO's codes, so each variant gets buffers of its own
        qt, dot = bd.alloc_qtensors(sha), bd.alloc_dotensors(sha)
        ab_ms = []
        for k in range(args.warmup + max(3, args.steps // 4)):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record(stream)
            bd.quantize(sha, Q, K, V, out=qt)
            ev[1].record(stream)
            bd.fwd(sha, qt, O, L)
            ev[2].record(stream)
            bd.bwd_pre(sha, O, dO, out=dot)
            ev[3].record(stream)
            bd.bwd(sha, qt, dot, V, dO, L, dQ, dK, dV, ws=bws)
            ev[4].record(stream)
            torch.cuda.synchronize()
            if k >= args.warmup:
                ab_ms.append([ev[i].elapsed_time(ev[i + 1]) for i in range(4)])
        ab = np.mean(np.array(ab_ms), axis=0)
        breakdown[key] = {
            "call_ms": {c: round(float(v), 4) for c, v in zip(calls, ab)},
            "fwd_kernel_tops": round(fwd_ops / (ab[1] * 1e-3) / 1e12, 1),
            "bwd_kernel_tops": round(bwd_ops / (ab[3] * 1e-3) / 1e12, 1),
            "fwd_bwd_tops": round(total_ops / (float(ab.sum()) * 1e-3) / 1e12, 1)}

    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
