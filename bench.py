"""Benchmark of the Top-theta hot path on one MI355X.

Default workload (``decode_8b``): one Top-theta decode step of a LLaMA-3-8B-like
attention layer -- batch 16, 32 query / 8 KV heads, d=128, 4096 cached keys,
bf16, theta calibrated for k=128 from 256 decode-style sequences, VMC on.  A
step is one ``topth_decode`` call (scores, row log-sum-exp, threshold,
compaction, sparse SV, SDC/VMC: the whole decode path) on inputs already
resident in HBM; steps rotate over several distinct KV caches so the 256 MB
last-level cache cannot hold them.

The metric is HBM throughput on the bytes the method must read: all of K, the
V rows in the union of the kept keys of each GQA group, q, the theta row,
v_mean and seq_lens, divided by the average kernel duration (HIP events on the
launch stream).  One JSON line is printed; it also carries the roofline object
and the CPU oracle timed on the host as a reported baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import calibrated_threshold_pruning_amd as tt  # noqa: E402
from synth import CONFIG_IDS, ROLE_CALIB, ROLE_TEST, attention_inputs_device, to_f64  # noqa: E402

METRIC = "decode Top-θ attn: HBM GB/s on bytes read (% of peak); prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

DECODE_WORKLOADS = {
    "decode_8b": dict(B=16, Hq=32, Hkv=8, d=128, n=4096, k=128, calib=256, sinks=1, buffers=3),
    "decode_70b_32k": dict(B=8, Hq=64, Hkv=8, d=128, n=32768, k=256, calib=256, sinks=4, buffers=2),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def calibrate_decode_theta(name, w, dev):
    """theta [Hq, n] for k from `calib` decode-style sequences, on the GPU."""
    cfg = CONFIG_IDS[name]
    Hq, Hkv, d, n, k = w["Hq"], w["Hkv"], w["d"], w["n"], w["k"]
    s1 = torch.zeros(1, Hq, n, dtype=torch.float64, device=dev)
    s2 = torch.zeros_like(s1)
    cnt = torch.zeros(1, Hq, n, dtype=torch.int32, device=dev)
    chunk = max(1, min(32, (1 << 29) // (Hkv * n * d * 2)))
    ws = tt.workspace(tt.TOPTH_OP_CALIBRATE, chunk, Hq, Hkv, 1, n, d, 1)
    done = 0
    while done < w["calib"]:
        S = min(chunk, w["calib"] - done)
        q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, 0, done, B=S, Hq=Hq, Hkv=Hkv, Lq=1, Lk=n,
                                           d=d, n_sinks=w["sinks"], device=dev, with_v=False)
        tt.topth_calibrate(q, kk, [k], s1, s2, cnt, ws, scale=1.0 / math.sqrt(d), q_pos0=n - 1)
        done += S
    theta = torch.empty(1, Hq, n, dtype=torch.float32, device=dev)
    tt.topth_calibrate_finalize(s1, s2, cnt, [k], theta)
    torch.cuda.synchronize()
    return theta[0].contiguous()


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            threads = max(blas)
    except Exception:
        pass
    return model, threads


def oracle_decode_baseline(bufs, lens, theta, vm, w, bytes_of, budget_s=20.0):
    """Time the CPU oracle (float64 NumPy) on the first batch elements of the same
    decode workload; report GB/s over the same algorithmic bytes."""
    import oracle
    q, k, v = bufs
    B = q.shape[0]
    nb = B
    if w["n"] > 8192:
        nb = max(1, B // 4)
    qf = to_f64(q[:nb].cpu()); kf = to_f64(k[:nb].cpu()); vf = to_f64(v[:nb].cpu())
    th = theta.cpu().numpy().astype(np.float64)
    vmf = vm[:nb].cpu().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(w["d"])
    t0 = time.perf_counter()
    passes = 0
    vrows = None
    while True:
        r = oracle.decode(qf, kf, vf, lens[:nb], th, vmf, scale, vmc=True)
        vrows = r.vrows_read
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s * 0.5 or el + el / passes > budget_s:
            break
    el = time.perf_counter() - t0
    nbytes = bytes_of(nb, vrows.sum()) * passes
    model, threads = cpu_info()
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 NumPy oracle decode of batch elements 0..{nb - 1} of the same "
                      f"workload, {passes} pass(es), {el:.1f} s, host '{model}', "
                      f"{os.cpu_count()} logical CPUs"}


def bench_decode(name, steps, warmup, with_cpu, eager=False):
    w = DECODE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    cfg = CONFIG_IDS[name]
    B, Hq, Hkv, d, n = w["B"], w["Hq"], w["Hkv"], w["d"], w["n"]
    esz = 2
    log(f"[bench] {name}: calibrating theta from {w['calib']} sequences")
    theta = calibrate_decode_theta(name, w, dev)
    lens = [n] * B
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    bufs, vms = [], []
    for i in range(w["buffers"]):
        q, kk, v = attention_inputs_device(cfg, ROLE_TEST, 0, i, B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=n,
                                           d=d, n_sinks=w["sinks"], device=dev)
        q = q[:, :, 0].contiguous()
        vm = torch.empty(B, Hkv, d, dtype=torch.float32, device=dev)
        tt.topth_vmean(v, lens_d, vm)
        bufs.append((q, kk, v)); vms.append(vm)
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    vr = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, n, d)
    scale = 1.0 / math.sqrt(d)

    def read_bytes(nbatch, union_rows):
        return (nbatch * Hkv * n * d * esz          # K, every cached key
                + int(union_rows) * d * esz          # V rows of the group unions
                + nbatch * Hq * d * esz              # q
                + nbatch * Hq * 4                    # one theta per head
                + nbatch * Hkv * d * 4               # v_mean
                + nbatch * 4)                        # seq_lens

    def step(i):
        q, kk, v = bufs[i % len(bufs)]
        tt.topth_decode(q, kk, v, lens_d, theta, out, ws, scale=scale, flags=tt.TOPTH_VMC,
                        v_mean=vms[i % len(bufs)], kept_count=kc, vrows_read=vr)

    # union sizes and kept counts of every buffer (deterministic per buffer)
    per_buf_bytes, kept_ratio, union_rows = [], [], []
    for i in range(len(bufs)):
        step(i)
        torch.cuda.synchronize()
        per_buf_bytes.append(read_bytes(B, vr.sum().item()))
        kept_ratio.append(kc.float().mean().item() / w["k"])
        union_rows.append(vr.float().mean().item())
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if eager:
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            step(i)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # the K steps are captured once into a HIP graph (one launch per step,
        # no host work in between) and the graph is replayed
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    status = int(ws[:4].view(torch.int32)[0].item())
    if status != 0:
        raise RuntimeError(f"decode exchange wait timed out (status {status})")
    total_span = start.elapsed_time(end) * 1e-3
    avg = total_span / steps
    nbytes = sum(per_buf_bytes[i % len(bufs)] for i in range(steps)) / steps
    gbs = nbytes / avg / 1e9
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(total_span / steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "cache_len": n, "k": w["k"], "calib_sequences": w["calib"], "vmc": True,
                   "kv_buffers_rotated": len(bufs), "launch": "eager" if eager else "hip_graph",
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "kept_over_k": round(float(np.mean(kept_ratio)), 4),
        "vrows_per_group": round(float(np.mean(union_rows)), 1),
        "bytes_read_per_step": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_bf16_kernel", "avg_kernel_us": round(avg * 1e6, 3)},
        "wall_s": round(wall, 4),
    }
    if with_cpu:
        log("[bench] timing the CPU oracle on a sample of the same workload")
        res["cpu_baseline"] = oracle_decode_baseline(bufs[0], lens, theta, vms[0], w, read_bytes)
    return res


def copy_probe(dev, mib=512):
    """One plain elementwise kernel of known traffic (reads and writes `mib` MiB),
    used to scale hardware byte counters."""
    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_8b", choices=sorted(DECODE_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python instead of "
                    "replaying a captured HIP graph")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one elementwise kernel of known size (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                          "(multi-GPU sharding is described, not implemented)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    tt.load_library()
    res = bench_decode(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu_baseline,
                       eager=args.eager)
    if args.copy_probe:
        copy_probe(torch.device("cuda:0"))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
