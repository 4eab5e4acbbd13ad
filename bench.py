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

The default run (``--workload all``) prints the decode_8b line with every
other workload below as a sub-object of ``workloads``, each with its own
roofline and CPU-oracle baseline, and a single-core oracle timing of decode_8b.

Other workloads (``--workload``):
  * ``decode_70b_32k``: batch 8, 64/8 heads, 32768 cached keys, 4 sink keys, k=256.
  * ``prefill_8k``: causal prefill of 4 layers (32/8 heads, d=128, L=8192, bf16;
    k=512 for layers 0-1, k=128 for layers 2-3; SDC, no VMC).  A step is one
    ``topth_prefill`` per layer; reported in TFLOP/s (algorithmic: one causal
    QK^T plus the kept P V; executed MFMA work alongside).
  * ``calib_sweep``: Algorithm-1 calibration of 8 heads, d=128, L=2048, k in
    {64, 128, 256}, 512 sequences per layer; a slice of layers is timed and
    the 32-layer sweep extrapolated.
  * ``prefill_8k_pre``: the prefill workload in the pre-softmax form (thresholds
    on the scores, calibrated on the scores; exp-threshold estimate of the
    discarded mass, gamma = 0.05): one sweep over the keys per query tile.
  * ``tiny_prefill_f32``: 1 head, d=64, L=256, fp32: calibration (k=32) from 64
    sequences, then prefill of 8 test sequences with SDC + VMC (latency-bound).
  * ``mkc``: multi-k cumulative calibration (Appendix D) over the decode_8b
    calibration set (256 sequences, 32/8 heads, 4096 keys, row 4095).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import re
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
from synth import (CONFIG_IDS, ROLE_CALIB, ROLE_TEST, attention_inputs, attention_inputs_device,  # noqa: E402
                   batch_of_sequences, to_f64)

METRIC = "decode Top-θ attn: HBM GB/s on bytes read (% of peak); prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

DECODE_WORKLOADS = {
    "decode_8b": dict(B=16, Hq=32, Hkv=8, d=128, n=4096, k=128, calib=256, sinks=1, buffers=3),
    "decode_70b_32k": dict(B=8, Hq=64, Hkv=8, d=128, n=32768, k=256, calib=256, sinks=4, buffers=2,
                           buckets=[("<512", 256, 511), ("512-2048", 512, 2047), ("2048-8192", 2048, 8191),
                                    (">8192", 8192, 32767)]),
}
PROBES_PER_BUCKET = 8


PREFILL_WORKLOAD = dict(B=1, Hq=32, Hkv=8, d=128, L=8192, ks=[512, 512, 128, 128], calib=64,
                        sinks=1)
CALIB_WORKLOAD = dict(layers=32, Hq=8, Hkv=8, d=128, L=2048, seqs=512, ks=[64, 128, 256], sinks=1,
                      chunk=64, timed_layers=2)
EXP_PEAK_PER_S = 256 * 4 * 16 / 4 * 2.4e9   # v_exp_f32: quarter-rate on 16-lane SIMDs
PRE_GAMMA = 0.05                            # exp-threshold estimate of the discarded mass


def code_sha256(sources):
    """SHA-256 of the device code in `sources` (a .hip file up to its host-side
    section) with comments and whitespace removed, so that edits to comments or
    to host code alone do not mark counter data as stale."""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        if f.endswith(".hip"):
            text = text.split("// ------------------------------------------------------------------ host side")[0]
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()


def measured_traffic(kernel, workload, sources):
    """HBM bytes per launch from the committed counter summary of `kernel` on
    `workload` (FETCH_SIZE + WRITE_SIZE, each scaled by a copy kernel of known
    size), or None when there is none or `sources` changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip().split()[0] if val.strip() else ""
    if fields.get("source_sha256") != code_sha256(sources) or "traffic_bytes_per_dispatch" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_dispatch"]))


DECODE_SOURCES = ["calibrated_threshold_pruning_amd/csrc/decode.hip",
                  "calibrated_threshold_pruning_amd/csrc/topth_internal.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def probe_rows(w):
    """Query positions p at which theta is calibrated and k~/k is reported: 8
    log-spaced rows per bucket (all with p + 1 > k), by bucket name."""
    out = {}
    for name, lo, hi in w.get("buckets", []):
        rows = np.unique(np.round(np.geomspace(max(lo, w["k"]), hi, PROBES_PER_BUCKET)).astype(int))
        out[name] = [int(r) for r in rows]
    return out


def calibrate_decode_theta(name, w, dev, rows=(), include_last=True, with_count=False):
    """theta [Hq, n] for k from `calib` decode-style sequences, on the GPU.  Row
    n - 1 (the timed decode step, unless `include_last` is False) and every row
    in `rows` are calibrated, each with its own query draw; other rows copy the
    nearest calibrated row.  With `with_count`, also the [1, Hq, n] counts."""
    cfg = CONFIG_IDS[name]
    Hq, Hkv, d, n, k = w["Hq"], w["Hkv"], w["d"], w["n"], w["k"]
    rows = sorted(set(int(r) for r in rows) | ({n - 1} if include_last else set()))
    s1 = torch.zeros(1, Hq, n, dtype=torch.float64, device=dev)
    s2 = torch.zeros_like(s1)
    cnt = torch.zeros(1, Hq, n, dtype=torch.int32, device=dev)
    chunk = max(1, min(32, (1 << 29) // (Hkv * n * d * 2)))
    ws = tt.workspace(tt.TOPTH_OP_CALIBRATE, chunk, Hq, Hkv, 1, n, d, 1)
    done = 0
    while done < w["calib"]:
        S = min(chunk, w["calib"] - done)
        q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, 0, done, B=S, Hq=Hq, Hkv=Hkv, Lq=len(rows), Lk=n,
                                           d=d, n_sinks=w["sinks"], device=dev, with_v=False)
        for i, p in enumerate(rows):
            tt.topth_calibrate(q[:, :, i:i + 1].contiguous(), kk, [k], s1, s2, cnt, ws,
                               scale=1.0 / math.sqrt(d), q_pos0=p)
        done += S
    theta = torch.empty(1, Hq, n, dtype=torch.float32, device=dev)
    tt.topth_calibrate_finalize(s1, s2, cnt, [k], theta)
    torch.cuda.synchronize()
    if with_count:
        return theta[0].contiguous(), cnt
    return theta[0].contiguous()


def theta_extrapolation(name, w, dev, buckets, buf, limit=2048):
    """k~/k on rows past the calibrated range: theta calibrated only at the
    probe rows below `limit`, then applied at the longer probe rows either as
    the nearest calibrated row or as a least-squares fit of ln(theta) in
    ln(p + 1) (degree 1 and 2), next to theta calibrated at the rows themselves."""
    short = [p for rows in buckets.values() for p in rows if p < limit]
    theta_near, cnt = calibrate_decode_theta(name, w, dev, rows=short, include_last=False, with_count=True)
    far = {b: rows for b, rows in buckets.items() if min(rows) >= limit}
    out = {"calibrated_rows": f"{len(short)} probe rows below {limit}",
           "nearest": kept_by_bucket(far, buf, theta_near, w, dev)}
    # near p + 1 = k the k-th largest is close to the row minimum, so theta first
    # rises with the row length before it falls: fits over all calibrated rows,
    # and fits over the rows with p + 1 >= 4 k only
    for label, min_len, deg in (("fitted_log_degree1_all_rows", 0, 1), ("fitted_log_degree2_all_rows", 0, 2),
                                ("fitted_log_degree1_rows_from_4k", 4, 1)):
        coef = torch.empty(1, w["Hq"], deg + 1, dtype=torch.float64, device=dev)
        tt.topth_theta_fit(theta_near[None].contiguous(), cnt, coef, [w["k"]], degree=deg, log_domain=True,
                           min_len_over_k=min_len)
        fitted = torch.empty(1, w["Hq"], w["n"], dtype=torch.float32, device=dev)
        tt.topth_theta_eval(coef, [w["k"]], fitted, log_domain=True)
        out[label] = kept_by_bucket(far, buf, fitted[0].contiguous(), w, dev)
    return out


def kept_by_bucket(buckets, buf, theta, w, dev):
    """Mean k~/k of decode steps at the probe rows of each bucket (seq_len = p + 1,
    same caches, VMC on)."""
    q, kk, v = buf
    B, Hq, Hkv, d = w["B"], w["Hq"], w["Hkv"], w["d"]
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    vm = torch.empty(B, Hkv, d, dtype=torch.float32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, w["n"], d)
    res = {}
    for name, rows in buckets.items():
        ratios = []
        for p in rows:
            lens = torch.full((B,), p + 1, dtype=torch.int32, device=dev)
            tt.topth_vmean(v, lens, vm)
            tt.topth_decode(q, kk, v, lens, theta, out, ws, scale=1.0 / math.sqrt(d), flags=tt.TOPTH_VMC,
                            v_mean=vm, kept_count=kc)
            ratios.append(kc.double().mean().item() / w["k"])
        res[name] = {"kept_over_k": round(float(np.mean(ratios)), 4), "rows": rows}
    return res


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


def single_thread():
    """Context in which NumPy's BLAS uses one thread (the single-core oracle)."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def oracle_decode_baseline(bufs, lens, theta, vm, w, bytes_of, budget_s=20.0, threads=None):
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
    model, threads_used = cpu_info()
    if threads is not None:
        threads_used = threads
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": threads_used,
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
    buckets = probe_rows(w)
    log(f"[bench] {name}: calibrating theta from {w['calib']} sequences"
        + (f" at row {n - 1} and {sum(len(r) for r in buckets.values())} probe rows" if buckets else ""))
    theta = calibrate_decode_theta(name, w, dev, rows=[p for r in buckets.values() for p in r])
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
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_bf16_kernel", name, DECODE_SOURCES),
                     "traffic_unit": "bytes per launch (HBM, counters)",
                     "algorithmic_bytes_per_launch": int(nbytes),
                     "kernel": "decode_bf16_kernel", "avg_kernel_us": round(avg * 1e6, 3)},
        "wall_s": round(wall, 4),
    }
    log("[bench] library streaming reference over the same K caches")
    res["stream_reference"] = stream_reference([buf[1] for buf in bufs])
    if name == "decode_8b":
        log("[bench] GQA selection variants on the same caches")
        res["gqa_variants"] = gqa_variants(bufs, vms, lens_d, theta, w, dev, read_bytes, steps=min(steps, 100))
        log("[bench] decode-serving helpers: running V mean and fitted theta")
        res["serving_helpers"] = serving_helpers(bufs, vms, lens_d, theta, w, dev, steps=min(steps, 100))
    if buckets:
        log("[bench] k~/k at the probe rows of each bucket")
        res["kept_over_k_by_row_bucket"] = kept_by_bucket(buckets, bufs[0], theta, w, dev)
        log("[bench] k~/k past the calibrated rows: nearest row against a fitted theta(n)")
        res["theta_extrapolation"] = theta_extrapolation(name, w, dev, buckets, bufs[0])
    if with_cpu:
        log("[bench] timing the CPU oracle on a sample of the same workload")
        res["cpu_baseline"] = oracle_decode_baseline(bufs[0], lens, theta, vms[0], w, read_bytes)
        if name == "decode_8b":
            log("[bench] timing the CPU oracle on one core")
            with single_thread():
                res["cpu_baseline_1core"] = oracle_decode_baseline(bufs[0], lens, theta, vms[0], w, read_bytes,
                                                                   threads=1)
    return res


def stream_reference(ks, steps=30):
    """Context for the decode line: what plain library kernels reach on the same
    K caches (rotated like the decode steps, so the MALL does not hold them):
    a reduction that reads each cache once, and a copy that reads and writes it."""
    nb = ks[0].numel() * ks[0].element_size()
    ops = (("read_GBps", lambda t: torch.sum(t, dtype=torch.float32), 1),
           ("copy_GBps_read_plus_write", lambda t: t.clone(), 2))
    res = {"ops": "torch.sum(K, dtype=float32); K.clone()", "bytes_per_cache": int(nb)}
    for key, fn, factor in ops:
        for t in ks:
            fn(t)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            fn(ks[i % len(ks)])
        b.record()
        torch.cuda.synchronize()
        res[key] = round(factor * nb * steps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    return res


def gqa_variants(bufs, vms, lens_d, theta, w, dev, read_bytes, steps):
    """V rows loaded per group, mean kept keys per head and step time of the
    GQA selection variants (keys kept by at least m heads; every head using
    all loaded keys), each over `steps` graph-replayed steps on the same
    rotating caches; bytes counted as for the plain decode step."""
    B, Hq, Hkv, d, n = w["B"], w["Hq"], w["Hkv"], w["d"], w["n"]
    g = Hq // Hkv
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    vr = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, n, d)
    res = {}
    for label, m, aug in (("min_votes_2", 2, False), ("min_votes_g", g, False), ("augment_union", 1, True),
                          ("augment_min_votes_2", 2, True)):
        def step(i):
            q, kk, v = bufs[i % len(bufs)]
            tt.topth_decode_gqa(q, kk, v, lens_d, theta, out, ws, scale=1.0 / math.sqrt(d), flags=tt.TOPTH_VMC,
                                min_votes=m, augment=aug, v_mean=vms[i % len(bufs)], kept_count=kc,
                                vrows_read=vr)
        nb, kept, rows = [], [], []
        for i in range(len(bufs)):
            step(i)
            torch.cuda.synchronize()
            nb.append(read_bytes(B, vr.sum().item()))
            kept.append(kc.float().mean().item() / w["k"])
            rows.append(vr.float().mean().item())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        avg = start.elapsed_time(end) * 1e-3 / steps
        nbytes = sum(nb[i % len(bufs)] for i in range(steps)) / steps
        res[label] = {"vrows_per_group": round(float(np.mean(rows)), 1),
                      "kept_over_k": round(float(np.mean(kept)), 4),
                      "us_per_step": round(avg * 1e6, 2), "GB_per_s": round(nbytes / avg / 1e9, 1)}
    status = int(ws[:4].view(torch.int32)[0].item())
    if status != 0:
        raise RuntimeError(f"decode exchange wait timed out (status {status})")
    return res


def replay_us(step, steps):
    """Average µs per step of `steps` calls captured into one HIP graph (after
    one untimed replay), from HIP events on the replay stream."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps


def serving_helpers(bufs, vms, lens_d, theta, w, dev, steps):
    """Per-token cost of the decode-serving helpers at the decode shape: the
    running V mean after appending one row per sequence, alone, followed by the
    decode step that uses it, and fused into that step (topth_decode_append);
    and evaluating a fitted theta(n) (one k, degree 1 in ln(p + 1), log domain)
    for every row of the cache.  The means are updated in copies, so the
    benchmark's own v_mean stays as it was."""
    B, Hq, Hkv, d, n = w["B"], w["Hq"], w["Hkv"], w["d"], w["n"]
    old = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
    mus = [vm.clone() for vm in vms]
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, n, d)

    def append(i):
        tt.topth_vmean_append(bufs[i % len(bufs)][2], old, lens_d, mus[i % len(bufs)])

    def append_and_decode(i):
        append(i)
        q, kk, v = bufs[i % len(bufs)]
        tt.topth_decode(q, kk, v, lens_d, theta, out, ws, scale=1.0 / math.sqrt(d), flags=tt.TOPTH_VMC,
                        v_mean=mus[i % len(bufs)])

    def decode_append(i):
        q, kk, v = bufs[i % len(bufs)]
        tt.topth_decode_append(q, kk, v, lens_d, theta, out, ws, mus[i % len(bufs)], scale=1.0 / math.sqrt(d),
                               flags=tt.TOPTH_VMC)

    coef = torch.tensor([[[-1.0, math.log(0.5)]] * Hq], dtype=torch.float64, device=dev)
    th_out = torch.empty(1, Hq, n, dtype=torch.float32, device=dev)

    def evaluate(i):
        tt.topth_theta_eval(coef, [w["k"]], th_out, log_domain=True)

    res = {"vmean_append_us": round(replay_us(append, steps), 2),
           "decode_step_with_vmean_append_us": round(replay_us(append_and_decode, steps), 2),
           "decode_append_fused_us": round(replay_us(decode_append, steps), 2),
           "theta_eval_all_rows_us": round(replay_us(evaluate, steps), 2),
           "vmean_append_bytes": B * Hkv * d * 2 + 2 * B * Hkv * d * 4}
    status = int(ws[:4].view(torch.int32)[0].item())
    if status != 0:
        raise RuntimeError(f"decode exchange wait timed out (status {status})")
    return res


def calibrate_prefill_theta(w, layer, k, dev, pre=False):
    """theta [Hq, L] for one layer from `calib` prefill-style sequences (GPU);
    with `pre`, thresholds on the scores and also the offline E~ table."""
    cfg = CONFIG_IDS["prefill_8k"]
    Hq, Hkv, d, L = w["Hq"], w["Hkv"], w["d"], w["L"]
    s1 = torch.zeros(1, Hq, L, dtype=torch.float64, device=dev)
    s2 = torch.zeros_like(s1)
    es = torch.zeros_like(s1)
    cnt = torch.zeros(1, Hq, L, dtype=torch.int32, device=dev)
    chunk = 8
    op = tt.TOPTH_OP_CALIBRATE_PRE_E if pre else tt.TOPTH_OP_CALIBRATE
    ws = tt.workspace(op, chunk, Hq, Hkv, L, L, d, 1)
    for done in range(0, w["calib"], chunk):
        S = min(chunk, w["calib"] - done)
        q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, layer, done, B=S, Hq=Hq, Hkv=Hkv, Lq=L,
                                           Lk=L, d=d, n_sinks=w["sinks"], device=dev, with_v=False)
        if pre:
            tt.topth_calibrate_pre(q, kk, [k], s1, s2, cnt, ws, scale=1.0 / math.sqrt(d), q_pos0=0, esum=es)
        else:
            tt.topth_calibrate(q, kk, [k], s1, s2, cnt, ws, scale=1.0 / math.sqrt(d), q_pos0=0)
        del q, kk
    theta = torch.empty(1, Hq, L, dtype=torch.float32, device=dev)
    tt.topth_calibrate_finalize(s1, s2, cnt, [k], theta)
    if not pre:
        torch.cuda.synchronize()
        return theta[0].contiguous()
    et = torch.empty_like(theta)
    tt.topth_calibrate_finalize_etilde(es, cnt, [k], et)
    torch.cuda.synchronize()
    return theta[0].contiguous(), et[0].contiguous()


def oracle_prefill_baseline(q, k, v, theta, w, budget_s=10.0, pre=False):
    """Time the CPU oracle on rows of layer 0, KV group 0 (its g query heads), spread
    over the whole length; report algorithmic TFLOP/s on the same flop count."""
    import oracle
    from oracle import presoftmax
    g = w["Hq"] // w["Hkv"]
    L, d = w["L"], w["d"]
    qf = to_f64(q[:1, :g].cpu()); kf = to_f64(k[:1, :1].cpu()); vf = to_f64(v[:1, :1].cpu())
    th = theta[:g].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(0)
    rows_all = rng.permutation(L)
    t0 = time.perf_counter()
    flops, done = 0.0, 0
    while time.perf_counter() - t0 < budget_s and done < L:
        ps = rows_all[done:done + 64]
        rows = [(0, h, int(p)) for h in range(g) for p in ps]
        if pre:
            r = presoftmax.prefill_pre(qf, kf, vf, th, 1.0 / math.sqrt(d), sdc="expth", vmc=False,
                                       gamma=PRE_GAMMA, rows=rows)
        else:
            r = oracle.prefill(qf, kf, vf, th, 1.0 / math.sqrt(d), vmc=False, rows=rows)
        for (_, h, p) in rows:
            flops += 2.0 * d * (p + 1) + 2.0 * d * r.kept_count[0, h, p]
        done += len(ps)
    el = time.perf_counter() - t0
    model, threads = cpu_info()
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 NumPy oracle {'pre-softmax ' if pre else ''}prefill of {done} random rows x {g} heads of layer 0 "
                      f"(KV group 0), {el:.1f} s, host '{model}', {os.cpu_count()} logical CPUs"}


def bench_prefill(steps, warmup, with_cpu, pre=False):
    name = "prefill_8k_pre" if pre else "prefill_8k"
    w = PREFILL_WORKLOAD
    dev = torch.device("cuda:0")
    cfg = CONFIG_IDS["prefill_8k"]
    B, Hq, Hkv, d, L = w["B"], w["Hq"], w["Hkv"], w["d"], w["L"]
    n_layers = len(w["ks"])
    scale = 1.0 / math.sqrt(d)
    layers = []
    for li, k in enumerate(w["ks"]):
        log(f"[bench] {name}: layer {li}: calibrating theta (k={k}) from {w['calib']} sequences")
        theta = calibrate_prefill_theta(w, li, k, dev, pre=pre)
        if pre:
            theta = theta[0]                # the exp-threshold estimate needs no E~ table
        q, kk, v = attention_inputs_device(cfg, ROLE_TEST, li, 0, B=B, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                                           n_sinks=w["sinks"], device=dev)
        out = torch.empty_like(q)
        kc = torch.empty(B, Hq, L, dtype=torch.int32, device=dev)
        layers.append(dict(k=k, theta=theta, q=q, kk=kk, v=v, out=out, kc=kc))
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, B, Hq, Hkv, L, L, d)

    def step():
        for lw in layers:
            if pre:
                tt.topth_prefill_pre(lw["q"], lw["kk"], lw["v"], lw["theta"], lw["out"], scale=scale,
                                     flags=tt.TOPTH_SDC_EXPTH, gamma=PRE_GAMMA, kept_count=lw["kc"], ws=ws)
            else:
                tt.topth_prefill(lw["q"], lw["kk"], lw["v"], lw["theta"], lw["out"], scale=scale, flags=0,
                                 kept_count=lw["kc"], ws=ws)

    step()
    torch.cuda.synchronize()
    causal = B * Hq * L * (L + 1) / 2                      # causal score elements per layer
    qk_flops = 2.0 * d * causal * n_layers
    kept = sum(float(lw["kc"].double().sum().item()) for lw in layers)
    pv_flops = 2.0 * d * kept
    per_layer = []
    for lw in layers:
        kc = lw["kc"][:, :, lw["k"]:].double()
        per_layer.append({"k": lw["k"], "kept_over_k": round(kc.mean().item() / lw["k"], 4),
                          "kept_p10_p50_p90": [round(x, 1) for x in
                                               torch.quantile(kc.flatten()[::97].float(),
                                                              torch.tensor([0.1, 0.5, 0.9], device=dev))
                                               .tolist()],
                          "elements_kept_frac": round(float(lw["kc"].double().sum().item()) / causal, 5)})
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = start.elapsed_time(end) * 1e-3
    t_step = span / steps
    algo = (qk_flops + pv_flops) / t_step / 1e12
    # executed MFMA work: QK^T in both sweeps (one in the pre-softmax form) plus
    # P V, one float16 product when every V element is within 16 in magnitude
    # (the library then takes that form, the workspace holding a float16 copy
    # of V), else two bf16 products (hi/lo split)
    f16_pv = all(float(lw["v"].abs().max().item()) <= 16.0 for lw in layers)
    executed = ((1.0 if pre else 2.0) + (1.0 if f16_pv else 2.0)) * qk_flops / t_step / 1e12
    res = {
        "metric": METRIC, "value": round(algo, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "seq_len": L, "layers": n_layers, "k_per_layer": w["ks"],
                   "calib_sequences": w["calib"], "threshold": "pre-softmax" if pre else "post-softmax",
                   "sdc": f"exp-threshold (gamma {PRE_GAMMA})" if pre else "exact", "vmc": False,
                   "parallelism": "single GPU"},
        "qk_tflops_algorithmic": round(qk_flops / t_step / 1e12, 2),
        "pv_form": "float16" if f16_pv else "bf16 high/low",
        "mfma_tflops_executed": round(executed, 2),
        "mfma_executed_frac_of_peak": round(executed / BF16_PEAK_TFLOPS, 4),
        "per_layer": per_layer,
        "roofline": {"bound": "mfma", "achieved": round(algo, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(algo / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_bf16_kernel",
                     "avg_kernel_us": round(t_step / n_layers * 1e6, 2)},
        "wall_s": round(wall, 4),
    }
    if with_cpu:
        log("[bench] timing the CPU oracle on a sample of the prefill workload")
        lw = layers[0]
        res["cpu_baseline"] = oracle_prefill_baseline(lw["q"], lw["kk"], lw["v"], lw["theta"], w, pre=pre)
    return res


def oracle_calib_baseline(w, dev, budget_s=10.0):
    """Time the CPU oracle's calibration (Algorithm 1: every row's k-th largest
    post-softmax value for each k) on whole sequences of layer 0, head after
    head, until the time budget is spent; report causal score elements per
    second."""
    import oracle
    cfg = CONFIG_IDS["calib_sweep"]
    L, d = w["L"], w["d"]
    t0 = time.perf_counter()
    elems, heads = 0, 0
    for seq in range(w["seqs"]):
        q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, 0, seq, B=1, Hq=w["Hq"], Hkv=w["Hkv"], Lq=L, Lk=L,
                                           d=d, n_sinks=w["sinks"], device=dev, with_v=False)
        qf = to_f64(q[0].cpu()); kf = to_f64(kk[0].cpu())
        for h in range(w["Hq"]):
            oracle.calibration_samples(qf[h:h + 1], kf[h:h + 1], w["ks"], 1.0 / math.sqrt(d), q_pos0=0)
            elems += L * (L + 1) // 2
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    model, threads = cpu_info()
    return {"value": round(elems / el, 1), "unit": "score elements/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 NumPy oracle calibration of {heads} (sequence, head) pairs of layer 0, all "
                      f"{L} rows each, {el:.1f} s, host '{model}'"}


def bench_calib(with_cpu):
    w = CALIB_WORKLOAD
    dev = torch.device("cuda:0")
    cfg = CONFIG_IDS["calib_sweep"]
    Hq, Hkv, d, L, ks = w["Hq"], w["Hkv"], w["d"], w["L"], w["ks"]
    n_k = len(ks)
    scale = 1.0 / math.sqrt(d)
    ws = tt.workspace(tt.TOPTH_OP_CALIBRATE, w["chunk"], Hq, Hkv, L, L, d, n_k)
    total_s, wall = 0.0, 0.0
    thetas = []
    # one untimed call first (kernel loading, LDS attributes)
    q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, 0, 0, B=w["chunk"], Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                                       n_sinks=w["sinks"], device=dev, with_v=False)
    s1 = torch.zeros(n_k, Hq, L, dtype=torch.float64, device=dev)
    tt.topth_calibrate(q, kk, ks, s1, torch.zeros_like(s1), torch.zeros(n_k, Hq, L, dtype=torch.int32, device=dev),
                       ws, scale=scale, q_pos0=0)
    torch.cuda.synchronize()
    del q, kk
    for layer in range(w["timed_layers"]):
        s1 = torch.zeros(n_k, Hq, L, dtype=torch.float64, device=dev)
        s2 = torch.zeros_like(s1)
        cnt = torch.zeros(n_k, Hq, L, dtype=torch.int32, device=dev)
        theta = torch.empty(n_k, Hq, L, dtype=torch.float32, device=dev)
        # every call's inputs resident in HBM first (about 4.3 GB per layer),
        # then the layer's calls and the finalize back to back in one timed region
        chunks = []
        for done in range(0, w["seqs"], w["chunk"]):
            S = min(w["chunk"], w["seqs"] - done)
            q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, layer, done, B=S, Hq=Hq, Hkv=Hkv, Lq=L,
                                               Lk=L, d=d, n_sinks=w["sinks"], device=dev, with_v=False)
            chunks.append((q, kk))
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        for q, kk in chunks:
            tt.topth_calibrate(q, kk, ks, s1, s2, cnt, ws, scale=scale, q_pos0=0)
        tt.topth_calibrate_finalize(s1, s2, cnt, ks, theta)
        b.record()
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
        total_s += a.elapsed_time(b) * 1e-3
        del chunks
        thetas.append(theta)
        log(f"[bench] calib_sweep: layer {layer} done ({total_s:.3f} s GPU so far)")
    seq_layers = w["seqs"] * w["timed_layers"]
    elems = seq_layers * Hq * L * (L + 1) / 2
    eps = elems / total_s
    qk = 2.0 * d * elems / total_s / 1e12
    full_s = total_s / w["timed_layers"] * w["layers"]
    fin = torch.isfinite(thetas[0])
    res = {
        "metric": METRIC, "value": round(eps / 1e9, 3), "unit": "G score elements/s", "n_gpus": 1,
        "steps": seq_layers, "warmup": 0, "ms_per_step": round(total_s / seq_layers * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "calib_sweep", "layers_total": w["layers"], "layers_timed": w["timed_layers"],
                   "heads": Hq, "head_dim": d, "seq_len": L, "sequences": w["seqs"], "ks": ks,
                   "parallelism": "single GPU"},
        "sequence_layers_per_s": round(seq_layers / total_s, 2),
        "full_sweep_s_extrapolated": round(full_s, 3),
        "theta_tensor_bytes_full_sweep": n_k * w["layers"] * Hq * L * 4,
        "theta_finite_frac_layer0": round(fin.float().mean().item(), 4),
        "roofline": {"bound": "alu", "achieved": round(eps / 1e12, 4), "peak": EXP_PEAK_PER_S / 1e12,
                     "unit": "T exp/s", "frac": round(eps / EXP_PEAK_PER_S, 4), "traffic": None,
                     "kernel": "calib_tiled_kernel",
                     "mfma_qk_tflops": round(qk, 2), "mfma_frac": round(qk / BF16_PEAK_TFLOPS, 4)},
        "wall_s": round(wall, 3),
    }
    if with_cpu:
        log("[bench] timing the CPU oracle on a sample of the calibration workload")
        res["cpu_baseline"] = oracle_calib_baseline(w, dev)
    return res


TINY_WORKLOAD = dict(L=256, d=64, k=32, calib=64, test=8)


def bench_tiny(steps, with_cpu):
    """The tiny fp32 workload end to end: calibration of theta (k=32) from 64
    sequences, finalize, then prefill of 8 test sequences with SDC + VMC; each
    step timed with events (the accumulators are zeroed before the event)."""
    w = TINY_WORKLOAD
    dev = torch.device("cuda:0")
    cfg = CONFIG_IDS["tiny_prefill_f32"]
    L, d, k = w["L"], w["d"], w["k"]
    qc, kc, _ = batch_of_sequences(cfg, ROLE_CALIB, 0, 0, w["calib"], Hq=1, Hkv=1, Lq=L, Lk=L, d=d,
                                   dtype=torch.float32)
    q, kk, v = attention_inputs(cfg, ROLE_TEST, 0, 0, B=w["test"], Hq=1, Hkv=1, Lq=L, Lk=L, d=d,
                                dtype=torch.float32)
    qc, kc, q, kk, v = (t.to(dev) for t in (qc, kc, q, kk, v))
    s1 = torch.zeros(1, 1, L, dtype=torch.float64, device=dev)
    s2, cnt = torch.zeros_like(s1), torch.zeros(1, 1, L, dtype=torch.int32, device=dev)
    theta = torch.empty(1, 1, L, dtype=torch.float32, device=dev)
    wsc = tt.workspace(tt.TOPTH_OP_CALIBRATE, w["calib"], 1, 1, L, L, d, 1)
    wsp = tt.workspace(tt.TOPTH_OP_PREFILL, w["test"], 1, 1, L, L, d)
    out = torch.empty_like(q)
    kcount = torch.empty(w["test"], 1, L, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(d)
    times = []
    for i in range(steps + 2):
        s1.zero_(); s2.zero_(); cnt.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tt.topth_calibrate(qc, kc, [k], s1, s2, cnt, wsc, scale=scale, q_pos0=0)
        tt.topth_calibrate_finalize(s1, s2, cnt, [k], theta)
        tt.topth_prefill(q, kk, v, theta[0], out, scale=scale, flags=tt.TOPTH_VMC, kept_count=kcount, ws=wsp)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(a.elapsed_time(b) * 1e-3)
    t = float(np.mean(times))
    seqs = w["calib"] + w["test"]
    res = {"value": round(seqs / t, 1), "unit": "sequences/s (64 calibrated + 8 prefilled)",
           "ms_per_step": round(t * 1e3, 4), "steps": steps, "dtype": "f32",
           "config": {"workload": "tiny_prefill_f32", "heads": 1, "head_dim": d, "seq_len": L, "k": k,
                      "calib_sequences": w["calib"], "test_sequences": w["test"], "sdc": "exact", "vmc": True},
           "kept_over_k": round(kcount[:, :, k:].double().mean().item() / k, 4),
           "roofline": None,
           "roofline_note": "latency-bound: 4.2 MFLOP of scores per sequence; no roofline claim"}
    if with_cpu:
        log("[bench] timing the full CPU oracle of the tiny workload (all cores, then one core)")
        qc64, kc64 = [to_f64(x.cpu()) for x in (qc, kc)]
        q64, k64, v64 = [to_f64(x.cpu()) for x in (q, kk, v)]

        def run_oracle():
            import oracle
            cal = oracle.Calibrator([k], 1, L)
            for c in range(w["calib"]):
                cal.observe(qc64[c], kc64[c], scale)
            oracle.prefill(q64, k64, v64, cal.finalize()[0], scale, vmc=True)

        def timed(budget_s=4.0):
            t0, n = time.perf_counter(), 0
            while True:
                run_oracle()
                n += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            return (time.perf_counter() - t0) / n, n

        model, threads = cpu_info()
        el, n = timed()
        res["cpu_baseline"] = {"value": round(seqs / el, 2), "unit": res["unit"], "cores": threads, "kind": "oracle",
                               "sample": f"the whole workload ({w['calib']} calibration + {w['test']} prefill "
                                         f"sequences), {n} pass(es), {el:.2f} s each, host '{model}'"}
        with single_thread():
            el, n = timed()
        res["cpu_baseline_1core"] = {"value": round(seqs / el, 2), "unit": res["unit"], "cores": 1, "kind": "oracle",
                                     "sample": f"the whole workload, one BLAS thread, {n} pass(es), {el:.2f} s each"}
    return res


MKC_WORKLOAD = dict(S=256, Hq=32, Hkv=8, d=128, n=4096, ks=[64, 128, 256])


def bench_mkc(with_cpu):
    """Multi-k cumulative calibration over the decode_8b calibration set: all 256
    sequences in one call (the merge needs every sample of a row at once),
    timed with events around five calls back to back."""
    w = MKC_WORKLOAD
    dev = torch.device("cuda:0")
    cfg = CONFIG_IDS["decode_8b"]
    S, Hq, Hkv, d, n = w["S"], w["Hq"], w["Hkv"], w["d"], w["n"]
    q, kk, _ = attention_inputs_device(cfg, ROLE_CALIB, 1, 0, B=S, Hq=Hq, Hkv=Hkv, Lq=1, Lk=n, d=d,
                                       n_sinks=1, device=dev, with_v=False)
    ws = torch.empty(tt.topth_workspace_size(tt.TOPTH_OP_CALIBRATE_MKC, S, Hq, Hkv, 1, n, d, 0), dtype=torch.uint8,
                     device=dev)
    theta = torch.empty(len(w["ks"]), Hq, n, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    tt.topth_calibrate_mkc(q, kk, w["ks"], theta, ws, scale=scale, q_pos0=n - 1)
    torch.cuda.synchronize()
    # five calls back to back between two events (every call recomputes the
    # same theta from the same inputs)
    reps = 5
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        tt.topth_calibrate_mkc(q, kk, w["ks"], theta, ws, scale=scale, q_pos0=n - 1)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    pooled = S * Hq * n
    # bytes the calibration must move at least: K of every sequence once, the
    # query rows, and the pooled values written and read once by the merge
    bytes_min = S * Hkv * n * d * 2 + S * Hq * d * 2 + 2 * pooled * 4
    res = {"value": round(pooled / t / 1e9, 4), "unit": "G pooled values/s",
           "ms_per_call": round(t * 1e3, 3), "dtype": "bf16",
           "config": {"workload": "mkc", "calib_sequences": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                      "cache_len": n, "row": n - 1, "ks": w["ks"]},
           "theta_row_4095": {str(k): round(float(theta[i, :, n - 1].mean().item()), 7) for i, k in enumerate(w["ks"])},
           "roofline": {"bound": "hbm", "achieved": round(bytes_min / t / 1e9, 2), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(bytes_min / t / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "whole call: mkc_values_bf16_kernel, the bound, compaction, radix sort and "
                                  "walk kernels",
                        "note": "the values kernel streams K once per KV head and counts the bound's first "
                                "histogram as it writes the pooled values; they are read twice more (the second "
                                "histogram, the compaction) and only those above the bound on theta are sorted, "
                                "which this minimum does not count"}}
    # thresholds for k = 128 from the merged function, applied to the decode_8b step
    wd = DECODE_WORKLOADS["decode_8b"]
    qt, kt, vt = attention_inputs_device(CONFIG_IDS["decode_8b"], ROLE_TEST, 0, 0, B=wd["B"], Hq=Hq, Hkv=Hkv, Lq=1,
                                         Lk=n, d=d, n_sinks=1, device=dev)
    qt = qt[:, :, 0].contiguous()
    lens = torch.full((wd["B"],), n, dtype=torch.int32, device=dev)
    vm = torch.empty(wd["B"], Hkv, d, dtype=torch.float32, device=dev)
    tt.topth_vmean(vt, lens, vm)
    out = torch.empty(wd["B"], Hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(wd["B"], Hq, dtype=torch.int32, device=dev)
    wsd = tt.workspace(tt.TOPTH_OP_DECODE, wd["B"], Hq, Hkv, 1, n, d)
    tt.topth_decode(qt, kt, vt, lens, theta[1].contiguous(), out, wsd, scale=scale, flags=tt.TOPTH_VMC, v_mean=vm,
                    kept_count=kc)
    torch.cuda.synchronize()
    res["kept_over_k_decode_8b_k128"] = round(kc.double().mean().item() / 128, 4)
    if with_cpu:
        log("[bench] timing the CPU oracle of MKC on one head")
        from oracle import mkc
        qf, kf = to_f64(q[:, :1].cpu()), to_f64(kk[:, :1].cpu())
        t0 = time.perf_counter()
        mkc.mkc_calibrate(qf, kf, scale, n - 1, w["ks"])
        el = time.perf_counter() - t0
        model, threads = cpu_info()
        res["cpu_baseline"] = {"value": round(S * n / el / 1e9, 6), "unit": res["unit"], "cores": threads,
                               "kind": "oracle",
                               "sample": f"float64 NumPy oracle of head 0 ({S} samples x {n} values), {el:.1f} s, "
                                         f"host '{model}'"}
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
    ap.add_argument("--workload", default="all",
                    choices=["all"] + sorted(DECODE_WORKLOADS) + ["prefill_8k", "prefill_8k_pre", "calib_sweep",
                                                                  "tiny_prefill_f32", "mkc"])
    ap.add_argument("--decode-only", action="store_true",
                    help="with --workload all: only the decode_8b line (no sub-workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python instead of "
                    "replaying a captured HIP graph")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one elementwise kernel of known size (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "topth runs on one GPU; --gpus must be 1 "
                          "(multi-GPU sharding is described, not implemented)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    tt.load_library()
    with_cpu = not args.no_cpu_baseline
    if args.workload in ("prefill_8k", "prefill_8k_pre"):
        res = bench_prefill(args.steps, args.warmup, with_cpu, pre=args.workload == "prefill_8k_pre")
    elif args.workload == "calib_sweep":
        res = bench_calib(with_cpu)
    elif args.workload == "tiny_prefill_f32":
        res = bench_tiny(args.steps, with_cpu)
    elif args.workload == "mkc":
        res = bench_mkc(with_cpu)
    elif args.workload == "all":
        res = bench_decode("decode_8b", args.steps, args.warmup, with_cpu=with_cpu, eager=args.eager)
        if not args.decode_only:
            keep = ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "wall_s")
            sub = {}
            log("[bench] decode_70b_32k")
            r = bench_decode("decode_70b_32k", min(args.steps, 100), args.warmup, with_cpu=with_cpu)
            sub["decode_70b_32k"] = {k: v for k, v in r.items() if k not in keep}
            for pre in (False, True):
                r = bench_prefill(steps=5, warmup=1, with_cpu=with_cpu, pre=pre)
                sub["prefill_8k_pre" if pre else "prefill_8k"] = {k: v for k, v in r.items() if k not in keep}
            log("[bench] calib_sweep")
            r = bench_calib(with_cpu)
            sub["calib_sweep"] = {k: v for k, v in r.items() if k not in keep}
            log("[bench] tiny_prefill_f32")
            sub["tiny_prefill_f32"] = bench_tiny(10, with_cpu)
            log("[bench] mkc")
            sub["mkc"] = bench_mkc(with_cpu)
            res["workloads"] = sub
    else:
        res = bench_decode(args.workload, args.steps, args.warmup, with_cpu=with_cpu, eager=args.eager)
    if args.copy_probe:
        copy_probe(torch.device("cuda:0"))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
