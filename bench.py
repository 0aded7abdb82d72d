"""Decode-step weight-stream benchmark on one MI355X.

One step = one pass of the single-token weight stream of the 4.5-bpw GEMV
workload: y_up = W_up x_up (Q45, 12288 x 4096) and y_down = W_down x_down
(Q65, 4096 x 12288), M = 1.  Weights rotate over >= 1 GiB of identical
copies at distinct addresses, so no step can be served from the 256 MB
Infinity Cache.  The launches of one pass over all copies are captured in a
HIP graph and replayed, so host launch overhead stays out of the GPU timing.
`value` is algorithmic bytes of the step / step time.

Also measured in the same run and reported beside the headline:
  * per-kernel average durations (HIP events on the launch stream);
  * microseconds per 4096-wide RMSNorm row (one row per launch);
  * the memory ceiling measured by a 4 GiB read probe;
  * the CPU oracle on a bounded sample of the same step (cpu_baseline),
    which also checks the GPU result on that sample before it is reported.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for M=1 4.5-bpw GEMV; µs per 4096 RMSNorm row"
PEAK_HBM_GBS = 8000.0           # MI355X published HBM3E bandwidth
ROTATION_BYTES = 1 << 30        # >= 4x the 256 MB Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_m1.json")
KERNEL_SOURCES = ["formats.h", "gemv_m1.hip", "device_common.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "memory_bound_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemv_bytes(W) -> int:
    """Algorithmic bytes of one M=1 product: every weight byte once, x, y."""
    return W.nbytes + 4 * W.K + 4 * W.N


def traffic_for(kernel_key: str):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = t.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, y_up_gpu, y_down_gpu, budget_s: float = 12.0):
    """The oracle on a bounded sample of the step, on the host cores."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    fmt_u, N_u, K_u, p_u = cfg["up"]
    fmt_d, N_d, K_d, p_d = cfg["down"]
    Wu = oracle.Planes(fmt_u, N_u, K_u, p_u)
    Wd = oracle.Planes(fmt_d, N_d, K_d, p_d)
    # sample: the first 1/8 of each table's rows, one pass each
    ru, rd = N_u // 8, N_d // 8
    import concurrent.futures as cf
    L = oracle.lib()

    def rows_job(W, x, y, r0, r1):
        L.oracle_gemv(W.fmt, W.cptr, W.N, W.K, x.ctypes.data, 1, W.K, y.ctypes.data, W.N, 0, r0, r1)

    xu = np.ascontiguousarray(cfg["x_up"], np.float32)
    xd = np.ascontiguousarray(cfg["x_down"], np.float32)
    yu = np.zeros(N_u, np.float32)
    yd = np.zeros(N_d, np.float32)
    reps, t_total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            bu = np.linspace(0, ru, threads + 1).astype(int)
            bd = np.linspace(0, rd, threads + 1).astype(int)
            futs = [ex.submit(rows_job, Wu, xu, yu, int(bu[i]), int(bu[i + 1])) for i in range(threads)]
            futs += [ex.submit(rows_job, Wd, xd, yd, int(bd[i]), int(bd[i + 1])) for i in range(threads)]
            for f in futs:
                f.result()
        t_total += time.perf_counter() - t0
        reps += 1
        if t_total >= budget_s:
            break
    table_u = sum(p.nbytes for p in p_u if p is not None)
    table_d = sum(p.nbytes for p in p_d if p is not None)
    sample_bytes = table_u * ru // N_u + table_d * rd // N_d + 4 * (K_u + K_d + ru + rd)
    gbs = sample_bytes * reps / t_total / 1e9

    def rel(a, b):
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    err_u = rel(y_up_gpu[:ru], yu[:ru])
    err_d = rel(y_down_gpu[:rd], yd[:rd])
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "rows [0, N/8) of both tables (%d of %d Q45 rows, %d of %d Q65 rows), "
                      "%d passes in %.1f s, fp64 oracle, row-parallel over %d threads"
                      % (ru, N_u, rd, N_d, reps, t_total, threads),
            "checked_rel_l2": {"q45_up": err_u, "q65_down": err_d}}


COPY_BYTES = 1 << 29            # plain copy of known size that calibrates the counters


def kernel_key(name: str):
    """Which GEMV of the step a counter row belongs to (by format argument)."""
    if "gemv_m1_kernel<1," in name:
        return "q45_up_12288x4096"
    if "gemv_m1_kernel<2," in name:
        return "q65_down_4096x12288"
    if "probe_copy_kernel" in name:
        return "copy"
    return None


def traffic_pass():
    """Launches profiled by the counter runs: each GEMV once per rotated weight
    copy (cold, no graph) and one copy of COPY_BYTES bytes."""
    import torch
    import memory_bound_quantized_amd as mbq
    import workloads
    dev = torch.device("cuda:0")
    cfg = workloads.config2()
    W_up0 = mbq.QWeight.from_host(*cfg["up"])
    W_dn0 = mbq.QWeight.from_host(*cfg["down"])
    ncopy = max(2, -(-ROTATION_BYTES // (W_up0.nbytes + W_dn0.nbytes)))
    ups = [W_up0] + [W_up0.clone() for _ in range(ncopy - 1)]
    dns = [W_dn0] + [W_dn0.clone() for _ in range(ncopy - 1)]
    x_up = torch.from_numpy(cfg["x_up"]).to(dev)
    x_dn = torch.from_numpy(cfg["x_down"]).to(dev)
    y_up = torch.empty(W_up0.N, device=dev)
    y_dn = torch.empty(W_dn0.N, device=dev)
    for i in range(ncopy):
        mbq.gemv_q(ups[i], x_up, out=y_up)
        mbq.gemv_q(dns[i], x_dn, out=y_dn)
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    mbq.probe_copy(dst, src)
    torch.cuda.synchronize()
    print("traffic pass: %d launches of each GEMV, one %d-byte copy" % (ncopy, COPY_BYTES))


def write_traffic(fetch_dir: str, write_dir: str):
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run of
    traffic_pass (rocprofv3 --pmc, KiB per dispatch), each scaled by what
    the same counter reads for the copy of COPY_BYTES bytes."""
    import csv
    import glob

    def per_dispatch(d, counter):
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = kernel_key(r.get("Kernel_Name", ""))
                    if k is None or r["Counter_Name"] != counter:
                        continue
                    acc.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / fetch["copy"]
    w_scale = COPY_BYTES / write["copy"]
    out = {"kernel_source_hash": kernel_source_hash(),
           "copy_bytes": COPY_BYTES,
           "copy_counter_bytes": {"FETCH_SIZE": fetch["copy"], "WRITE_SIZE": write["copy"]},
           "scale": {"FETCH_SIZE": f_scale, "WRITE_SIZE": w_scale},
           "kernels": {}}
    for k in ("q45_up_12288x4096", "q65_down_4096x12288"):
        fb, wb = fetch[k] * f_scale, write[k] * w_scale
        out["kernels"][k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                             "hbm_bytes_per_launch": round(fb + wb)}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="only the launches that the counter runs profile")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs into the traffic file")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(every box has one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.traffic_pass:
        traffic_pass()
        return

    import torch
    import memory_bound_quantized_amd as mbq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    cfg = workloads.config2()
    fu, Nu, Ku, pu = cfg["up"]
    fd, Nd, Kd, pd = cfg["down"]
    W_up0 = mbq.QWeight.from_host(fu, Nu, Ku, pu)
    W_dn0 = mbq.QWeight.from_host(fd, Nd, Kd, pd)
    per_copy = W_up0.nbytes + W_dn0.nbytes
    ncopy = max(2, -(-ROTATION_BYTES // per_copy))
    ups = [W_up0] + [W_up0.clone() for _ in range(ncopy - 1)]
    dns = [W_dn0] + [W_dn0.clone() for _ in range(ncopy - 1)]
    x_up = torch.from_numpy(cfg["x_up"]).to(dev)
    x_dn = torch.from_numpy(cfg["x_down"]).to(dev)
    y_up = torch.empty(Nu, device=dev)
    y_dn = torch.empty(Nd, device=dev)

    def capture(fn):
        """A HIP graph of fn's launches (one pass over every weight copy)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()                       # first run outside capture (lazy init)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def pass_step():
        for i in range(ncopy):
            mbq.gemv_q(ups[i], x_up, out=y_up)
            mbq.gemv_q(dns[i], x_dn, out=y_dn)

    def pass_up():
        for i in range(ncopy):
            mbq.gemv_q(ups[i], x_up, out=y_up)

    def pass_dn():
        for i in range(ncopy):
            mbq.gemv_q(dns[i], x_dn, out=y_dn)

    g_step, g_up, g_dn = capture(pass_step), capture(pass_up), capture(pass_dn)
    reps = max(1, -(-args.steps // ncopy))          # graph replays in the timed region
    steps = reps * ncopy
    warm_reps = max(1, -(-args.warmup // ncopy))
    for _ in range(warm_reps):
        g_step.replay()
    torch.cuda.synchronize()
    y_up_first = y_up.cpu().numpy().copy()
    y_dn_first = y_dn.cpu().numpy().copy()

    def timed(graph, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    # timed region: `steps` steps = reps replays of the whole-step graph
    total_ms = timed(g_step, reps)
    ms_per_step = total_ms / steps
    # per-kernel averages: graphs of one kernel kind, same rotation
    up_ms = timed(g_up, reps) / steps
    dn_ms = timed(g_dn, reps) / steps
    b_up, b_dn = gemv_bytes(W_up0), gemv_bytes(W_dn0)
    value = (b_up + b_dn) / (ms_per_step * 1e-3) / 1e9

    # RMSNorm of one 4096-wide row (the metric's second part), one row per launch
    c1 = workloads.config1()
    xr = torch.from_numpy(c1["x"]).to(dev)
    gr = torch.from_numpy(c1["gamma"]).to(dev)
    yr = torch.empty_like(xr)
    nrm = 64

    def pass_norm():
        for _ in range(nrm):
            mbq.rmsnorm(xr, gr, c1["eps"], out=yr)

    g_norm = capture(pass_norm)
    g_norm.replay()
    rms_us = timed(g_norm, 20) / (20 * nrm) * 1e3

    # measured memory ceiling: 4 GiB read, best of 5
    buf = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, device=dev)
    mbq.probe_read(buf, sink, stream)
    best = 0.0
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        mbq.probe_read(buf, sink, stream)
        b.record(stream)
        torch.cuda.synchronize()
        best = max(best, buf.numel() / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf

    kern = {"q45_up_12288x4096": (b_up, up_ms), "q65_down_4096x12288": (b_dn, dn_ms)}
    dom = max(kern, key=lambda k: kern[k][1])
    d_bytes, d_ms = kern[dom]
    achieved = d_bytes / (d_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dom), "algorithmic_bytes_per_launch": d_bytes,
                "avg_launch_us": round(d_ms * 1e3, 3)}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warm_reps * ncopy, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "M=1 GEMV: Q45 12288x4096 (4.5 bpw) + Q65 4096x12288 (6.5625 bpw), "
                               "fp32 x and accumulation, weights rotated over %d copies (%.2f GB)"
                               % (ncopy, ncopy * per_copy / 1e9),
                   "global_batch": 1, "seq_len": 1, "parallelism": "none"},
        "roofline": roofline,
        "kernels": {k: {"avg_us": round(v[1] * 1e3, 3), "gbs": round(v[0] / (v[1] * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(v[0] / (v[1] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                    for k, v in kern.items()},
        "rmsnorm_us_per_4096_row": round(rms_us, 3),
        "measured_read_peak_gbs": round(best, 1),
        "q45_frac_of_measured_peak": round(b_up / (up_ms * 1e-3) / 1e9 / best, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, y_up_first, y_dn_first)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
