"""Decode-step benchmark on one MI355X.

Headline step = one pass of the single-token weight stream of the 4.5-bpw
GEMV workload: y_up = W_up x_up (Q45, 12288 x 4096) and y_down = W_down x_down
(Q65, 4096 x 12288), M = 1, fp32 x in and y out.  Weights rotate over >= 1 GiB
of identical copies at distinct addresses, so no launch can be served from the
256 MB Infinity Cache.  The launches of one pass over all copies are captured
in a HIP graph and replayed, so host launch overhead stays out of the GPU
timing.  `value` is algorithmic bytes of the step / step time.

Every other step of the hot path is measured in the same run, in the same way
(graph replays, cold weights), under "rows":
  * RMSNorm of one 4096 row (us per row) and the bf16 512 x 4096 product;
  * M = 1 products at each decode table shape, fused forms included;
  * small batches M = 1 .. 64 of the 12288 x 4096 Q45 table (the vector
    units below M = 4, the matrix cores from M = 4, staged x and fp32 x),
    the 512-token batch, and the 4096 x 12288 table with K whole and split;
  * 8 gathered Q25 experts of 1536 x 4096; LayerNorm of 4096 rows of 2048;
  * the quantizer into each format; decode attention at 512, 4096 and 32768
    positions;
  * one token through the 36-layer decode stream (ms per token, tokens/s,
    against the measured read ceiling) as a graph of launches, in one
    launch, and with attention over 512 cached positions in every layer.
Also: the measured ceilings (the larger of a 4 GiB read and a 2 GiB copy,
memory latency from a pointer chase, matrix and vector issue rates), and the
CPU oracle timed single-threaded and on every core on a bounded sample of the
headline step (cpu_baseline); that leg also checks the GPU's headline
products and its whole 36-layer decode token, with and without attention,
against the oracle, and the run fails instead of printing a line when they
disagree.

The timed region is exactly --steps steps (one replay of a graph of that
many steps) after --warmup untimed ones.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-rows] [--no-one-launch]
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
LEDGER_MIN_LAUNCHES = 1536      # launches per ledger window (about 28 ms of steps)
DEFAULT_PEAK_GBS = 6080.0  # the ceiling for --decode-only runs; a full run measures it live
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_m1.json")
KERNEL_SOURCES = ["formats.h", "gemv_m1.hip", "staging.h", "device_common.h"]


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


def host_cores():
    """Cores this process may run on, and the thread count the oracle legs
    use: the affinity set, capped by OMP_NUM_THREADS when the job sets it
    (the machine's CPU share)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    use = min(avail, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else avail
    return {"nproc": os.cpu_count(), "affinity": avail, "omp_num_threads": cap, "threads": use}


def cpu_baseline(cfg, y_up_gpu, y_down_gpu, decode=None, budget_s: float = 10.0):
    """The oracle on the host cores: a bounded sample of the headline step,
    timed single-threaded and row-parallel on every core the process has; and,
    when the decode row ran, the oracle's whole 36-layer token, which checks
    the GPU's token before its time is reported."""
    import concurrent.futures as cf
    import oracle
    cores = host_cores()
    threads = cores["threads"]
    fmt_u, N_u, K_u, p_u = cfg["up"]
    fmt_d, N_d, K_d, p_d = cfg["down"]
    Wu = oracle.Planes(fmt_u, N_u, K_u, p_u)
    Wd = oracle.Planes(fmt_d, N_d, K_d, p_d)
    # sample: the first 1/8 of each table's rows
    ru, rd = N_u // 8, N_d // 8
    L = oracle.lib()

    def rows_job(W, x, y, r0, r1):
        L.oracle_gemv(W.fmt, W.cptr, W.N, W.K, x.ctypes.data, 1, W.K, y.ctypes.data, W.N, 0, r0, r1)

    xu = np.ascontiguousarray(cfg["x_up"], np.float32)
    xd = np.ascontiguousarray(cfg["x_down"], np.float32)
    yu = np.zeros(N_u, np.float32)
    yd = np.zeros(N_d, np.float32)

    def leg(nthreads, budget):
        reps, t_total = 0, 0.0
        bu = np.linspace(0, ru, nthreads + 1).astype(int)
        bd = np.linspace(0, rd, nthreads + 1).astype(int)
        with cf.ThreadPoolExecutor(nthreads) as ex:
            while t_total < budget:
                t0 = time.perf_counter()
                futs = [ex.submit(rows_job, Wu, xu, yu, int(bu[i]), int(bu[i + 1])) for i in range(nthreads)]
                futs += [ex.submit(rows_job, Wd, xd, yd, int(bd[i]), int(bd[i + 1])) for i in range(nthreads)]
                for f in futs:
                    f.result()
                t_total += time.perf_counter() - t0
                reps += 1
        return reps, t_total

    table_u = sum(p.nbytes for p in p_u if p is not None)
    table_d = sum(p.nbytes for p in p_d if p is not None)
    sample_bytes = table_u * ru // N_u + table_d * rd // N_d + 4 * (K_u + K_d + ru + rd)
    reps1, t1 = leg(1, budget_s / 2)
    repsn, tn = leg(threads, budget_s)
    gbs1 = sample_bytes * reps1 / t1 / 1e9
    gbsn = sample_bytes * repsn / tn / 1e9

    def rel(a, b):
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    err_u = rel(y_up_gpu[:ru], yu[:ru])
    err_d = rel(y_down_gpu[:rd], yd[:rd])
    if max(err_u, err_d) > 1e-4:
        raise SystemExit("headline products disagree with the oracle: rel-L2 %.3e, %.3e" % (err_u, err_d))
    out = {"value": round(gbsn, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "rows [0, N/8) of both tables (%d of %d Q45 rows, %d of %d Q65 rows), "
                     "%d passes in %.1f s, fp64 oracle, row-parallel over %d threads"
                     % (ru, N_u, rd, N_d, repsn, tn, threads),
           "single_thread": {"value": round(gbs1, 4), "unit": "GB/s", "passes": reps1,
                             "seconds": round(t1, 2)},
           "host": cores,
           "checked_rel_l2": {"q45_up": err_u, "q65_down": err_d}}
    if decode is not None:
        # the whole token in the oracle (each product's rows over the threads)
        t0 = time.perf_counter()
        lay = [{k: oracle.Planes(*v) for k, v in e.items()} for e in decode["cfg"]["layers"]]
        c3 = decode["cfg"]
        h_ref, lg_ref = oracle.decode_token_parallel(lay, oracle.Planes(*c3["vocab"]), c3["g1"],
                                                     c3["g2"], c3["gf"], c3["eps"], c3["h0"],
                                                     threads=threads)
        t_tok = time.perf_counter() - t0
        errs = {}
        for name, (h, lg) in decode["outputs"].items():
            errs[name] = {"h": rel(h, h_ref), "logits": rel(lg, lg_ref)}
        out["decode_token"] = {"seconds_per_token": round(t_tok, 3), "threads": threads,
                               "checked_rel_l2": errs}
        bad = [n for n, e in errs.items() if max(e["h"], e["logits"]) > 1e-4]
        if bad:
            raise SystemExit("decode token disagrees with the oracle chain (%s): %s"
                             % (", ".join(bad), json.dumps(errs)))
        if "kv" in decode:
            # the token with attention over the cache (the oracle updates its
            # own copies of the caches' row T)
            kv = decode["kv"]
            t0 = time.perf_counter()
            kc = [c.copy() for c in kv["k"]]
            vc = [c.copy() for c in kv["v"]]
            h_ref, lg_ref = oracle.decode_token_kv(lay, oracle.Planes(*c3["vocab"]), c3["g1"], c3["g2"],
                                                   c3["gf"], c3["eps"], c3["h0"], kc, vc, kv["T"],
                                                   threads=threads)
            t_kv = time.perf_counter() - t0
            h, lg = kv["out"]
            e = {"h": rel(h, h_ref), "logits": rel(lg, lg_ref)}
            out["decode_token_with_attention_512"] = {"seconds_per_token": round(t_kv, 3),
                                                      "threads": threads, "checked_rel_l2": e}
            if max(e.values()) > 1e-4:
                raise SystemExit("decode token with attention disagrees with the oracle: %s" % json.dumps(e))
    return out


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


def mfma_pass(reps: int = 8, tokens=(16, 64)):
    """Launches profiled by the matrix-core counter run: the staged-x product
    of workload 4's 12288 x 4096 Q45 table at each batch size in tokens
    (16 and 64 by default), each on cold weights (one rotated copy per
    launch, no graph)."""
    import torch
    import memory_bound_quantized_amd as mbq
    import workloads
    dev = torch.device("cuda:0")
    for M in tokens:
        c4 = workloads.config4(M)
        W0 = mbq.QWeight.from_host(*c4["W"])
        Ws = rotated(W0)
        X = torch.from_numpy(c4["X"]).to(dev)
        Xq = mbq.stage_x(W0.fmt, X)
        Y = torch.empty((M, W0.N), device=dev)
        for i in range(reps):
            mbq.gemv_xq(Ws[i % len(Ws)], Xq, M=M, out=Y)
        torch.cuda.synchronize()
        del Ws
        torch.cuda.empty_cache()
    print("mfma pass: %d launches at each of M = %s" % (reps, ", ".join(str(m) for m in tokens)))


def rows_traffic_pass(reps: int = 4):
    """Launches profiled by the counter runs of the other rows: the BF16
    512 x 4096 product, the fused-norm qkv (Q45 6144 x 4096) and vocabulary
    (Q65 151936 x 4096) products, the gather of 8 Q25 experts, one RMSNorm
    row of 4096 and LayerNorm 4096 x 2048, each reps times on its own copy of
    the data (no graph), then one copy of COPY_BYTES bytes."""
    import torch
    import memory_bound_quantized_amd as mbq
    import workloads
    dev = torch.device("cuda:0")
    alg = {}
    c1 = workloads.config1()
    Ws = [mbq.QWeight.from_host(*c1["W"]) for _ in range(reps)]
    x = torch.from_numpy(c1["x"]).to(dev)
    y = torch.empty(Ws[0].N, device=dev)
    for W in Ws:
        mbq.gemv_q(W, x, out=y)
    alg["bf16_512x4096"] = Ws[0].nbytes + 4 * (Ws[0].N + Ws[0].K)
    del Ws
    rng = np.random.default_rng(77)
    for name, fmt, N, K in (("qkv_6144x4096_q45_norm", 1, 6144, 4096),
                            ("vocab_151936x4096_q65_norm", 2, 151936, 4096)):
        W0 = mbq.QWeight.from_host(fmt, N, K, workloads.weight_planes(rng, fmt, N, K))
        Ws = [W0] + [W0.clone() for _ in range(reps - 1)]
        x = torch.randn(K, device=dev)
        gam = torch.rand(K, device=dev) + 0.5
        y = torch.empty(N, device=dev)
        for W in Ws:
            mbq.gemv_fused(W, x, gam, 1e-6, out=y)
        alg[name] = W0.nbytes + 4 * (2 * K + N)
        del Ws, W0
        torch.cuda.empty_cache()
    c5 = workloads.config5()
    fmt, N, K, planes = c5["W"]
    Ws = [mbq.QWeight.from_host(fmt, N, K, planes) for _ in range(reps)]
    idx = torch.from_numpy(c5["idx"]).to(dev)
    x = torch.from_numpy(c5["x"]).to(dev)
    rpe, ns = c5["rows_per_expert"], len(c5["idx"])
    y = torch.empty((ns, rpe), device=dev)
    for W in Ws:
        mbq.gemv_q_gather(W, rpe, idx, x, out=y)
    alg["gather_8_of_64_q25_1536x4096"] = ns * Ws[0].nbytes // (N // rpe) + 4 * K + 4 * ns * rpe + 4 * ns
    del Ws
    xr = torch.from_numpy(c1["x"]).to(dev)
    gr = torch.from_numpy(c1["gamma"]).to(dev)
    yr = torch.empty_like(xr)
    for _ in range(reps):
        mbq.rmsnorm(xr, gr, c1["eps"], out=yr)
    alg["rmsnorm_4096"] = 3 * 4 * xr.numel()
    X = torch.from_numpy(c5["ln_x"]).to(dev)
    Xs = [X] + [X.clone() for _ in range(reps - 1)]
    gam = torch.from_numpy(c5["ln_gamma"]).to(dev)
    bet = torch.from_numpy(c5["ln_beta"]).to(dev)
    Yl = torch.empty_like(X)
    for Xi in Xs:
        mbq.layernorm(Xi, gam, bet, c5["ln_eps"], out=Yl)
    alg["layernorm_4096x2048"] = 2 * X.numel() * 4 + 2 * X.shape[1] * 4
    del Xs, X
    torch.cuda.empty_cache()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    mbq.probe_copy(dst, src)
    torch.cuda.synchronize()
    print("rows traffic pass: %d launches of each row, one %d-byte copy; algorithmic bytes per launch %s"
          % (reps, COPY_BYTES, json.dumps(alg)))


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


def capture(fn):
    """A HIP graph of fn's launches (fn is run once outside capture first)."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def upload(graph, stream):
    """hipGraphUpload of a captured graph's executable: the runtime's per-graph
    set-up done before a timed region instead of inside its first replay."""
    import ctypes
    import torch
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    rc = hip.hipGraphUpload(ctypes.c_void_p(graph.raw_cuda_graph_exec()),
                            ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("hipGraphUpload failed: %d" % rc)
    torch.cuda.synchronize()


def timed(graph, n, stream=None):
    """Milliseconds for n replays of graph, HIP events on the launch stream."""
    import torch
    stream = stream or torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def per_launch_us(make_launch, copies, launches_target=200, warm_ms=20.0):
    """Average us of one launch: a graph of one launch per weight copy, replayed
    after warm-up replays worth at least 16 launches and warm_ms of GPU time
    (a row measured right after seconds of host-side setup ran up to 13 %
    slower than the same launches a little later)."""
    g = capture(lambda: [make_launch(c) for c in copies])
    once = timed(g, 1)
    warm = max(2, -(-16 // len(copies)), int(warm_ms / max(once, 1e-3)) + 1)
    for _ in range(min(warm, 10000)):
        g.replay()
    reps = max(2, -(-launches_target // len(copies)))
    return timed(g, reps) / (reps * len(copies)) * 1e3


def rotated(W0, min_bytes=ROTATION_BYTES):
    n = max(2, -(-min_bytes // W0.nbytes))
    return [W0] + [W0.clone() for _ in range(n - 1)]


def decode_row(workloads, torch, dev, peak_gbs, ntok=20, one_launch=True, keep=None):
    """Workload 3: ms per token of the 36-layer step, one HIP graph per token,
    and the same token in one cooperative launch.  keep: a dict that receives
    the host inputs and each form's h and logits after one token from h0, for
    the oracle check in the CPU leg."""
    from memory_bound_quantized_amd.decode import DecodeModel
    c3 = workloads.config3()
    model = DecodeModel(c3["layers"], c3["vocab"], c3["g1"], c3["g2"], c3["gf"], c3["eps"])
    h0 = torch.from_numpy(c3["h0"]).to(dev)
    h = h0.clone()
    logits = torch.empty(model.vocab, device=dev)
    g = capture(lambda: model.step(h, logits))
    h.copy_(h0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    outputs = {"graph of launches": (h.cpu().numpy(), logits.cpu().numpy())}
    g.replay()
    ms = timed(g, ntok) / ntok
    B = model.weight_bytes + 4 * 36 * 2 * model.d + 4 * model.d
    B_all = B + 4 * (36 * (model.dq + 2 * model.dkv + model.f + 6 * model.d) + model.vocab)
    floor_ms = B / (peak_gbs * 1e9) * 1e3
    row = {"ms_per_token": round(ms, 4), "tokens_per_s": round(1e3 / ms, 1),
           "weight_bytes": model.weight_bytes, "bytes_per_token": int(B_all),
           "gbs": round(B_all / (ms * 1e-3) / 1e9, 1),
           "floor_ms_at_measured_peak": round(floor_ms, 4), "ratio_to_floor": round(ms / floor_ms, 3),
           "launches_per_token": 4 * 36 + 1, "tokens_timed": ntok}
    if one_launch:
        # the same token in one cooperative launch (not capturable: timed as
        # back-to-back launches between HIP events on the current stream)
        hp, lp = h0.clone(), torch.empty_like(logits)
        model.step_persistent(hp, lp)
        torch.cuda.synchronize()
        ok_first = model.status() == 0
        outputs["one launch"] = (hp.cpu().numpy(), lp.cpu().numpy())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(ntok):
            model.step_persistent(hp, lp)
        b.record()
        torch.cuda.synchronize()
        ms_p = a.elapsed_time(b) / ntok
        ok = ok_first and model.status() == 0
        if not ok:
            raise SystemExit("one-launch decode step reported status %d" % model.status())
        row["one_launch"] = {"ms_per_token": round(ms_p, 4), "ratio_to_floor": round(ms_p / floor_ms, 3),
                             "status_ok": ok}
    # the same token with attention over 512 cached positions in every layer
    # (mbq_decode_step_kv: the cache append fused into the attention's first
    # launch), captured in one graph; row 512 of each cache is rewritten with
    # the same values by every replay
    T = 512
    kh, vh = workloads.kv_caches(36, T + 1, model.dkv, seed=3000)
    kd = [torch.from_numpy(c.view(np.int16)).to(dev) for c in kh]
    vd = [torch.from_numpy(c.view(np.int16)).to(dev) for c in vh]
    ws = model.kv_workspace(T)
    hk, lk = h0.clone(), torch.empty_like(logits)
    gk = capture(lambda: model.step_kv(hk, lk, kd, vd, T, workspace=ws))
    hk.copy_(h0)
    torch.cuda.synchronize()
    gk.replay()
    torch.cuda.synchronize()
    kv_out = (hk.cpu().numpy(), lk.cpu().numpy())
    gk.replay()
    ms_kv = timed(gk, ntok) / ntok
    kv_read = 36 * 2 * T * model.dkv * 2                 # rows 0 .. 511 of K and V, every layer
    kv_write = 36 * 2 * model.dkv * 2                    # row 512
    Bk = B + kv_read + kv_write
    Bk_all = B_all + kv_read + kv_write + 4 * 36 * model.dq     # + the attention outputs
    floor_kv = Bk / (peak_gbs * 1e9) * 1e3
    row["with_attention_512"] = {
        "ms_per_token": round(ms_kv, 4), "tokens_per_s": round(1e3 / ms_kv, 1),
        "kv_bytes_per_token": kv_read + kv_write, "bytes_per_token": int(Bk_all),
        "gbs": round(Bk_all / (ms_kv * 1e-3) / 1e9, 1),
        "floor_ms_at_measured_peak": round(floor_kv, 4), "ratio_to_floor": round(ms_kv / floor_kv, 3),
        "attention_ms_per_token": round(ms_kv - ms, 4),
        "launches_per_token": 6 * 36 + 1, "tokens_timed": ntok}
    if keep is not None:
        keep["cfg"] = {k: v for k, v in c3.items()}
        keep["outputs"] = outputs
        keep["kv"] = {"T": T, "k": kh, "v": vh, "out": kv_out}
    del model, g, gk, kd, vd, ws
    torch.cuda.empty_cache()
    return row


def rows_bench(mbq, workloads, torch, dev, peak_gbs, one_launch=True, keep=None):
    """Every other step of the hot path, each on cold weights."""
    from memory_bound_quantized_amd.decode import DecodeModel, interleave_rows, concat_rows
    rows = {}
    gbs = lambda b, us: round(b / (us * 1e-6) / 1e9, 1)

    # ---- workload 1: RMSNorm row (below) and the bf16 512 x 4096 product
    c1 = workloads.config1()
    fmt, N, K, planes = c1["W"]
    Ws = rotated(mbq.QWeight.from_host(fmt, N, K, planes))
    x = torch.from_numpy(c1["x"]).to(dev)
    y = torch.empty(N, device=dev)
    us = per_launch_us(lambda W: mbq.gemv_q(W, x, out=y), Ws)
    b = Ws[0].nbytes + 4 * (N + K)
    rows["bf16_512x4096_m1"] = {"us": round(us, 3), "gbs": gbs(b, us), "bytes": b}
    del Ws

    # ---- M = 1 at the decode table shapes (fp32 x; fused forms as the decode step runs them)
    rng = np.random.default_rng(77)
    shapes = [("q_o_4096x4096_q45", 1, 4096, 4096, "plain"), ("k_v_1024x4096_q45", 1, 1024, 4096, "plain"),
              ("qkv_6144x4096_q45_norm", 1, 6144, 4096, "norm"),
              ("gate_up_24576x4096_q45_norm_silu", 1, 24576, 4096, "silu"),
              ("down_4096x12288_q65_acc", 2, 4096, 12288, "acc"), ("down_4096x12288_q45_acc", 1, 4096, 12288, "acc"),
              ("vocab_151936x4096_q65_norm", 2, 151936, 4096, "norm")]
    per_shape = {}
    for name, fmt, N, K, kind in shapes:
        W0 = mbq.QWeight.from_host(fmt, N, K, workloads.weight_planes(rng, fmt, N, K))
        Ws = rotated(W0)
        x = torch.randn(K, device=dev)
        gam = torch.rand(K, device=dev) + 0.5
        y = torch.zeros(N // 2 if kind == "silu" else N, device=dev)
        if kind == "plain":
            f = lambda W: mbq.gemv_q(W, x, out=y)
        elif kind == "acc":
            f = lambda W: mbq.gemv_q(W, x, out=y, accumulate=True)
        elif kind == "norm":
            f = lambda W: mbq.gemv_fused(W, x, gam, 1e-6, out=y)
        else:
            f = lambda W: mbq.gemv_fused(W, x, gam, 1e-6, mbq.EPI_SILU_MUL, out=y)
        us = per_launch_us(f, Ws)
        b = W0.nbytes + 4 * (K + (N // 2 if kind == "silu" else N)) + (4 * K if kind in ("norm", "silu") else 0) \
            + (4 * N if kind == "acc" else 0)
        per_shape[name] = {"us": round(us, 3), "gbs": gbs(b, us), "frac_of_measured_peak": round(b / (us * 1e-6) / 1e9 / peak_gbs, 4)}
        del Ws, W0
        torch.cuda.empty_cache()
    rows["m1_decode_shapes"] = per_shape

    # ---- small batches of the 12288 x 4096 Q45 table
    small = {}
    for M in (1, 2, 4, 6, 8, 16, 64):
        c4 = workloads.config4(M)
        fmt, N, K, planes = c4["W"]
        Ws = rotated(mbq.QWeight.from_host(fmt, N, K, planes))
        X = torch.from_numpy(c4["X"]).to(dev)
        Y = torch.empty((M, N) if M > 1 else (N,), device=dev)
        Xq = mbq.stage_x(fmt, X if M > 1 else X[0])
        kern_us = per_launch_us(lambda W: mbq.gemv_xq(W, Xq, M=M, out=Y), Ws)
        Xin = X if M > 1 else X[0]
        step_us = per_launch_us(lambda W: (mbq.stage_x(fmt, Xin, out=Xq), mbq.gemv_xq(W, Xq, M=M, out=Y)), Ws)
        fp32_us = per_launch_us(lambda W: mbq.gemv_q(W, Xin, out=Y), Ws)
        b = Ws[0].nbytes + 4 * M * (N + K)
        ent = {"stage_plus_product_us": round(step_us, 3), "product_us": round(kern_us, 3),
               "us_per_token": round(step_us / M, 3), "product_gbs": gbs(b, kern_us),
               "path": "matrix cores" if M >= 4 else "vector units",
               "fp32_x_path": "matrix cores, x converted in the product" if M >= 4 else "vector units"}
        if fp32_us is not None:
            ent["fp32_x_us"] = round(fp32_us, 3)
        if M >= 4:
            tf = 2.0 * M * N * K / (kern_us * 1e-6) / 1e12
            ent["useful_tflops"] = round(tf, 2)
            # issued: 16-token tiles, two fp16 MFMAs (x high and low parts) per
            # block, against the 2.5 PF/s fp16 peak
            issued = 16 * ((M + 15) // 16)
            ent["mfma_busy_frac_of_fp16_peak"] = round(2 * tf * issued / M / 2500.0, 4)
        small["M%d" % M] = ent
        del Ws
        torch.cuda.empty_cache()
    rows["small_batch_12288x4096_q45"] = small

    # ---- workload 5: 8 gathered Q25 experts, and LayerNorm 4096 x 2048
    c5 = workloads.config5()
    fmt, N, K, planes = c5["W"]
    Wall = mbq.QWeight.from_host(fmt, N, K, planes)
    Ws = rotated(Wall, 4 * ROTATION_BYTES)
    idx = torch.from_numpy(c5["idx"]).to(dev)
    x = torch.from_numpy(c5["x"]).to(dev)
    rpe = c5["rows_per_expert"]
    y = torch.empty((len(c5["idx"]), rpe), device=dev)
    us = per_launch_us(lambda W: mbq.gemv_q_gather(W, rpe, idx, x, out=y), Ws)
    b = len(c5["idx"]) * Wall.nbytes // (N // rpe) + 4 * K + 4 * len(c5["idx"]) * rpe + 4 * len(c5["idx"])
    rows["gather_8_of_64_q25_1536x4096"] = {"us": round(us, 3), "gbs": gbs(b, us), "bytes": b}
    del Ws, Wall
    X = torch.from_numpy(c5["ln_x"]).to(dev)
    gam = torch.from_numpy(c5["ln_gamma"]).to(dev)
    bet = torch.from_numpy(c5["ln_beta"]).to(dev)
    Xs = [X] + [X.clone() for _ in range(15)]
    Yl = torch.empty_like(X)
    us = per_launch_us(lambda Xi: mbq.layernorm(Xi, gam, bet, c5["ln_eps"], out=Yl), Xs)
    b = 2 * X.numel() * 4 + 2 * X.shape[1] * 4
    rows["layernorm_4096x2048"] = {"us": round(us, 3), "gbs": gbs(b, us), "bytes": b}
    del Xs, X
    torch.cuda.empty_cache()

    # ---- prefill-sized batch: 512 tokens of the 12288 x 4096 Q45 table on
    # the matrix cores (staged x), and the separate staging launch
    M = 512
    c4 = workloads.config4(16)
    fmt, N, K, planes = c4["W"]
    W0 = mbq.QWeight.from_host(fmt, N, K, planes)
    Ws = rotated(W0)
    X = torch.from_numpy(np.random.default_rng(512).normal(size=(M, K)).astype(np.float32)).to(dev)
    Xq = mbq.stage_x(fmt, X)
    Y = torch.empty((M, N), device=dev)
    kern_us = per_launch_us(lambda W: mbq.gemv_xq(W, Xq, M=M, out=Y), Ws, 40)
    stage_us = per_launch_us(lambda W: mbq.stage_x(fmt, X, out=Xq), Ws, 40)
    tf = 2.0 * M * N * K / (kern_us * 1e-6) / 1e12
    rows["prefill_12288x4096_q45_m512"] = {
        "product_us": round(kern_us, 2), "staging_us": round(stage_us, 2),
        "useful_tflops": round(tf, 1),
        "mfma_issue_frac_of_fp16_peak": round(2 * tf / 2500.0, 4)}
    del Ws, W0, X, Xq, Y
    torch.cuda.empty_cache()

    # ---- the 4096 x 12288 Q45 table (the down projection's shape): the
    # matrix-core product with K whole per workgroup, and split in 4 along K
    # through a workspace (mbq_gemv_xq_ws)
    fmt, N, K = 1, 4096, 12288
    W0 = mbq.QWeight.from_host(fmt, N, K, workloads.weight_planes(np.random.default_rng(4), fmt, N, K))
    Ws = rotated(W0)
    down = {}
    for M in (16, 64, 512):
        X = torch.from_numpy(np.random.default_rng(M).normal(size=(M, K)).astype(np.float32)).to(dev)
        Xq = mbq.stage_x(fmt, X)
        Y = torch.empty((M, N), device=dev)
        ws = mbq.gemv_xq_workspace(W0, M)
        whole_us = per_launch_us(lambda W: mbq.gemv_xq(W, Xq, M=M, out=Y), Ws, 60)
        split_us = per_launch_us(lambda W: mbq.gemv_xq_ws(W, Xq, M, ws, out=Y), Ws, 60)
        down["M%d" % M] = {"product_us": round(whole_us, 2), "split_product_us": round(split_us, 2),
                           "split_useful_tflops": round(2.0 * M * N * K / (split_us * 1e-6) / 1e12, 1)}
        del X, Xq, Y, ws
    rows["down_4096x12288_q45_k_split"] = down
    del Ws, W0
    torch.cuda.empty_cache()

    # ---- the quantizer: fp32 weights to each format's planes, 12288 x 4096
    # (two inputs of 201 MB alternate, so that neither stays in the 256 MB
    # Infinity Cache)
    wq = torch.from_numpy(np.random.default_rng(11).normal(0, 0.02, size=(12288, 4096)).astype(np.float32)).to(dev)
    wqs = [wq, wq.clone()]
    quant = {}
    for fmt, name in ((1, "q45"), (2, "q65"), (3, "q25"), (0, "bf16")):
        Q = mbq.quantize(fmt, wq)
        us = per_launch_us(lambda w: mbq.quantize(fmt, w, out=Q), wqs * 4, 80)
        b = wq.numel() * 4 + Q.nbytes
        quant[name] = {"us": round(us, 2), "gbs": gbs(b, us), "bytes": b,
                       "frac_of_measured_peak": round(b / (us * 1e-6) / 1e9 / peak_gbs, 4)}
        del Q
    rows["quantize_12288x4096"] = quant
    del wq, wqs
    torch.cuda.empty_cache()

    # ---- decode attention, 32 query heads on 8 key/value heads of 128, cold
    # fp16 caches of T positions
    att = {}
    H, Hkv = 32, 8
    for T in (512, 4096, 32768):
        rng = np.random.default_rng(T)
        per = 2 * T * Hkv * 128 * 2
        caches = []
        for _ in range(max(2, min(64, ROTATION_BYTES // per))):
            kc = torch.from_numpy(rng.normal(size=(T, Hkv * 128)).astype(np.float16).view(np.int16)).to(dev)
            caches.append((kc, kc.clone()))
        q = torch.from_numpy(rng.normal(size=H * 128).astype(np.float32)).to(dev)
        o = torch.empty(H * 128, device=dev)
        wsb = torch.empty(mbq.attention_workspace_bytes(T, H, Hkv) // 4 + 4, device=dev)
        us = per_launch_us(lambda c: mbq.attention_decode(q, c[0], c[1], H, Hkv, out=o, workspace=wsb), caches)
        att["T%d" % T] = {"us": round(us, 2), "gbs": gbs(per, us), "kv_bytes": per,
                          "frac_of_measured_peak": round(per / (us * 1e-6) / 1e9 / peak_gbs, 4)}
        del caches
        torch.cuda.empty_cache()
    rows["attention_h32_kv8_d128"] = att

    # ---- workload 3: one token through the 36-layer stream
    rows["decode_36_layers"] = decode_row(workloads, torch, dev, peak_gbs, one_launch=one_launch,
                                          keep=keep)
    return rows


def ceilings(mbq, torch, dev, stream, full=True):
    """The measured ceilings: HBM bandwidth as the larger of a 4 GiB read and
    a 2 GiB in-device copy (read and write both counted), best of 5 each; the
    memory latency from a dependent pointer chase over 2 GiB; the issue rates
    of the fp16 matrix instructions, fp32 FMA and the int8 dot4 the vector
    kernels use."""
    def best_of(fn, n=5):
        best = float("inf")
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) * 1e-3)
        return best

    out = {}
    buf = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, device=dev)
    mbq.probe_read(buf, sink, stream)
    out["read_gbs"] = round(buf.numel() / best_of(lambda: mbq.probe_read(buf, sink, stream)) / 1e9, 1)
    half = 1 << 31
    src, dst = buf[:half], buf[half:]
    mbq.probe_copy(dst, src, stream)
    out["copy_gbs"] = round(2 * half / best_of(lambda: mbq.probe_copy(dst, src, stream)) / 1e9, 1)
    out["peak_gbs"] = max(out["read_gbs"], out["copy_gbs"])
    if full:
        chase = buf[:half]
        n = mbq.probe_chase_init(chase, stream)
        isink = torch.zeros(4, dtype=torch.int32, device=dev)
        hops = 20000
        mbq.probe_chase(chase, n, 1000, isink, stream)
        t = best_of(lambda: mbq.probe_chase(chase, n, hops, isink, stream), 3)
        lat_ns = t / hops * 1e9
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        out["latency"] = {"ns_per_hop": round(lat_ns, 1), "entries": n, "span_bytes": half,
                          "bytes_in_flight_at_peak": int(out["peak_gbs"] * lat_ns),
                          "bytes_in_flight_per_cu": int(out["peak_gbs"] * lat_ns / cus),
                          "compute_units": cus}
        psink = torch.empty(2048, device=dev)
        rates = {}
        for kind, name, iters in ((mbq.PEAK_MFMA_F16, "mfma_f16_tflops", 4000),
                                  (mbq.PEAK_MFMA_F16_32, "mfma_f16_32x32_tflops", 2000),
                                  (mbq.PEAK_FMA_F32, "fma_f32_tflops", 20000),
                                  (mbq.PEAK_DOT4_I8, "dot4_i8_tops", 20000)):
            ops = mbq.probe_peak(kind, iters, psink, stream)
            rates[name] = round(ops / best_of(lambda: mbq.probe_peak(kind, iters, psink, stream), 3) / 1e12, 2)
        out.update(rates)
        # M* = (w/16)(R/BW) for the 4.5-bit table at the measured bandwidth,
        # with R the multiply-adds per second each path's arithmetic turns
        # into useful sums: the matrix path issues two fp16 products per sum
        # (x as high and low parts), the vector path three byte products per
        # sum (x as three byte digits, four byte products per dot4)
        bw = out["peak_gbs"] * 1e9
        r_mfma = rates["mfma_f16_tflops"] * 1e12 / 2 / 2
        r_vec = rates["dot4_i8_tops"] * 1e12 / 2 / 3
        out["m_star_q45"] = {"matrix_cores": round(4.5 / 16 * r_mfma / bw, 2),
                             "vector_units": round(4.5 / 16 * r_vec / bw, 2),
                             "rule": "M* = (w/16)(R/BW), w = 4.5, R = multiply-adds/s of each path's arithmetic"}
        # per compute unit, the two streams of the 16-token matrix-core product
        # (its 110 KB of weights from HBM, the 264 KB staged x every unit reads
        # from L2), alone and together: whether they overlap or queue
        dbytes, sbytes = 112 * 1024, 264 * 1024
        dist = buf[:cus * dbytes]
        shared = buf[half:half + sbytes]
        msink = torch.empty(cus, device=dev)
        mixed = {}
        for mode, name in ((0, "hbm_distinct_112k_per_cu_us"), (1, "l2_shared_264k_us"),
                           (2, "both_interleaved_us"), (3, "both_separate_waves_us")):
            # the distinct data rotates over 16 regions so that it comes from HBM
            regs = [buf[r * cus * dbytes:(r + 1) * cus * dbytes] for r in range(16)]
            for rg in regs:
                mbq.probe_mixed(rg, dbytes, shared, sbytes, mode, cus, msink, stream)
            torch.cuda.synchronize()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for k in range(4):
                for rg in regs:
                    mbq.probe_mixed(rg, dbytes, shared, sbytes, mode, cus, msink, stream)
            b_.record(stream)
            torch.cuda.synchronize()
            mixed[name] = round(a_.elapsed_time(b_) * 1e3 / 64, 2)
        out["per_cu_streams"] = mixed
    del buf
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="headline step only")
    ap.add_argument("--no-one-launch", action="store_true",
                    help="leave out the cooperative one-launch decode step (for profiled runs)")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="only the launches that the counter runs profile")
    ap.add_argument("--rows-traffic-pass", action="store_true",
                    help="only the other rows' launches that the counter runs profile")
    ap.add_argument("--mfma-pass", action="store_true",
                    help="only the matrix-core launches that the counter runs profile")
    ap.add_argument("--mfma-pass-tokens", default="16,64", metavar="M,M,...",
                    help="batch sizes of --mfma-pass (default 16,64)")
    ap.add_argument("--decode-only", type=int, metavar="TOKENS", default=0,
                    help="only the 36-layer decode step, TOKENS graph replays (for profiling)")
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
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    if args.traffic_pass:
        traffic_pass()
        return
    if args.mfma_pass:
        mfma_pass(tokens=tuple(int(t) for t in args.mfma_pass_tokens.split(",")))
        return
    if args.rows_traffic_pass:
        rows_traffic_pass()
        return

    import torch
    import memory_bound_quantized_amd as mbq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode_only:
        print(json.dumps({"decode_36_layers": decode_row(workloads, torch, dev, DEFAULT_PEAK_GBS,
                                                          ntok=args.decode_only,
                                                          one_launch=not args.no_one_launch)}))
        return
    stream = torch.cuda.current_stream()
    ceil = ceilings(mbq, torch, dev, stream, full=not args.no_rows)
    peak = ceil["peak_gbs"]

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

    # step i uses weight copy i % ncopy: consecutive steps never share weights
    def steps_graph(n, up=True, down=True):
        def body():
            for i in range(n):
                if up:
                    mbq.gemv_q(ups[i % ncopy], x_up, out=y_up)
                if down:
                    mbq.gemv_q(dns[i % ncopy], x_dn, out=y_dn)
        return capture(body)

    K, W = args.steps, args.warmup
    g_steps = steps_graph(K)
    g_warm = steps_graph(W) if W > 0 else None

    # ledger: 3 windows in alternating order of the step and each kernel kind
    # alone (graphs of max(K, 2 ncopy, LEDGER_MIN_LAUNCHES) launches each, so
    # that a window spans 10-30 ms and not a few ms of clock noise), medians,
    # and whether the windows agree within 3 %.  It runs before the timed
    # steps: its ~0.3 s of launches also bring the clocks from the idle of the
    # host-side set-up to their working state, which a warm-up of a few ms
    # does not.
    nl = max(K, 2 * ncopy, LEDGER_MIN_LAUNCHES)
    g_all, g_up, g_dn = steps_graph(nl), steps_graph(nl, down=False), steps_graph(nl, up=False)
    wins = {"step": [], "up": [], "down": []}
    orders = (("step", "up", "down"), ("down", "up", "step"), ("up", "step", "down"))
    graphs = {"step": g_all, "up": g_up, "down": g_dn}
    for k in ("step", "up", "down"):
        graphs[k].replay()
    for order in orders:
        for k in order:
            wins[k].append(timed(graphs[k], 1, stream) / nl)
    med = {k: float(np.median(v)) for k, v in wins.items()}
    spread = {k: (max(v) - min(v)) / med[k] for k, v in wins.items()}
    up_ms, dn_ms = med["up"], med["down"]
    del g_all, g_up, g_dn

    upload(g_steps, stream)
    if g_warm is not None:
        g_warm.replay()
        del g_warm
    torch.cuda.synchronize()
    y_up_first = y_up.cpu().numpy().copy()
    y_dn_first = y_dn.cpu().numpy().copy()

    # timed region: exactly K steps (one replay of the K-step graph)
    total_ms = timed(g_steps, 1, stream)
    ms_per_step = total_ms / K
    b_up, b_dn = gemv_bytes(W_up0), gemv_bytes(W_dn0)
    value = (b_up + b_dn) / (ms_per_step * 1e-3) / 1e9
    del g_steps, ups, dns

    # RMSNorm of one 4096-wide row (the metric's second part), one row per launch
    c1 = workloads.config1()
    xr = torch.from_numpy(c1["x"]).to(dev)
    gr = torch.from_numpy(c1["gamma"]).to(dev)
    yr = torch.empty_like(xr)
    nrm = 64
    g_norm = capture(lambda: [mbq.rmsnorm(xr, gr, c1["eps"], out=yr) for _ in range(nrm)])
    g_norm.replay()
    rms_us = timed(g_norm, 20, stream) / (20 * nrm) * 1e3
    # the same graph of one-workgroup launches that read nothing: what a
    # launch alone costs in this setting
    sink1 = torch.zeros(4, device=dev)
    g_null = capture(lambda: [mbq.probe_mixed(xr, 0, xr, 0, 0, 1, sink1) for _ in range(nrm)])
    g_null.replay()
    null_us = timed(g_null, 20, stream) / (20 * nrm) * 1e3
    del g_norm, g_null

    kern = {"q45_up_12288x4096": (b_up, up_ms), "q65_down_4096x12288": (b_dn, dn_ms)}
    dom = max(kern, key=lambda k: kern[k][1])
    d_bytes, d_ms = kern[dom]
    achieved = d_bytes / (d_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dom), "algorithmic_bytes_per_launch": d_bytes,
                "avg_launch_us": round(d_ms * 1e3, 3),
                "measured_peak_gbs": peak,
                "frac_of_measured_peak": round(achieved / peak, 4)}
    # what a plain read of the same byte count achieves per launch, timed the
    # same way (graph of cold launches over >= 1 GiB of distinct buffers)
    rd_bytes = d_bytes
    n_rd = max(2, -(-ROTATION_BYTES // rd_bytes))
    rbufs = [torch.empty(rd_bytes, dtype=torch.uint8, device=dev) for _ in range(n_rd)]
    rd_sink = torch.empty(4096, device=dev)
    rd_us = per_launch_us(lambda b: mbq.probe_read(b, rd_sink), rbufs)
    del rbufs
    torch.cuda.empty_cache()
    roofline["same_size_read_us"] = round(rd_us, 3)
    roofline["frac_of_same_size_read"] = round(rd_us / (d_ms * 1e3), 4)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "M=1 GEMV: Q45 12288x4096 (4.5 bpw) + Q65 4096x12288 (6.5625 bpw), "
                               "fp32 x and accumulation, step i on weight copy i mod %d (%.2f GB)"
                               % (ncopy, ncopy * per_copy / 1e9),
                   "tokens_per_product": 1, "gpus": 1},
        "roofline": roofline,
        "kernels": {k: {"avg_us": round(v[1] * 1e3, 3), "gbs": round(v[0] / (v[1] * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(v[0] / (v[1] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "frac_of_measured_peak": round(v[0] / (v[1] * 1e-3) / 1e9 / peak, 4)}
                    for k, v in kern.items()},
        "ledger": {"launches_per_window": nl, "windows_ms_per_launch": {k: [round(x * 1e3, 3) for x in v]
                                                                        for k, v in wins.items()},
                   "spread": {k: round(v, 4) for k, v in spread.items()},
                   "windows_agree_within_3pct": all(v <= 0.03 for v in spread.values())},
        "rmsnorm_us_per_4096_row": round(rms_us, 3),
        "rmsnorm_row_vs_empty_launch": {"empty_launch_us": round(null_us, 3),
                                        "above_empty_launch_us": round(rms_us - null_us, 3)},
        "ceilings": ceil,
    }
    keep = {} if not args.no_rows else None
    if not args.no_rows:
        out["rows"] = rows_bench(mbq, workloads, torch, dev, peak, one_launch=not args.no_one_launch,
                                 keep=keep)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, y_up_first, y_dn_first,
                                           decode=keep if keep else None)
        if "rows" in out:
            out["rows"]["decode_36_layers"]["checked_against_oracle"] = True
            out["rows"]["decode_36_layers"]["with_attention_512"]["checked_against_oracle"] = True
    elif "rows" in out:
        out["rows"]["decode_36_layers"]["checked_against_oracle"] = False
        out["rows"]["decode_36_layers"]["with_attention_512"]["checked_against_oracle"] = False
    print(json.dumps(out))


if __name__ == "__main__":
    main()
