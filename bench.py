"""Throughput of one exact Lloyd iteration (assign + sort-inverse update) on one MI355X.

Default workload (--config c3): N=8,388,608 points, D=128, bf16 storage,
K=65,536 centroids, 65,536-component Gaussian mixture with Zipf(1.1)
weights (synthetic, seeded; the pages name no dataset).

A step is one full Lloyd iteration through the C ABI on inputs already
resident in HBM: centroid prep + fused MFMA distance/argmin + inertia, then
radix argsort + offsets + segment means.  `value` times K steps of the
library's own loop (one kmeans_fit call); a second pass calls kmeans_assign
and kmeans_update per step with HIP events on the stream the library launches
on, for the per-stage times and rooflines.  Prints one JSON line.
`--config` picks another workload (c1, c2, c4, c5).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Lloyd iter/s + assign TFLOP/s (2NKD) at N=8M,D=128,K=64K; % of roofline"
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--n", type=int, default=None, help="override rows (tests / quick runs)")
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None, help="rows in the oracle timing sample")
    ap.add_argument("--epilogue", default="argmax", choices=["argmax", "top2", "soft", "gauss"],
                    help="also time the assignment kernel with this epilogue (top-2 labels, the Gaussian-mixture "
                         "log density with sigma2=1, or signed Gauss sums over the centroids with sigma2=1) on the "
                         "same workload")
    ap.add_argument("--seeding", action="store_true",
                    help="also time k-means++ seeding of the workload's K centroids (kmeans_seed) and report the "
                         "bandwidth of its per-pick D^2 pass")
    ap.add_argument("--zipf-update", action="store_true",
                    help="also time kmeans_update with labels drawn from finite Zipf(1.1) over the K clusters "
                         "(the hot-cluster stress case: the top cluster holds about 1/H_K of all rows)")
    ap.add_argument("--tune", action="store_true",
                    help="time every compiled assign configuration on this shape first (kmeans_tune) and report it")
    ap.add_argument("--probe", action="store_true",
                    help="counter-collection target: one 1 GiB device copy (calibration) and one step, no timing")
    return ap.parse_args()


def cpu_baseline(p, sample_rows):
    """Time the fp64 oracle (as it stands) for one Lloyd iteration on a row
    sample of the same workload, scaled linearly to the full N."""
    import oracle
    from tests.gpu_harness import decode
    host = host_info()
    cores = host["blas"]["threads"] or 1
    B = p.B
    rows = min(sample_rows, p.N)
    Xs = p.X[0, :rows]
    Xd = decode(Xs, p.dtype)
    C = p.C0[0].numpy().astype(np.float64)
    t0 = time.perf_counter()
    Ch = oracle.round_to_format(C, p.dtype)
    lab, dmin = oracle.assign(Xd, Ch)
    oracle.inertia(dmin)
    oracle.update(Xd, lab, C, p.K)
    dt = time.perf_counter() - t0
    sec_per_iter = dt * (p.N / rows) * B
    return {"value": 1.0 / sec_per_iter, "unit": "iter/s", "cores": cores, "kind": "oracle",
            "sample": (f"one oracle Lloyd iteration (fp64 assign + update) on the first {rows:,} of "
                       f"{p.N:,} rows x {B} instance(s), all K={p.K:,} centroids, {dt:.1f} s, scaled "
                       f"linearly by N/{rows:,}; cores = the BLAS threads (the oracle's matrix products; its "
                       f"other numpy steps run on one thread)"),
            "cpu_count": host["cpu_count"], "cpu_model": host["cpu_model"], "blas": host["blas"]}


def host_info():
    """The host the oracle runs on: logical CPUs, the CPU model from
    /proc/cpuinfo, and numpy's BLAS (vendor, version, threads) as
    threadpoolctl reports it."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = {"vendor": None, "version": None, "threads": None}
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": int(i.get("num_threads") or 0) or None}
                break
    except Exception:  # pragma: no cover
        pass
    return {"cpu_count": os.cpu_count(), "cpu_model": model, "blas": blas}


ASSIGN_SOURCES = ["exact_means_clustering_amd/csrc/assign.hip", "exact_means_clustering_amd/csrc/common.h"]


def assign_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ASSIGN_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def assign_traffic(name, B, N, D, K):
    """HBM bytes per assign launch from the committed counter summary
    profiles/traffic_<workload>.txt, or None if absent, for another shape, or
    taken on a different assign kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("assign_source_sha256") != assign_source_sha():
            return None
        if (int(kv["B"]), int(kv["N"]), int(kv["D"]), int(kv["K"])) != (B, N, D, K):
            return None
        fetch_factor = float(kv["copy_bytes"]) / (float(kv["copy_fetch_kib"]) * 1024)
        write_factor = float(kv["copy_bytes"]) / (float(kv["copy_write_kib"]) * 1024)
        return (float(kv["assign_fetch_kib"]) * 1024 * fetch_factor
                + float(kv["assign_write_kib"]) * 1024 * write_factor)
    except (KeyError, ValueError):
        return None


def probe(args):
    """Counter-collection target: a plain 1 GiB device copy (calibrates
    FETCH_SIZE / WRITE_SIZE) followed by one assign and one update (and, with
    --zipf-update, one more update with Zipf(1.1) labels)."""
    import torch

    import datagen
    import exact_means_clustering_amd as km

    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    p = datagen.make(args.config, n=args.n, k=args.k)
    X = (p.X if p.B > 1 else p.X[0]).cuda()
    C = (p.C0 if p.B > 1 else p.C0[0]).cuda()
    ws = torch.empty(km.workspace_bytes(p.N, p.D, p.K, p.B, X.dtype), dtype=torch.uint8, device="cuda")
    labels, _, _ = km.assign(X, C, ws=ws)
    km.update(X, labels, C, ws=ws)
    if args.zipf_update:  # then one update with the Zipf(1.1) labels of --zipf-update
        zl = torch.from_numpy(datagen.zipf_labels(p.N, p.K, 1.1, seed=3, batch=p.B)).cuda()
        km.update(X, zl if p.B > 1 else zl[0], C, ws=ws)
    torch.cuda.synchronize()
    print(json.dumps({"probe": args.config, "B": p.B, "N": p.N, "D": p.D, "K": p.K,
                      "assign_source_sha256": assign_source_sha()}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch

    import datagen
    import exact_means_clustering_amd as km

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(2)
    name = args.config
    if args.probe:
        return probe(args)
    if name == "c5":
        return bench_streamed(args)
    t0 = time.time()
    p = datagen.make(name, n=args.n, k=args.k)
    print(f"[bench] generated {name}: B={p.B} N={p.N} D={p.D} K={p.K} {p.dtype} in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    X = (p.X if p.B > 1 else p.X[0]).to(dev)
    C0 = (p.C0 if p.B > 1 else p.C0[0]).to(dev)
    B, N, D, K = p.B, p.N, p.D, p.K
    dt_torch = X.dtype
    ws = torch.empty(km.workspace_bytes(N, D, K, B, dt_torch), dtype=torch.uint8, device=dev)
    labels = torch.empty(X.shape[:-1], dtype=torch.int32, device=dev)
    C = C0.clone()
    C_next = torch.empty_like(C)
    stream = torch.cuda.current_stream()
    tuning = None
    if args.tune:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pb, waves, t_ms = km.tune(X, C0, ws=ws)
        tuning = {"pb": pb, "waves": waves, "assign_ms_per_launch": t_ms,
                  "tuning_wall_s": time.perf_counter() - t0}

    def step(ev=None):
        nonlocal C, C_next
        if ev is not None:
            ev[0].record(stream)
        km.assign(X, C, ws=ws, labels=labels)
        if ev is not None:
            ev[1].record(stream)
        km.update(X, labels, C, C_new=C_next, ws=ws)
        if ev is not None:
            ev[2].record(stream)
        C, C_next = C_next, C

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    assign_ms = [e[0].elapsed_time(e[1]) for e in evs]
    update_ms = [e[1].elapsed_time(e[2]) for e in evs]
    # Headline: the same K steps run by the library's own Lloyd loop
    # (kmeans_fit, one call, no host round trip between kernels).  The
    # library captures a fit into a HIP graph on the first call with a new
    # argument list and replays it afterwards, so after the W-step warm-up
    # one untimed call with exactly the timed arguments does the capture;
    # the timed call replays all K iterations' kernels.
    out = (torch.empty_like(labels), torch.empty_like(C0), torch.empty(B, dtype=torch.float64, device=dev), None)
    km.fit(X, C0, args.warmup, ws=ws, out=out)
    km.fit(X, C0, args.steps, ws=ws, out=out)
    torch.cuda.synchronize()
    t_start.record(stream)
    km.fit(X, C0, args.steps, ws=ws, out=out)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    a_ms = float(np.mean(assign_ms))
    u_ms = float(np.mean(update_ms))
    flops = 2.0 * B * N * K * D
    a_tflops = flops / (a_ms * 1e-3) / 1e12
    sz = X.element_size()
    upd_bytes = B * (N * D * sz + 4 * N + 4 * K * D + 4 * K)
    u_gbs = upd_bytes / (u_ms * 1e-3) / 1e9
    peak = PEAK_TFLOPS[p.dtype]
    traffic = assign_traffic(name, B, N, D, K)
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms_step,
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": f"{name}: " + datagen.WORKLOADS[name]["desc"], "B": B, "N": N, "D": D, "K": K,
                   "storage": p.dtype, "accumulate": "fp32", "step": "one Lloyd iteration (assign + sort-inverse update); value from kmeans_fit over the timed steps (a replay of the fit's captured HIP graph), per-stage times from kmeans_assign / kmeans_update"},
        "assign_ms": a_ms,
        "update_ms": u_ms,
        "assign_tflops": a_tflops,
        "assign_frac_mfma_peak": a_tflops / peak,
        "update_gbs": u_gbs,
        "update_frac_hbm_peak": u_gbs / PEAK_HBM_GBS,
        "roofline": {"bound": "mfma", "achieved": a_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": a_tflops / peak, "traffic": traffic},
        "roofline_update": {"bound": "hbm", "achieved": u_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": u_gbs / PEAK_HBM_GBS, "algorithmic_bytes": upd_bytes},
    }
    if tuning is not None:
        out["tuning"] = tuning
    if args.zipf_update:
        zl = torch.from_numpy(datagen.zipf_labels(N, K, 1.1, seed=3, batch=B)).to(dev)
        zl = zl if B > 1 else zl[0]
        counts_top = int(torch.bincount(zl.reshape(-1).to(torch.int64)).max())
        for _ in range(max(1, args.warmup)):
            km.update(X, zl, C0, C_new=C_next, ws=ws)
        torch.cuda.synchronize()
        t_start.record(stream)
        for _ in range(args.steps):
            km.update(X, zl, C0, C_new=C_next, ws=ws)
        t_end.record(stream)
        torch.cuda.synchronize()
        z_ms = t_start.elapsed_time(t_end) / args.steps
        out["update_zipf"] = {"labels": "finite Zipf(1.1) over K", "top_cluster_rows": counts_top, "ms": z_ms,
                              "gbs": upd_bytes / (z_ms * 1e-3) / 1e9,
                              "frac_hbm_peak": upd_bytes / (z_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                              "time_vs_kmeans_labels": z_ms / u_ms}
    if args.seeding:
        su = torch.rand(C0.shape[:-1], dtype=torch.float64, generator=torch.Generator().manual_seed(3)).to(dev)
        km.seed(X, su, method="kmeans++", ws=ws)          # warm-up (kernel loads)
        torch.cuda.synchronize()
        t_start.record(stream)
        km.seed(X, su, method="kmeans++", ws=ws)
        t_end.record(stream)
        torch.cuda.synchronize()
        s_ms = t_start.elapsed_time(t_end)
        per_pick = s_ms / max(1, K - 1)
        pass_bytes = B * N * (D * sz + 8)                 # one D^2 pass: X once, D^2 read and written
        out["seeding"] = {"method": "kmeans++", "ms": s_ms, "ms_per_pick": per_pick,
                          "d2_pass_bytes": pass_bytes, "gbs_per_pick": pass_bytes / (per_pick * 1e-3) / 1e9}
    if args.epilogue != "argmax":
        if args.epilogue == "top2":
            def epi():
                km.assign_top2(X, C0, ws=ws)
        elif args.epilogue == "soft":
            def epi():
                km.assign_soft(X, C0, 1.0, ws=ws)
        else:
            gw = torch.randn(C0.shape[:-1], generator=torch.Generator().manual_seed(1)).to(dev)

            def epi():
                km.gauss_sum(X, C0, gw, 1.0, ws=ws)
        for _ in range(max(1, args.warmup)):
            epi()
        torch.cuda.synchronize()
        t_start.record(stream)
        for _ in range(args.steps):
            epi()
        t_end.record(stream)
        torch.cuda.synchronize()
        e_ms = t_start.elapsed_time(t_end) / args.steps
        e_tf = flops / (e_ms * 1e-3) / 1e12
        out["epilogue"] = {"mode": args.epilogue, "ms": e_ms, "tflops": e_tf, "frac_mfma_peak": e_tf / peak,
                           "time_vs_argmax_assign": e_ms / a_ms}
    if not args.no_cpu_baseline:
        # rows of the oracle's timing sample: about 10-30 s of host work each
        sample = args.cpu_sample or {"c1": 65536, "c2": 1 << 20, "c3": 1 << 17, "c4": 16384}[name]
        out["cpu_baseline"] = cpu_baseline(p, sample)
    print(json.dumps(out), flush=True)


def bench_streamed(args):
    """Out-of-core workload: X in pinned host memory, streamed in chunks."""
    import torch

    import datagen
    import exact_means_clustering_amd as km

    n = args.n or (1 << 27)
    t0 = time.time()
    p = datagen.make("c5", n=n, k=args.k)
    X = p.X[0].pin_memory()
    budget = X.numel() * X.element_size() // 8       # device slots hold 1/8 of X
    print(f"[bench] generated c5 N={p.N} in {time.time() - t0:.1f}s, budget {budget / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)
    C0 = p.C0[0].cuda()
    km.fit_streamed(X, C0, 1, budget)                 # warm-up
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    iters = max(1, args.steps)
    km.fit_streamed(X, C0, iters, budget)
    dt = time.perf_counter() - t1
    gb = X.numel() * X.element_size() / 1e9
    row_bytes = p.D * X.element_size()
    chunk = min(budget // 2 // row_bytes, p.N)
    issued = iters * ((p.N + chunk - 1) // chunk)
    out = {"metric": METRIC, "value": iters / dt, "unit": "iter/s", "n_gpus": 1, "steps": iters, "warmup": 1,
           "ms_per_step": dt / iters * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": p.dtype, "data": "synthetic",
           "config": {"workload": f"c5 (scaled to N={p.N:,}): pinned-host X streamed through two device slots",
                      "N": p.N, "D": p.D, "K": p.K, "device_x_budget": budget},
           "h2d_gbs": gb * iters / dt,
           "assign_tflops_effective": 2.0 * p.N * p.K * p.D * iters / dt / 1e12,
           "overlap": stream_overlap(km.stream_timeline(), issued, gb * 1e9 * iters)}
    print(json.dumps(out), flush=True)


def _union(iv):
    """Merged, sorted list of the intervals [a, b)."""
    out = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _length(iv):
    return sum(b - a for a, b in iv)


def _intersection(u, v):
    i = j = 0
    total = 0.0
    while i < len(u) and j < len(v):
        a, b = max(u[i][0], v[j][0]), min(u[i][1], v[j][1])
        total += max(0.0, b - a)
        if u[i][1] < v[j][1]:
            i += 1
        else:
            j += 1
    return total


def stream_overlap(tl, issued, h2d_bytes):
    """Copy / compute overlap of a streamed fit from its per-chunk HIP-event
    timeline (rows: iteration, chunk, copy-in start/end, compute start/end,
    labels-out start/end, ms): busy time of the host-to-device copies and of
    the compute, the time both run at once, and what share of the shorter of
    the two is hidden under the other."""
    if not tl:
        return {"chunks_recorded": 0, "chunks_issued": issued}
    cin = _union([(r[2], r[3]) for r in tl])
    comp = _union([(r[4], r[5]) for r in tl])
    cout = _union([(r[6], r[7]) for r in tl])
    wall = max(r[7] for r in tl) - min(r[2] for r in tl)
    both = _intersection(cin, comp)
    shorter = min(_length(cin), _length(comp))
    return {"chunks_recorded": len(tl), "chunks_issued": issued, "wall_ms": wall,
            "h2d_busy_ms": _length(cin), "compute_busy_ms": _length(comp), "d2h_busy_ms": _length(cout),
            "both_busy_ms": both, "h2d_busy_frac": _length(cin) / wall,
            "hidden_frac_of_shorter": both / shorter if shorter > 0 else None,
            "h2d_gbs_while_copying": h2d_bytes / (_length(cin) * 1e-3) / 1e9}


if __name__ == "__main__":
    main()
