"""Benchmark of the GDLA attention core on one MI355X.

One step = one pass of the fused prefill kernel over the full-causal workload
(batch 1, T = 4096, 16 KV heads / 64 signal / 16 noise heads, qk 192 / v 128,
bf16, synthetic seeded inputs already resident in HBM).  The kernel does the
whole hot path: band limits, K/V tiles, QK^T, mask, softmax, PV, the
differential combine and the gate.

Printed: ONE JSON line with the throughput (unmasked FLOPs / time), the
roofline of the prefill kernel (timed with HIP events on the stream it runs
on), the CPU oracle timed on a bounded sample of the same workload, and the
other workloads (sliding-window prefill, 128K prefill, prefill after a
prefix, decode over the expanded and the latent cache, the pre-attention step)
under "extra".

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                    [--extras pf_swa_32k,dec_full,...]
"""
import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDLA prefill TFLOP/s + decode HBM GB/s, each as % of MI355X roofline"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
FLOP_PER_PAIR = 640            # 2*192 (QK^T) + 2*128 (PV) per (query head, query, key)
N_HEADS = 80                   # 64 signal + 16 noise query heads


def pairs_prefill(B, T, window, prefix=0):
    """Unmasked (query, key) pairs per head: queries at positions prefix .. T-1."""
    def upto(n):            # sum over positions t < n of the keys t sees
        if window <= 0 or window >= n:
            return n * (n + 1) // 2
        return window * (window + 1) // 2 + (n - window) * window
    return B * (upto(T) - upto(prefix))


def prefill_bytes(B, T, n_kv=16, n_sig=64, prefix=0):
    # q_signal, q_noise, lambda, gate in and out written for each query token;
    # k, v in for every token (prefix included); each once, bf16
    per_q = 2 * (n_sig * 192 + n_kv * 192 + n_sig + 2 * n_sig * 128)
    per_kv = 2 * (n_kv * 192 + n_kv * 128)
    return B * ((T - prefix) * per_q + T * per_kv)


def decode_bytes(lengths, window, n_kv=16, n_sig=64):
    vis = [min(L, window) if window > 0 else L for L in lengths]
    per_seq = 2 * (n_sig * 192 + n_kv * 192 + n_sig + 2 * n_sig * 128)
    return sum(vis) * n_kv * (192 + 128) * 2 + len(lengths) * per_seq + 4 * (len(lengths) + 1)


def decode_latent_bytes(lengths, window, n_kv=16, n_sig=64):
    vis = [min(L, window) if window > 0 else L for L in lengths]
    per_seq = 2 * (n_sig * 192 + n_kv * 192 + n_sig + 2 * n_sig * 128)
    weights = 2 * n_kv * (128 + 128) * 512             # the two up-projections, read once
    return sum(vis) * 576 * 2 + len(lengths) * per_seq + weights + 4 * (len(lengths) + 1)


PREFILL_SOURCES = ("prefill_gfx950.hip", "gdla_device.h")


def source_hash():
    """Hash of the files the prefill kernel is built from (its traffic figures
    hold while these are unchanged)."""
    h = hashlib.sha256()
    for name in PREFILL_SOURCES:
        h.update(open(os.path.join(ROOT, "attention_gdla_prefill_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def _counter_rows(run_dir, counter):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv run."""
    import csv
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    rows = []
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def record_traffic(workload, fetch_dir, write_dir):
    """Writes profiles/traffic_<workload>.json from two counter runs of
    `bench.py --workload <workload> --steps 5 --warmup 2 --no-cpu-baseline
    --no-extra --copy-probe` (FETCH_SIZE, then WRITE_SIZE): the prefill
    kernel's median per dispatch, each counter scaled by what it reads for the
    1 GiB device copy that ends the run."""
    import statistics
    out = {"kernel": "prefill_kernel", "workload": workload, "source_hash": source_hash()}
    scaled = {}
    for key, run_dir, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(run_dir, counter)
        kern = [v for n, v in rows if "prefill_kernel" in n]
        copy = [v for n, v in rows if "copy" in n.lower()]
        if not kern or not copy:
            raise SystemExit("%s: prefill or copy dispatches missing" % run_dir)
        per = statistics.median(kern)
        probe = copy[-1]
        scale = (1 << 30) / 1024.0 / probe
        out["%s_kib_per_dispatch" % key] = per
        out["%s_scale" % key] = scale
        out["copy_probe_%s_kib" % key] = probe
        scaled[key] = per * 1024.0 * scale
    out["read_bytes"] = scaled["fetch"]
    out["written_bytes"] = scaled["write"]
    out["bytes_per_launch"] = scaled["fetch"] + scaled["write"]
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def time_kernel(fn, steps, warmup, stream):
    """Run fn warmup+steps times; return (wall ms/step, per-launch HIP-event ms list)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [a.elapsed_time(b) for a, b in ev]


def cpu_baseline(budget_s=15.0):
    """The oracle, untuned, on a random sample of query rows of the 4K workload."""
    import numpy as np
    import torch
    import oracle
    import workload as W
    w = W.WORKLOADS["pf_full_4k"]
    x = W.prefill_inputs(w, seed=0, device="cpu")
    f = {k: v.float().numpy() for k, v in x.items()}
    rng = np.random.default_rng(0)
    n, done_rows, done_pairs, elapsed = 32, 0, 0, 0.0
    while elapsed < budget_s:
        rt = rng.integers(0, w.T, size=n).astype(np.int32)
        rb = np.zeros(n, np.int32)
        t0 = time.perf_counter()
        oracle.prefill_rows(f["k"], f["v"], f["q_signal"][0, rt], f["q_noise"][0, rt], f["lam"][0, rt],
                            f["gate"][0, rt], rb, rt, window=0)
        elapsed += time.perf_counter() - t0
        done_rows += n
        done_pairs += int((rt.astype(np.int64) + 1).sum())
        n *= 2
    tflops = done_pairs * N_HEADS * FLOP_PER_PAIR / elapsed / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d random query rows (all 80 heads) of the B=1 T=4096 full-causal prefill, "
                      "%.1f s of CPU time, fp64 oracle" % (done_rows, elapsed)}


def load_traffic(name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


def bench_prefill(name, steps, warmup):
    import torch
    import attention_gdla_prefill_amd as gdla
    import workload as W
    w = W.WORKLOADS[name]
    x = W.prefill_inputs(w, seed=0, device="cuda")
    P = w.prefix
    stream = torch.cuda.current_stream()
    if P == 0:
        out = torch.empty((w.B, w.T, w.n_sig, 128), dtype=torch.bfloat16, device="cuda")
        fn = lambda: gdla.prefill(x["q_signal"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"],
                                  window=w.window, out=out)
    else:
        for key in ("q_signal", "q_noise", "lam", "gate"):       # the queries: positions P .. T-1
            x[key] = x[key][:, P:].contiguous()
        out = torch.empty((w.B, w.T - P, w.n_sig, 128), dtype=torch.bfloat16, device="cuda")
        fn = lambda: gdla.prefill_prefix(x["q_signal"], x["q_noise"], x["k"], x["v"], x["lam"],
                                         x["gate"], window=w.window, out=out)
    wall, ev = time_kernel(fn, steps, warmup, stream)
    kern_ms = sum(ev) / len(ev)
    flops = pairs_prefill(w.B, w.T, w.window, P) * N_HEADS * FLOP_PER_PAIR
    nbytes = prefill_bytes(w.B, w.T, prefix=P)
    del x, out
    torch.cuda.empty_cache()
    return {"wall_ms": wall, "kernel_ms": kern_ms, "flops": flops, "bytes": nbytes,
            "tflops": flops / (kern_ms * 1e-3) / 1e12, "gbs": nbytes / (kern_ms * 1e-3) / 1e9}


def prep_bytes(w, d_model=4096):
    """Algorithmic HBM bytes of the pre-attention step at prefill workload w:
    the rotary parts of the query heads read and written, the rotary key read
    once and written into every KV head, x read, W^lambda read once, lambda
    written, the gate's pre-activations read and the gate written."""
    n_tok = w.B * w.T
    return (n_tok * (w.n_sig + w.n_kv) * 64 * 2 * 2 + n_tok * 64 * 2 + n_tok * w.n_kv * 64 * 2
            + n_tok * d_model * 2 + w.n_sig * d_model * 2 + n_tok * w.n_sig * 2
            + n_tok * w.n_sig * w.d_v * 2 * 2)


def bench_prep(name, steps, warmup):
    """The pre-attention step (rotary embedding, lambda, gate) at the shapes of
    prefill workload name, cold cache (a 512 MB buffer is rewritten before each
    launch).  It rotates in place, so the inputs drift between launches; the
    time does not depend on the values."""
    import torch
    import attention_gdla_prefill_amd as gdla
    import workload as W
    w = W.WORKLOADS[name]
    d = W.prep_inputs(w, seed=0, device="cuda")
    lam = torch.empty((w.B, w.T, w.n_sig), dtype=torch.bfloat16, device="cuda")
    gate = torch.empty_like(d["gate_pre"])
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: gdla.prep(d["q_signal"], d["q_noise"], d["k_rope"], d["k"], d["x"], d["w_lambda"],
                             d["gate_pre"], lam_out=lam, gate_out=gate)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    nbytes = prep_bytes(w)
    del d, lam, gate, flush
    torch.cuda.empty_cache()
    return {"kernel_ms": ms, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "cache": "cold (512 MB buffer rewritten before each launch)"}


def bench_backward(name, steps, warmup):
    """The prefill backward (forward recomputed inside) at prefill workload
    name, warm.  Algorithmic FLOPs: 1664 per unmasked (head, query, key) pair
    -- the scores again (2*192), dP = dH V^T (2*128), dV (2*128), dK (2*192),
    dQ (2*192); the kernels issue 2944 (the saving forward's 640, and the
    scores and dP once in each of the two gradient kernels)."""
    import torch
    import attention_gdla_prefill_amd as gdla
    import workload as W
    w = W.WORKLOADS[name]
    x = W.prefill_inputs(w, seed=0, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    d_out = torch.randn((w.B, w.T, w.n_sig, w.d_v), generator=gen, device="cuda").to(torch.bfloat16)
    ws = torch.empty(gdla.prefill_backward_workspace_size(w.B, w.T, w.n_kv), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: gdla.prefill_backward(x["q_signal"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"], d_out,
                                       window=w.window, workspace=ws)
    wall, ev = time_kernel(fn, steps, warmup, stream)
    ms = sum(ev) / len(ev)
    pairs = pairs_prefill(w.B, w.T, w.window, 0) * (w.n_sig + w.n_kv)
    del x, d_out, ws
    torch.cuda.empty_cache()
    return {"ms": ms, "tflops": pairs * 1664 / (ms * 1e-3) / 1e12,
            "mfma_frac": pairs * 1664 / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "issued_tflops": pairs * 2944 / (ms * 1e-3) / 1e12, "steps": steps}


def bench_decode(name, steps, warmup):
    import torch
    import attention_gdla_prefill_amd as gdla
    import workload as W
    w = W.WORKLOADS[name]
    d = W.decode_inputs(w, seed=0, device="cuda")
    lengths = d["lengths"].tolist()
    max_len = max(lengths)
    out = torch.empty((w.B, w.n_sig, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(16, gdla.decode_workspace_size(w.B, w.n_kv, max_len, w.window)),
                     dtype=torch.uint8, device="cuda")
    # a buffer larger than the 256 MB Infinity Cache, rewritten before each launch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: gdla.decode(d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"],
                               d["cu_seqlens"], max_len, d["lam"], d["gate"], window=w.window,
                               out=out, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    kern_ms = sorted(times)[len(times) // 2]
    nbytes = decode_bytes(lengths, w.window)
    del d, out, ws, flush
    torch.cuda.empty_cache()
    return {"kernel_ms": kern_ms, "bytes": nbytes, "gbs": nbytes / (kern_ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "cache": "cold (512 MB buffer rewritten before each launch)"}


def measured_peaks():
    """Achievable rates on this GPU for context: a library bf16 GEMM and a copy."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    n = 8192
    a = torch.randn(n, n, device="cuda", generator=g).bfloat16()
    b = torch.randn(n, n, device="cuda", generator=g).bfloat16()
    for _ in range(5):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_gemm_8192_tflops": gemm_tflops, "bf16_gemm_frac_of_peak": gemm_tflops / PEAK_BF16_TFLOPS,
            "copy_1gib_gbs": copy_gbs, "copy_frac_of_peak": copy_gbs / PEAK_HBM_GBS}


def bench_decode_latent(name, steps, warmup):
    import torch
    import attention_gdla_prefill_amd as gdla
    import workload as W
    w = W.WORKLOADS[name]
    d = W.latent_decode_inputs(w, seed=0, device="cuda")
    lengths = d["lengths"].tolist()
    max_len = max(lengths)
    out = torch.empty((w.B, w.n_sig, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdla.decode_latent_workspace_size(w.B, w.n_kv, max_len, w.window),
                     dtype=torch.uint8, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: gdla.decode_latent(d["q_signal"], d["q_noise"], d["latent"], d["cu_seqlens"], max_len,
                                      d["w_uk"], d["w_uv"], d["lam"], d["gate"], window=w.window,
                                      out=out, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    kern_ms = sorted(times)[len(times) // 2]
    nbytes = decode_latent_bytes(lengths, w.window)
    expanded = decode_bytes(lengths, w.window)
    del d, out, ws, flush
    torch.cuda.empty_cache()
    return {"kernel_ms": kern_ms, "bytes": nbytes, "gbs": nbytes / (kern_ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "expanded_equivalent_gbs": expanded / (kern_ms * 1e-3) / 1e9,
            "cache": "cold (512 MB buffer rewritten before each launch)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clock needs ~0.1 s of steady work to settle: the default
    # warmup covers that (about 0.1 s at 4K) before 100 timed steps
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="pf_full_4k",
                    choices=["pf_full_4k", "pf_swa_32k", "pf_full_128k", "pf_prefix_4k_32k", "pf_swa_rank"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--extras", default="pf_swa_32k,pf_full_128k,pf_prefix_4k_32k,pf_swa_rank,"
                                        "dec_full,dec_swa,dec_latent_full,dec_latent_swa,prep_4k,prep_swa_32k,bwd_4k",
                    help="comma-separated extra workloads to time (a profile of one workload "
                         "names just that one)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--peaks", action="store_true",
                    help="also time a bf16 8192^3 GEMM (hipBLASLt via torch) and a 1 GiB device "
                         "copy: achievable-rate references, reported under 'peaks'")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of this script with --copy-probe, then exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    wanted = [] if args.no_extra else [x for x in args.extras.split(",") if x]
    for name in wanted:
        if name not in ("pf_swa_32k", "pf_full_128k", "pf_prefix_4k_32k", "pf_swa_rank", "dec_full",
                        "dec_swa", "dec_latent_full", "dec_latent_swa", "prep_4k", "prep_swa_32k", "bwd_4k"):
            print("unknown extra workload %r" % name, file=sys.stderr)
            sys.exit(2)

    import torch
    import workload as W
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    import attention_gdla_prefill_amd._lib as L
    L.load()          # fails loudly if the HIP library is missing

    w = W.WORKLOADS[args.workload]
    print("[bench] %s steps=%d warmup=%d" % (args.workload, args.steps, args.warmup),
          file=sys.stderr, flush=True)
    main_res = bench_prefill(args.workload, args.steps, args.warmup)

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    extra = {}
    if wanted:
        for name in ("pf_swa_32k", "pf_full_128k", "pf_prefix_4k_32k", "pf_swa_rank"):
            if name == args.workload or name not in wanted:
                continue
            print("[bench] extra %s" % name, file=sys.stderr, flush=True)
            steps, warm = (3, 1) if name == "pf_full_128k" else (50, 50)
            r = bench_prefill(name, steps, warm)
            extra[name] = {"tflops": r["tflops"], "mfma_frac": r["tflops"] / PEAK_BF16_TFLOPS,
                           "gbs": r["gbs"], "hbm_frac": r["gbs"] / PEAK_HBM_GBS,
                           "kernel_ms": r["kernel_ms"], "steps": steps}
        for name in ("dec_full", "dec_swa", "dec_latent_full", "dec_latent_swa"):
            if name not in wanted:
                continue
            print("[bench] extra %s" % name, file=sys.stderr, flush=True)
            fn = bench_decode_latent if name.startswith("dec_latent") else bench_decode
            extra[name] = fn(name, 10, 2)
        for name, shape in (("prep_4k", "pf_full_4k"), ("prep_swa_32k", "pf_swa_32k")):
            if name not in wanted:
                continue
            print("[bench] extra %s" % name, file=sys.stderr, flush=True)
            extra[name] = dict(bench_prep(shape, 20, 5), shapes=shape)
        if "bwd_4k" in wanted:
            print("[bench] extra bwd_4k", file=sys.stderr, flush=True)
            extra["bwd_4k"] = dict(bench_backward("pf_full_4k", 20, 10), shapes="pf_full_4k")

    peaks = measured_peaks() if args.peaks else None

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline()

    traffic = load_traffic(args.workload)
    line = {
        "metric": METRIC,
        "value": main_res["flops"] / (main_res["wall_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["wall_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: prefill B=%d T=%d, %d KV / %d signal / %d noise heads, qk 192 / "
                               "v 128, %s" % (w.name, w.B, w.T, w.n_kv, w.n_sig, w.n_kv,
                                              "full causal" if w.window == 0 else "window %d" % w.window),
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": main_res["tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": main_res["tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "kernel": "prefill_kernel",
                     "kernel_ms": main_res["kernel_ms"], "flops_per_launch": main_res["flops"],
                     "algorithmic_bytes_per_launch": main_res["bytes"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if peaks is not None:
        line["peaks"] = peaks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
