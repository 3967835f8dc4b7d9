"""Benchmark of the GDLA attention core on one MI355X.

One step = one pass of the fused prefill kernel over the long-context
full-causal workload (batch 1, T = 131072, 16 KV heads / 64 signal / 16 noise
heads, qk 192 / v 128, bf16, synthetic seeded inputs already resident in HBM).
The kernel does the whole hot path: band limits, K/V tiles, QK^T, mask,
softmax, PV, the differential combine and the gate.

Before the timed steps the kernel runs untimed until at least --warmup
launches and --settle-s seconds of steady work have passed (the GPU clock
needs about a tenth of a second of load to settle); the JSON reports both.

Printed: ONE JSON line with the throughput (unmasked FLOPs / time), the
roofline of the prefill kernel (timed with HIP events on the stream it runs
on), the roofline of the full-causal decode (cold cache, HBM-bound), the fp32
CPU oracle timed on a bounded sample of the same workload (extrapolated by
unmasked pairs) and in full on the small configs, and the other workloads
under "extra".

    python bench.py [--steps K] [--warmup W] [--settle-s S] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-full] [--no-decode] [--no-extra]
                    [--extras a,b,...]
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

PEAK_CLOCK_MHZ = 2400.0          # the clock the published dense peaks assume
METRIC = "GDLA prefill TFLOP/s + decode HBM GB/s, each as % of MI355X roofline"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP32_TFLOPS = 157.3      # fp32 vector arithmetic, dense
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


# kernels and sources behind each workload's traffic figures: the figures
# hold while these sources are unchanged
TRAFFIC_SOURCES = {
    "prefill": ("prefill_gfx950.hip", "gdla_device.h"),
    "decode": ("decode_gfx950.hip", "gdla_device.h"),
}


def traffic_kind(workload):
    return "decode" if workload.startswith("dec_") else "prefill"


def traffic_kernels(workload):
    if workload == "dec_swa":
        return ("decode_window_kernel",)
    if workload.startswith("dec_"):
        return ("decode_split_kernel", "decode_combine_kernel")
    return ("prefill_kernel",)


def strip_comments(src):
    """C/C++ source without its comments and blank space: // and /* */
    comments outside string and character literals are dropped, and every run
    of white space becomes one blank."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(kind="prefill"):
    """Hash of the code (comments and spacing aside) of the files a workload's
    kernels are built from."""
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES[kind]:
        src = open(os.path.join(ROOT, "attention_gdla_prefill_amd", "csrc", name), encoding="utf-8").read()
        h.update(strip_comments(src).encode())
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
    `bench.py --workload <workload> --steps 3 --warmup 1 --settle-s 0
    --no-cpu-baseline --no-decode --no-extra --copy-probe` (FETCH_SIZE, then
    WRITE_SIZE): per kernel of the workload the median per dispatch, summed
    over its kernels, each counter scaled by what it reads for the 1 GiB
    device copy that ends the run."""
    import statistics
    kind = traffic_kind(workload)
    kernels = traffic_kernels(workload)
    out = {"kernels": list(kernels), "workload": workload, "source_hash": source_hash(kind)}
    scaled = {}
    for key, run_dir, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(run_dir, counter)
        copy = [v for n, v in rows if "copy" in n.lower()]
        if not copy:
            raise SystemExit("%s: copy dispatch missing" % run_dir)
        per = 0.0
        for kname in kernels:
            vals = [v for n, v in rows if kname in n]
            if not vals:
                raise SystemExit("%s: no %s dispatches" % (run_dir, kname))
            out["%s_kib_per_dispatch_%s" % (key, kname)] = statistics.median(vals)
            per += statistics.median(vals)
        probe = copy[-1]
        scale = (1 << 30) / 1024.0 / probe
        out["%s_kib_per_launch" % key] = per
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


def load_traffic(name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_hash") != source_hash(traffic_kind(name)):
        return None
    return t.get("bytes_per_launch")


class ClockSampler:
    """Samples the GPU's graphics clock (mean over its XCDs) and socket power
    every 50 ms through amdsmi while running; all None where amdsmi is not
    usable.  Informational: the rooflines are priced at the published peaks."""

    def __init__(self, period_s=0.05):
        self.period, self.clk, self.power, self._stop, self._th = period_s, [], [], None, None

    def _read(self, amdsmi, h):
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        if clks:
            self.clk.append(sum(clks) / len(clks))
        pw = m.get("current_socket_power")
        if isinstance(pw, (int, float)):
            self.power.append(pw)

    def start(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            return self
        self._stop = threading.Event()

        def loop():
            try:
                while not self._stop.is_set():
                    self._read(amdsmi, h)
                    self._stop.wait(self.period)
            except Exception:
                pass
            finally:
                try:
                    amdsmi.amdsmi_shut_down()
                except Exception:
                    pass
        self._th = threading.Thread(target=loop, daemon=True)
        self._th.start()
        return self

    def stop(self):
        if self._th is not None:
            self._stop.set()
            self._th.join(timeout=5)
        mean = lambda v: sum(v) / len(v) if v else None
        return {"gfx_clock_mhz": mean(self.clk), "socket_power_w": mean(self.power), "samples": len(self.clk)}


def time_kernel(fn, steps, warmup, stream, settle_s=0.0, sampler=None):
    """Run fn untimed until at least `warmup` launches and `settle_s` seconds
    of steady work have passed, then `steps` timed launches (with `sampler`
    running over them, if given).  Returns (wall ms/step, per-launch HIP-event
    ms list, settle record)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < settle_s:
        fn()
        n += 1
        if n % 4 == 0 or n >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle = {"launches": n, "seconds": round(time.perf_counter() - t0, 3)}
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    if sampler is not None:
        sampler.start()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    if sampler is not None:
        settle = dict(settle, clock=sampler.stop())
    return wall, [a.elapsed_time(b) for a, b in ev], settle


COLD = ("cold: a 512 MB buffer (twice the 256 MB Infinity Cache) is read before each launch, so the "
        "launch's inputs are in no cache and no dirty line is left for it to write back")


def cold_times(call, steps, warmup):
    """Median and per-launch HIP-event times (ms) of `call` with cold caches:
    before each launch a 512 MB buffer is read (a sum over it), which evicts
    the L2s and the Infinity Cache without leaving dirty lines.  Also the
    median with the older protocol, a 512 MB buffer *written* before each
    launch: that leaves up to the Infinity Cache's size of dirty lines, which
    the timed launch then writes back (reported for comparison only)."""
    import torch
    stream = torch.cuda.current_stream()
    sweep = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    dirty = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    res = {}
    for mode in ("clean", "dirty"):
        times = []
        for _ in range(steps):
            if mode == "clean":
                sweep.sum()
            else:
                dirty.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        res[mode] = sorted(times)[len(times) // 2]
    del sweep, dirty
    torch.cuda.empty_cache()
    return res["clean"], res["dirty"]


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline_headline(x, w, budget_s=15.0, out=None):
    """The fp32 oracle, untuned, on random query rows (all 80 heads) of the
    headline workload's own inputs (copied from the GPU), extrapolated to the
    whole launch by unmasked (query, key) pairs.  With the launch's output
    `out`, the same rows are also compared with it (relative L2 and max abs
    over the sampled rows, against the fp32 oracle)."""
    import numpy as np
    import torch
    import oracle
    lib = oracle.library_fp32()
    k = x["k"].float().cpu().numpy()
    v = x["v"].float().cpu().numpy()
    rng = np.random.default_rng(0)
    n, rows, pairs, sec = 8, 0, 0, 0.0
    err2 = ref2 = max_abs = 0.0
    while sec < budget_s:
        rt = np.sort(rng.integers(0, w.T, size=n)).astype(np.int32)
        rb = np.zeros(n, np.int32)
        idx = torch.as_tensor(rt, device=x["k"].device).long()
        q = {key: x[key][0, idx].float().cpu().numpy() for key in ("q_signal", "q_noise", "lam", "gate")}
        t0 = time.perf_counter()
        want = oracle.prefill_rows(k, v, q["q_signal"], q["q_noise"], q["lam"], q["gate"], rb, rt,
                                   window=w.window, lib=lib)
        sec += time.perf_counter() - t0
        if out is not None:
            got = out[0, idx].double().cpu().numpy()
            d = got - np.asarray(want, np.float64)
            err2 += float((d * d).sum())
            ref2 += float((np.asarray(want, np.float64) ** 2).sum())
            max_abs = max(max_abs, float(np.abs(d).max()))
        rows += n
        vis = rt.astype(np.int64) + 1
        if w.window > 0:
            vis = np.minimum(vis, w.window)
        pairs += int(vis.sum())
        n *= 2
    tflops = pairs * N_HEADS * FLOP_PER_PAIR / sec / 1e12
    total = pairs_prefill(w.B, w.T, w.window) * N_HEADS * FLOP_PER_PAIR
    model, ncpu = cpu_info()
    res = {"value": tflops, "unit": "TFLOP/s", "cores": oracle.num_threads(lib), "kind": "oracle",
           "arithmetic": "fp32 (the oracle's source built with fp32 sums and expf)",
           "sample": "%d random query rows (all 80 heads) of the %s workload, %.1f s of compute; "
                     "extrapolated to the whole launch by unmasked pairs" % (rows, w.name, sec),
           "extrapolated_s_per_step": total / (tflops * 1e12),
           "cpu_model": model, "host_cpus": ncpu}
    if out is not None:
        res["parity"] = {"rows": rows, "rel_l2": (err2 / ref2) ** 0.5 if ref2 > 0 else 0.0, "max_abs": max_abs}
    return res


def git_sha():
    """The commit, or where the tree is not a git checkout, "src:" and a hash
    of the library's sources."""
    try:
        import subprocess
        r = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT, capture_output=True, text=True,
                           timeout=10)
        if r.returncode == 0 and r.stdout.strip():
            return r.stdout.strip()
    except Exception:
        pass
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "attention_gdla_prefill_amd", "csrc", "*"))):
        h.update(open(path, "rb").read())
    return "src:" + h.hexdigest()[:12]


class Results:
    """--results FILE: one JSON record per measured configuration, appended as
    it finishes (config, seed, time, rates, fractions of peak, host, git SHA,
    and the sampled parity of the CPU-baseline leg where there is one).  With
    --resume, configurations already recorded in the file for the same commit
    are skipped, so an interrupted run can be continued."""

    def __init__(self, path, resume):
        self.path, self.sha, self.done = path, git_sha(), set()
        if path and resume and os.path.exists(path):
            with open(path) as f:
                for ln in f:
                    try:
                        r = json.loads(ln)
                    except ValueError:
                        continue
                    if r.get("git_sha") == self.sha:
                        self.done.add(r.get("config"))

    def skip(self, name):
        return name in self.done

    def add(self, name, rec):
        if not self.path:
            return
        model, ncpu = cpu_info()
        row = {"config": name, "seed": 0, "time_unix": time.time(), "git_sha": self.sha,
               "host_cpus": ncpu, "cpu_model": model}
        row.update(rec)
        with open(self.path, "a") as f:
            f.write(json.dumps(row) + "\n")
        self.done.add(name)


def cpu_baseline_configs(full=False):
    """The fp32 oracle in full on whole workloads: the tiny config (all threads
    and one thread) and the 128-key window decode; with full=True also the 4K
    prefill, the 32K window prefill and the full-causal decode."""
    import numpy as np
    import torch
    import oracle
    import workload as W
    lib = oracle.library_fp32()
    threads = oracle.num_threads(lib)
    res = {}

    def f32(t):
        return t.float().cpu().numpy()

    def prefill_full(name, n_threads=None):
        w = W.WORKLOADS[name]
        x = W.prefill_inputs(w, seed=0, device="cuda")
        a = {k: f32(t) for k, t in x.items()}
        del x
        torch.cuda.empty_cache()
        if n_threads:
            oracle.set_threads(n_threads, lib)
        t0 = time.perf_counter()
        oracle.prefill(a["q_signal"], a["q_noise"], a["k"], a["v"], a["lam"], a["gate"], window=w.window, lib=lib)
        sec = time.perf_counter() - t0
        oracle.set_threads(threads, lib)
        flops = pairs_prefill(w.B, w.T, w.window) * (w.n_sig + w.n_kv) * FLOP_PER_PAIR
        return {"seconds": sec, "tflops": flops / sec / 1e12, "threads": n_threads or threads}

    def decode_full(name):
        w = W.WORKLOADS[name]
        d = W.decode_inputs(w, seed=0, device="cuda")
        cu = d["cu_seqlens"].cpu().numpy().astype(np.int64)
        lengths = d["lengths"].tolist()
        vis = [min(L, w.window) if w.window > 0 else L for L in lengths]
        # the rows each query sees, packed (positions do not enter the scores)
        keep = torch.cat([torch.arange(int(cu[b + 1]) - vis[b], int(cu[b + 1])) for b in range(w.B)])
        kc = np.empty((len(keep),) + tuple(d["k_cache"].shape[1:]), np.float32)
        vc = np.empty((len(keep),) + tuple(d["v_cache"].shape[1:]), np.float32)
        step = 1 << 18
        for i in range(0, len(keep), step):
            sel = keep[i:i + step].to("cuda")
            kc[i:i + step] = f32(d["k_cache"][sel])
            vc[i:i + step] = f32(d["v_cache"][sel])
        cu_v = np.concatenate([[0], np.cumsum(vis)]).astype(np.int32)
        q = {k: f32(d[k]) for k in ("q_signal", "q_noise", "lam", "gate")}
        del d
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        oracle.decode(q["q_signal"], q["q_noise"], kc, vc, cu_v, q["lam"], q["gate"], window=0, lib=lib)
        sec = time.perf_counter() - t0
        nbytes = decode_bytes(lengths, w.window)
        flops = sum(vis) * N_HEADS * FLOP_PER_PAIR
        return {"seconds": sec, "gbs": nbytes / sec / 1e9, "tflops": flops / sec / 1e12, "threads": threads}

    res["tiny"] = prefill_full("tiny")
    res["tiny_1_thread"] = prefill_full("tiny", n_threads=1)
    res["dec_swa"] = decode_full("dec_swa")
    if full:
        res["pf_full_4k"] = prefill_full("pf_full_4k")
        res["pf_swa_32k"] = prefill_full("pf_swa_32k")
        res["dec_full"] = decode_full("dec_full")
    return res


def bench_prefill(name, steps, warmup, settle_s=0.0, keep_inputs=False, sample_clock=False):
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
    wall, ev, settle = time_kernel(fn, steps, warmup, stream, settle_s,
                                   sampler=ClockSampler() if sample_clock else None)
    kern_ms = sum(ev) / len(ev)
    flops = pairs_prefill(w.B, w.T, w.window, P) * N_HEADS * FLOP_PER_PAIR
    nbytes = prefill_bytes(w.B, w.T, prefix=P)
    res = {"wall_ms": wall, "kernel_ms": kern_ms, "kernel_ms_min": min(ev), "kernel_ms_max": max(ev),
           "flops": flops, "bytes": nbytes, "settle": settle,
           "tflops": flops / (kern_ms * 1e-3) / 1e12, "gbs": nbytes / (kern_ms * 1e-3) / 1e9}
    if keep_inputs:
        res["inputs"] = x
        res["out"] = out
    else:
        del x, out
        torch.cuda.empty_cache()
    return res


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
    call = lambda: gdla.prep(d["q_signal"], d["q_noise"], d["k_rope"], d["k"], d["x"], d["w_lambda"],
                             d["gate_pre"], lam_out=lam, gate_out=gate)
    ms, ms_dirty = cold_times(call, steps, warmup)
    nbytes = prep_bytes(w)
    del d, lam, gate
    torch.cuda.empty_cache()
    return {"kernel_ms": ms, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "cache": COLD,
            "kernel_ms_dirty_flush": ms_dirty}


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
    wall, ev, _ = time_kernel(fn, steps, warmup, stream)
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
    call = lambda: gdla.decode(d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"],
                               d["cu_seqlens"], max_len, d["lam"], d["gate"], window=w.window,
                               out=out, workspace=ws)
    kern_ms, ms_dirty = cold_times(call, steps, warmup)
    nbytes = decode_bytes(lengths, w.window)
    del d, out, ws
    torch.cuda.empty_cache()
    return {"kernel_ms": kern_ms, "bytes": nbytes, "gbs": nbytes / (kern_ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "cache": COLD,
            "kernel_ms_dirty_flush": ms_dirty}


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
    call = lambda: gdla.decode_latent(d["q_signal"], d["q_noise"], d["latent"], d["cu_seqlens"], max_len,
                                      d["w_uk"], d["w_uv"], d["lam"], d["gate"], window=w.window,
                                      out=out, workspace=ws)
    kern_ms, ms_dirty = cold_times(call, steps, warmup)
    nbytes = decode_latent_bytes(lengths, w.window)
    expanded = decode_bytes(lengths, w.window)
    del d, out, ws
    torch.cuda.empty_cache()
    res = {"kernel_ms": kern_ms, "bytes": nbytes, "gbs": nbytes / (kern_ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "expanded_equivalent_gbs": expanded / (kern_ms * 1e-3) / 1e9, "cache": COLD,
           "kernel_ms_dirty_flush": ms_dirty}
    if 1 <= w.window <= 128:
        # the one-launch window kernel does its weight products on the vector
        # ALUs: per (sequence, KV head) q~ = W_uk^T q^C for 5 heads (5 x 128 x 512
        # multiply-adds), o~ = sum_s p_s c_s over the visible rows (5 x rows x
        # 512) and D = W_uv d~ for 4 heads (4 x 512 x 128); its bound is the fp32
        # vector peak, beside which the bytes are few
        rows = sum(min(L, w.window) for L in lengths)
        flops = 2 * 512 * (w.B * w.n_kv * (5 * 128 + 4 * 128) + rows * w.n_kv * 5)
        res.update(valu_flops=flops, valu_tflops=flops / (kern_ms * 1e-3) / 1e12,
                   valu_frac=flops / (kern_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS)
    return res


PREFILL_WORKLOADS = ("pf_full_128k", "pf_full_4k", "pf_swa_32k", "pf_prefix_4k_32k", "pf_swa_rank")
EXTRA_NAMES = ("pf_full_4k", "pf_swa_32k", "pf_full_128k", "pf_prefix_4k_32k", "pf_swa_rank", "dec_swa",
               "dec_latent_full", "dec_latent_swa", "prep_4k", "prep_swa_32k", "bwd_4k")
# measured only when named in --extras
OPT_IN_EXTRAS = ("bwd_swa_32k",)


def decode_roofline(r, name):
    traffic = load_traffic(name)
    return {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": r["gbs"] / PEAK_HBM_GBS, "traffic": traffic, "workload": name,
            "kernel": " + ".join(traffic_kernels(name)), "kernel_ms": r["kernel_ms"],
            "kernel_ms_dirty_flush": r["kernel_ms_dirty_flush"],
            "algorithmic_bytes_per_launch": r["bytes"], "cache": r["cache"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="untimed steady work before the timed steps, in seconds (with at least "
                         "--warmup launches): the GPU clock needs ~0.1 s of load to settle")
    ap.add_argument("--workload", default="pf_full_128k", choices=PREFILL_WORKLOADS + ("dec_full", "dec_swa"))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the fp32 oracle in full on the 4K prefill, the 32K window prefill "
                         "and the full-causal decode (about a minute of CPU)")
    ap.add_argument("--no-decode", action="store_true", help="skip the full-causal decode roofline")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--extras", default=",".join(EXTRA_NAMES),
                    help="comma-separated extra workloads to time (a profile of one workload names just that one); "
                         "also %s, measured only when named" % ", ".join(OPT_IN_EXTRAS))
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--peaks", action="store_true",
                    help="also time a bf16 8192^3 GEMM (hipBLASLt via torch) and a 1 GiB device "
                         "copy: achievable-rate references, reported under 'peaks'")
    ap.add_argument("--results", metavar="FILE",
                    help="append one JSON record per measured configuration to FILE")
    ap.add_argument("--resume", action="store_true",
                    help="with --results: skip the configurations FILE already holds for this commit")
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
        if name not in EXTRA_NAMES + OPT_IN_EXTRAS:
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
    results = Results(args.results, args.resume)
    print("[bench] %s steps=%d warmup=%d settle=%.2fs" % (args.workload, args.steps, args.warmup, args.settle_s),
          file=sys.stderr, flush=True)
    decode_main = args.workload.startswith("dec_")
    cpu = None
    if decode_main:
        main_res = bench_decode(args.workload, args.steps, args.warmup)
        results.add(args.workload, {"time_ms": main_res["kernel_ms"], "gbs": main_res["gbs"],
                                    "hbm_frac": main_res["gbs"] / PEAK_HBM_GBS})
    else:
        main_res = bench_prefill(args.workload, args.steps, args.warmup, args.settle_s,
                                 keep_inputs=not args.no_cpu_baseline, sample_clock=True)
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline (fp32 oracle, sampled rows of %s)" % args.workload, file=sys.stderr,
                  flush=True)
            cpu = cpu_baseline_headline(main_res["inputs"], w, out=main_res["out"])
            del main_res["inputs"], main_res["out"]
            torch.cuda.empty_cache()
        results.add(args.workload, {
            "time_ms": main_res["kernel_ms"], "tflops": main_res["tflops"], "gbs": main_res["gbs"],
            "mfma_frac": main_res["tflops"] / PEAK_BF16_TFLOPS, "hbm_frac": main_res["gbs"] / PEAK_HBM_GBS,
            "oracle_s_per_step": cpu["extrapolated_s_per_step"] if cpu else None,
            "rel_l2": cpu["parity"]["rel_l2"] if cpu and "parity" in cpu else None,
            "max_abs": cpu["parity"]["max_abs"] if cpu and "parity" in cpu else None})

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    dec_roof = None
    if not args.no_decode and not decode_main:
        print("[bench] decode roofline dec_full", file=sys.stderr, flush=True)
        dec_roof = decode_roofline(bench_decode("dec_full", 10, 2), "dec_full")
        results.add("dec_full", {"time_ms": dec_roof["kernel_ms"], "gbs": dec_roof["achieved"],
                                 "hbm_frac": dec_roof["frac"]})

    extra = {}
    for name in ("pf_full_4k", "pf_swa_32k", "pf_full_128k", "pf_prefix_4k_32k", "pf_swa_rank"):
        if name == args.workload or name not in wanted or results.skip(name):
            continue
        print("[bench] extra %s" % name, file=sys.stderr, flush=True)
        steps, warm = (3, 1) if name == "pf_full_128k" else (50, 10)
        r = bench_prefill(name, steps, warm, args.settle_s)
        extra[name] = {"tflops": r["tflops"], "mfma_frac": r["tflops"] / PEAK_BF16_TFLOPS,
                       "gbs": r["gbs"], "hbm_frac": r["gbs"] / PEAK_HBM_GBS, "kernel_ms": r["kernel_ms"],
                       "steps": steps, "settle": r["settle"], "traffic": load_traffic(name)}
        results.add(name, {"time_ms": r["kernel_ms"], "tflops": r["tflops"], "gbs": r["gbs"],
                           "mfma_frac": extra[name]["mfma_frac"], "hbm_frac": extra[name]["hbm_frac"]})
    for name in ("dec_swa", "dec_latent_full", "dec_latent_swa"):
        if name == args.workload or name not in wanted or results.skip(name):
            continue
        print("[bench] extra %s" % name, file=sys.stderr, flush=True)
        fn = bench_decode_latent if name.startswith("dec_latent") else bench_decode
        extra[name] = fn(name, 10, 2)
        if name == "dec_swa":
            extra[name]["traffic"] = load_traffic(name)
        results.add(name, {"time_ms": extra[name]["kernel_ms"], "gbs": extra[name]["gbs"],
                           "hbm_frac": extra[name]["hbm_frac"]})
    for name, shape in (("prep_4k", "pf_full_4k"), ("prep_swa_32k", "pf_swa_32k")):
        if name not in wanted or results.skip(name):
            continue
        print("[bench] extra %s" % name, file=sys.stderr, flush=True)
        extra[name] = dict(bench_prep(shape, 20, 5), shapes=shape)
        results.add(name, {"time_ms": extra[name]["kernel_ms"], "gbs": extra[name]["gbs"],
                           "hbm_frac": extra[name]["hbm_frac"]})
    if "bwd_4k" in wanted and not results.skip("bwd_4k"):
        print("[bench] extra bwd_4k", file=sys.stderr, flush=True)
        extra["bwd_4k"] = dict(bench_backward("pf_full_4k", 20, 10), shapes="pf_full_4k")
        results.add("bwd_4k", {"time_ms": extra["bwd_4k"]["ms"], "tflops": extra["bwd_4k"]["tflops"],
                               "mfma_frac": extra["bwd_4k"]["mfma_frac"]})
    if "bwd_swa_32k" in wanted and not results.skip("bwd_swa_32k"):
        print("[bench] extra bwd_swa_32k", file=sys.stderr, flush=True)
        extra["bwd_swa_32k"] = dict(bench_backward("pf_swa_32k", 10, 3), shapes="pf_swa_32k")
        results.add("bwd_swa_32k", {"time_ms": extra["bwd_swa_32k"]["ms"], "tflops": extra["bwd_swa_32k"]["tflops"],
                                    "mfma_frac": extra["bwd_swa_32k"]["mfma_frac"]})

    peaks = measured_peaks() if args.peaks else None

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: whole small configs%s" % (" and --cpu-full" if args.cpu_full else ""),
              file=sys.stderr, flush=True)
        configs = cpu_baseline_configs(full=args.cpu_full)
        if cpu is None:
            import oracle
            model, ncpu = cpu_info()
            cpu = {"value": configs["dec_swa"]["gbs"], "unit": "GB/s", "kind": "oracle",
                   "cores": oracle.num_threads(oracle.library_fp32()),
                   "sample": "the whole dec_swa workload", "cpu_model": model, "host_cpus": ncpu}
        cpu["configs"] = configs

    if decode_main:
        value, unit = main_res["gbs"], "GB/s"
        roof = decode_roofline(main_res, args.workload)
        ms_per_step = main_res["kernel_ms"]
        config = {"workload": "%s: decode, %d sequences, cached lengths U{%d..%d}, %d KV / %d signal / %d noise "
                              "heads, qk 192 / v 128, %s, cold cache"
                              % (w.name, w.B, w.len_lo, w.len_hi, w.n_kv, w.n_sig, w.n_kv,
                                 "full causal" if w.window == 0 else "window %d" % w.window),
                  "global_batch": w.B, "parallelism": "single GPU"}
    else:
        value, unit = main_res["flops"] / (main_res["wall_ms"] * 1e-3) / 1e12, "TFLOP/s"
        ms_per_step = main_res["wall_ms"]
        roof = {"bound": "mfma", "achieved": main_res["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": main_res["tflops"] / PEAK_BF16_TFLOPS,
                "traffic": load_traffic(args.workload), "kernel": "prefill_kernel",
                "kernel_ms": main_res["kernel_ms"], "kernel_ms_min": main_res["kernel_ms_min"],
                "kernel_ms_max": main_res["kernel_ms_max"], "flops_per_launch": main_res["flops"],
                "algorithmic_bytes_per_launch": main_res["bytes"],
                "hbm_frac_algorithmic": main_res["gbs"] / PEAK_HBM_GBS}
        clk = (main_res.get("settle") or {}).get("clock") or {}
        if clk.get("gfx_clock_mhz"):
            # the published peak assumes 2.4 GHz; the same kernel's share of
            # the peak at the clock the box held over the timed launches
            roof["gfx_clock_mhz"] = clk["gfx_clock_mhz"]
            roof["frac_at_measured_clock"] = roof["frac"] * PEAK_CLOCK_MHZ / clk["gfx_clock_mhz"]
        config = {"workload": "%s: prefill B=%d T=%d, %d KV / %d signal / %d noise heads, qk 192 / v 128, %s"
                              % (w.name, w.B, w.T, w.n_kv, w.n_sig, w.n_kv,
                                 "full causal" if w.window == 0 else "window %d" % w.window),
                  "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU"}
    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": main_res.get("settle"),
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "decode_roofline": dec_roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if peaks is not None:
        line["peaks"] = peaks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
