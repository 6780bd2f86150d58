"""Throughput of the N:M mask layer on one MI355X.

One step = the whole hot path over one LLaMA-2-7B-shaped decoder layer (q, k, v, o 4096x4096;
gate, up 11008x4096; down 4096x11008; 202,375,168 bf16 weights, fp32 logits, 2:4, kappa = 100,
tau = 4, logits from the magnitude prior): forward (soft mask times frozen weights), backward to
the logits, hard-mask extraction with compressed pack, and unpack, for all seven matrices.
Inputs are synthetic, seeded, generated on the GPU and resident in HBM before timing starts.

Prints one JSON line.  `value` is the metric: masked weights per second of the forward and
backward passes, timed with HIP events inside each of the K whole-path steps (ms_per_step is the
whole step).  Alongside: the per-pass breakdown (each pass timed on its own, and each pass's
share of the timed steps), the roofline of the dominant kernel (HIP-event timing, algorithmic
bytes), the 32-layer annealed sweep (32 such layers x 10 steps of forward,
backward and harden/pack, tau 4 -> 0.05, kappa 100 -> 500), and the oracle's CPU baseline on a
bounded sample on every host core available.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-sweep]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "masked weights/sec fwd+bwd (GB/s, % of HBM peak) on 7B-shaped 2:4 layers"
N, M, K = 2, 4, 6
KAPPA, TAU = 100.0, 4.0
WB = 2  # bf16 bytes


def bytes_per_weight(wb=WB, n=N, m=M, k=K):
    """Algorithmic HBM bytes per weight of each pass (what the pass must read and write)."""
    fwd = 2 * wb + 4 * k / m                       # read w and logits, write w_masked
    bwd = 2 * wb + 8 * k / m                       # read w, grad, logits; write dlogits
    idx_bits = (m - 1).bit_length()
    pack = wb + 4 * k / m + wb * n / m + n * idx_bits / (8 * m)   # read w, logits; write packed
    unpack = wb * n / m + n * idx_bits / (8 * m) + wb              # read packed; write dense
    return {"fwd": fwd, "bwd": bwd, "harden_pack": pack, "unpack": unpack}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", default="llama7b_layer",
                   choices=["llama7b_layer", "sweep32", "general_nm", "nemotron_pack", "single256",
                            "prior_init", "monitor", "spmm", "wreg"],
                   help="llama7b_layer (default): one LLaMA-2-7B-shaped layer per step; sweep32: 32 such "
                        "layers x 10 annealed steps of fwd+bwd+pack; general_nm: 4096x11008 with 1:4, 2:8, "
                        "4:8; nemotron_pack: pack+unpack of every Nemotron-15B-shaped matrix; single256: "
                        "one 256x256 fp32 weight (latency-bound); prior_init: magnitude-prior "
                        "logit initialisation; monitor: forward with the fused Fig. 5 monitors; spmm: "
                        "sparse x dense product on the packed weights; wreg: backward with the fused "
                        "weight regulariser")
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--kernel-reps", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="leave out the 32-layer annealed sweep")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="least CPU time of the baseline")
    p.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                   help="print the path kernels' average durations from rocprofv3 --stats output")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run 4 plain 1 GiB device copies (counter calibration under a profiler)")
    return p.parse_args()


def kernel_prior(w, n, m):
    """Prior candidate of every group from the library's own magnitude-prior kernel."""
    import semi_structured_sparsity_amd as S
    return S.nm_prior_init(w, n, m, 1.0, with_idx=True)[1]


def make_layer(dev):
    import torch

    import nm_synth
    mats = []
    for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
        seed = nm_synth.input_seed(2, 0, i)
        w, L, G = nm_synth.matrix_inputs(rows, cols, N, M, torch.bfloat16, 0.02, seed,
                                         logits="prior", device=dev, prior=kernel_prior)
        mats.append(dict(name=name, rows=rows, cols=cols, seed=seed, w=w, L=L, G=G,
                         out=torch.empty_like(w),
                         dl=torch.empty_like(L),
                         values=torch.empty((rows, cols // M * N), dtype=w.dtype, device=dev),
                         indices=torch.empty((rows, cols // 32), dtype=torch.int32, device=dev),
                         dense=torch.empty_like(w)))
    return mats


def run_pass(S, mt, which, step):
    if which == "fwd":
        S.nm_mask_forward(mt["w"], mt["L"], N, M, KAPPA, TAU, mt["seed"], step, out=mt["out"])
    elif which == "bwd":
        S.nm_mask_backward(mt["w"], mt["L"], mt["G"], N, M, KAPPA, TAU, mt["seed"], step, out=mt["dl"])
    elif which == "harden_pack":
        # values and indices only: the optional hard-index bytes are not part of the pass
        S.nm_mask_harden_pack(mt["w"], mt["L"], N, M, out=(mt["values"], mt["indices"], None))
    else:
        S.nm_unpack(mt["values"], mt["indices"], mt["cols"], N, M, out=mt["dense"])


PASSES = ("fwd", "bwd", "harden_pack", "unpack")


def step_all(S, mats, step, marks=None):
    # pass-major, as in a training step (all forwards, then all backwards, ...): each pass moves
    # >= 2 GB across the seven matrices, so no pass finds a matrix's data left in the 256 MB
    # last-level cache by the previous pass over the same matrix.  `marks`: len(PASSES) + 1
    # events recorded on the launch stream at the pass boundaries (before the forward, after
    # each pass).
    if marks is not None:
        marks[0].record()
    for i, p in enumerate(PASSES):
        for mt in mats:
            run_pass(S, mt, p, step)
        if marks is not None:
            marks[i + 1].record()


def host_cores():
    """(threads to use, what the host reports): all cores this process may run on -- the CPU
    affinity set, capped by a cgroup CPU quota when one is set -- next to os.cpu_count()."""
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    threads = min(affinity, quota) if quota else affinity
    return threads, {"os_cpu_count": os.cpu_count(), "affinity": affinity, "cgroup_cpu_quota": quota}


def cpu_baseline(min_seconds=10.0, max_passes=8):
    """The oracle over the same layer (same shapes, generators and parameters, CPU copies):
    forward, backward, pack and unpack of all seven matrices, repeated over successive steps
    until at least `min_seconds` of CPU time has been spent, on every core available to the
    process.  Returns weights/s of whole steps, and the forward + backward alone."""
    import torch

    import nm_synth
    import oracle
    threads, host = host_cores()
    mats = []
    for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
        seed = nm_synth.input_seed(2, 0, i)
        w = nm_synth.normal((rows, cols), 0.02, 3 * seed, torch.bfloat16)
        prior = torch.from_numpy(oracle.prior_init(w, N, M)[1].astype("int64"))
        mats.append((seed, cols, w, nm_synth.prior_logits(prior, K, 3 * seed + 1),
                     nm_synth.normal((rows, cols), 1.0, 3 * seed + 2, torch.bfloat16)))
    total_w, elapsed, fb_elapsed, passes = 0, 0.0, 0.0, 0
    while passes < max_passes and (passes == 0 or elapsed < min_seconds):
        for seed, cols, w, L, G in mats:
            t0 = time.perf_counter()
            oracle.forward(w, L, N, M, KAPPA, TAU, seed, passes, nthreads=threads)
            oracle.backward(w, L, G, N, M, KAPPA, TAU, seed, passes, nthreads=threads)
            t1 = time.perf_counter()
            v, idx, _ = oracle.pack(w, L, N, M, nthreads=threads)
            oracle.unpack(v, idx, cols, N, M, nthreads=threads)
            elapsed += time.perf_counter() - t0
            fb_elapsed += t1 - t0
            total_w += w.numel()
        passes += 1
    # the same four passes on one thread over the first matrix (q, 4096x4096)
    seed, cols, w, L, G = mats[0]
    t0 = time.perf_counter()
    oracle.forward(w, L, N, M, KAPPA, TAU, seed, 0, nthreads=1)
    oracle.backward(w, L, G, N, M, KAPPA, TAU, seed, 0, nthreads=1)
    v, idx, _ = oracle.pack(w, L, N, M, nthreads=1)
    oracle.unpack(v, idx, cols, N, M, nthreads=1)
    t1 = time.perf_counter() - t0
    return {"value": total_w / fb_elapsed, "unit": "weights/s", "cores": oracle.threads_used(threads),
            "kind": "oracle", "host": host,
            "sample": f"{passes} step(s) of the whole layer ({total_w} weight-passes) in binary64 on "
                      f"{threads} threads: value = forward + backward ({fb_elapsed:.1f} s), "
                      f"whole_step = fwd+bwd+harden_pack+unpack ({elapsed:.1f} s)",
            "whole_step": {"value": total_w / elapsed, "unit": "weights/s"},
            "single_thread": {"value": w.numel() / t1, "unit": "weights/s",
                              "sample": f"fwd+bwd+harden_pack+unpack of the 4096x4096 q matrix on 1 thread, "
                                        f"{t1:.1f} s"}}


def copy_ceiling(dev, reps=10):
    """GB/s (read + write) of the library's plain flat copy over 1 GiB: the streaming ceiling
    of this GPU, measured in the same run."""
    import torch

    import semi_structured_sparsity_amd as S
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t = _elapsed_ms(lambda r: S.nm_debug_copy(src, dst), reps=reps)
    del src, dst
    return 2 * (1 << 30) / (t * 1e-3) / 1e9


# ---------------------------------------------------------------------------------------------
# rocprofv3 summaries (run on the CSV output of the commands printed in profiles/)

KERNELS = {"fwd": "k_forward<2, 4, nm::BF16, 0>", "bwd": "k_backward<2, 4, nm::BF16, 0>",
           "harden_pack": "k_pack_bytes<2, nm::BF16>", "unpack": "k_unpack_bytes<2, nm::BF16>"}
COPY_BYTES = 1 << 30  # the --copy-calibration copies


def kernel_source_hash():
    """Hash of the sources of the path's kernels (their translation units and the device headers
    they include), so stored counter readings can be matched to the kernels they were taken on."""
    import hashlib
    import semi_structured_sparsity_amd.build as b
    h = hashlib.sha256()
    for name in ("nm_forward.hip", "nm_backward.hpp", "nm_backward.hip", "nm_backward_wreg.hip", "nm_pack.hip",
                 "nm_layer.hpp", "nm_device.hpp"):
        h.update(open(os.path.join(b.CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def _rows(csv_path):
    import csv
    with open(csv_path) as f:
        return list(csv.DictReader(f))


def summarize_trace(stats_csv):
    """Average launch duration of each path kernel from a --kernel-trace --stats run."""
    out = {}
    for row in _rows(stats_csv):
        for p, k in KERNELS.items():
            if k in row["Name"]:
                out[p] = {"kernel": k, "calls": int(row["Calls"]), "avg_us": float(row["AverageNs"]) / 1e3}
    return out


def summarize_pmc(fetch_csv, write_csv):
    """HBM bytes per dispatch of each path kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each divided by what the same counter reads, per byte, for the 1 GiB calibration copies."""
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _rows(path) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]
                  and float(r["Counter_Value"]) * 1024 > 0.4 * COPY_BYTES]
        if not copies:
            raise SystemExit(f"no calibration copy in {path}")
        scale = (sum(copies) / len(copies)) / COPY_BYTES
        for p, k in KERNELS.items():
            vals = [float(r["Counter_Value"]) * 1024 for r in rows if k in r["Kernel_Name"]]
            if vals:
                res.setdefault(p, {})[counter] = {"dispatches": len(vals), "copy_scale": round(scale, 4),
                                                  "bytes_per_dispatch": sum(vals) / len(vals) / scale}
    return res


def write_traffic(fetch_csv, write_csv, out_json):
    pmc = summarize_pmc(fetch_csv, write_csv)
    doc = {"source_hash": kernel_source_hash(), "unit": "bytes per launch (average over the layer)",
           "kernels": {p: v["FETCH_SIZE"]["bytes_per_dispatch"] + v["WRITE_SIZE"]["bytes_per_dispatch"]
                       for p, v in pmc.items() if "FETCH_SIZE" in v and "WRITE_SIZE" in v},
           "detail": pmc}
    with open(out_json, "w") as f:
        json.dump(doc, f, indent=1)
    return doc


def stored_traffic(kernel):
    """Measured bytes per launch of `kernel` if the counters were taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    if doc.get("source_hash") != kernel_source_hash():
        return None
    v = doc.get("kernels", {}).get(kernel)
    return None if v is None else round(v, 0)


# ---------------------------------------------------------------------------------------------
# other workloads (reported separately; the default line is the LLaMA-7B layer)

def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _elapsed_ms(fn, reps=1, warm=None, warm_seconds=0.25):
    """Average ms of fn(r) over `reps` calls, after untimed calls that bring the GPU to its
    working clocks: at least `warm` of them (default: reps) and at least `warm_seconds` of
    wall time (the clocks ramp up over tens of milliseconds of sustained load)."""
    import torch
    t0, r = time.perf_counter(), 0
    while r < (reps if warm is None else warm) or time.perf_counter() - t0 < warm_seconds:
        fn(r)
        r += 1
        if r % 8 == 0:
            torch.cuda.synchronize()
    a, b = _events()
    torch.cuda.synchronize()
    a.record()
    for r in range(reps):
        fn(r)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def workload_sweep32(args):
    """32 LLaMA-7B-shaped layers resident in HBM; 10 steps with tau 4 -> 0.05 and kappa
    100 -> 500 (linear), offset = step; per step the forward of every matrix (layers 0..31),
    then the backward (layers 31..0), then harden+pack."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    layers = []
    for layer in range(nm_synth.LAYERS):
        mats = []
        for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
            seed = nm_synth.input_seed(3, layer, i)
            w, L, G = nm_synth.matrix_inputs(rows, cols, N, M, torch.bfloat16, 0.02, seed,
                                             logits="prior", device=dev, prior=kernel_prior)
            mats.append(dict(rows=rows, cols=cols, seed=seed, w=w, L=L, G=G))
        layers.append(mats)
    outs = {}
    for name, rows, cols in nm_synth.LLAMA2_7B_LAYER:
        outs[(rows, cols)] = dict(out=torch.empty((rows, cols), dtype=torch.bfloat16, device=dev),
                                  dl=torch.empty((rows, cols // M, K), device=dev),
                                  values=torch.empty((rows, cols // M * N), dtype=torch.bfloat16, device=dev),
                                  indices=torch.empty((rows, cols // 32), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()

    def step(s):
        f = s / 9.0
        kappa, tau = 100.0 + 400.0 * f, 4.0 + (0.05 - 4.0) * f
        for mats in layers:
            for mt in mats:
                o = outs[(mt["rows"], mt["cols"])]
                S.nm_mask_forward(mt["w"], mt["L"], N, M, kappa, tau, mt["seed"], s, out=o["out"])
        for mats in reversed(layers):
            for mt in mats:
                o = outs[(mt["rows"], mt["cols"])]
                S.nm_mask_backward(mt["w"], mt["L"], mt["G"], N, M, kappa, tau, mt["seed"], s, out=o["dl"])
        for mats in layers:
            for mt in mats:
                o = outs[(mt["rows"], mt["cols"])]
                S.nm_mask_harden_pack(mt["w"], mt["L"], N, M, out=(o["values"], o["indices"], None))

    def step_fused(s):
        # the same outputs, with the forward and the pack of each matrix in one call
        f = s / 9.0
        kappa, tau = 100.0 + 400.0 * f, 4.0 + (0.05 - 4.0) * f
        for mats in layers:
            for mt in mats:
                o = outs[(mt["rows"], mt["cols"])]
                S.nm_mask_forward_pack(mt["w"], mt["L"], N, M, kappa, tau, mt["seed"], s,
                                       out=(o["out"], o["values"], o["indices"], None))
        for mats in reversed(layers):
            for mt in mats:
                o = outs[(mt["rows"], mt["cols"])]
                S.nm_mask_backward(mt["w"], mt["L"], mt["G"], N, M, kappa, tau, mt["seed"], s, out=o["dl"])

    step(0)  # warm-up
    ms = _elapsed_ms(step, reps=10)  # the 10 annealed steps, timed together
    step_fused(0)
    ms_fused = _elapsed_ms(step_fused, reps=10)
    weights = nm_synth.LAYERS * nm_synth.layer_weights(nm_synth.LLAMA2_7B_LAYER)
    bpw = bytes_per_weight()
    byts = weights * (bpw["fwd"] + bpw["bwd"] + bpw["harden_pack"])
    # one pass over w and the logits for both: the pack's second read of them is not needed
    byts_fused = weights * (bpw["fwd"] + bpw["bwd"] + bpw["harden_pack"] - WB - 4 * K / M)
    return {"metric": "masked weights/sec fwd+bwd+pack over a 32-layer 7B-shaped sweep", "value": weights / (ms * 1e-3),
            "unit": "weights/s", "ms_per_step": round(ms, 3), "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
            "forward_pack_in_one_call": {
                "weights_per_s": weights / (ms_fused * 1e-3), "ms_per_step": round(ms_fused, 3),
                "bytes_per_weight": bpw["fwd"] + bpw["bwd"] + bpw["harden_pack"] - WB - 4 * K / M,
                "GBps": round(byts_fused / (ms_fused * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * byts_fused / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
                "speedup": round(ms / ms_fused, 3)},
            "config": {"workload": "32 LLaMA-2-7B-shaped layers (6,476,005,376 bf16 weights), 2:4, 10 annealed "
                                   "steps (tau 4->0.05, kappa 100->500), fwd+bwd+harden_pack per step",
                       "steps_timed": 10}}


def workload_general_nm(args):
    """4096x11008 bf16, 1:4 / 2:8 / 4:8, kappa 100, tau 1: every pass timed on its own.  Each
    pass cycles through copies of its inputs and outputs that together exceed 600 MB, so that
    every call reads and writes HBM rather than the 256 MB last-level cache."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    rows, cols = 4096, 11008
    res = {}
    for n, m in ((1, 4), (2, 8), (4, 8)):
        k = S.num_candidates(n, m)
        seed = nm_synth.input_seed(5, 0, m * 10 + n)
        w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, seed, device=dev)
        out, dl = torch.empty_like(w), torch.empty_like(L)
        wpr = S.index_words_per_row(cols, n, m)
        values = torch.empty((rows, cols // m * n), dtype=w.dtype, device=dev)
        idx = torch.empty((rows, wpr), dtype=torch.int32, device=dev)
        dense = torch.empty_like(w)
        bpw = bytes_per_weight(2, n, m, k)
        S.nm_mask_harden_pack(w, L, n, m, out=(values, idx, None))  # unpack's input
        base = {"fwd": (w, L, out), "bwd": (w, L, G, dl), "harden_pack": (w, L, values, idx),
                "unpack": (values, idx, dense)}
        entry = {}
        for p in ("fwd", "bwd", "harden_pack", "unpack"):
            ncopy = -(-600_000_000 // int(bpw[p] * rows * cols))
            sets = [base[p]] + [tuple(t.clone() for t in base[p]) for _ in range(ncopy - 1)]
            if p == "fwd":
                fn = lambda r: (lambda a: S.nm_mask_forward(a[0], a[1], n, m, 100.0, 1.0, seed, r, out=a[2]))(sets[r % ncopy])
            elif p == "bwd":
                fn = lambda r: (lambda a: S.nm_mask_backward(a[0], a[1], a[2], n, m, 100.0, 1.0, seed, r, out=a[3]))(sets[r % ncopy])
            elif p == "harden_pack":
                fn = lambda r: (lambda a: S.nm_mask_harden_pack(a[0], a[1], n, m, out=(a[2], a[3], None)))(sets[r % ncopy])
            else:
                fn = lambda r: (lambda a: S.nm_unpack(a[0], a[1], cols, n, m, out=a[2]))(sets[r % ncopy])
            for r in range(ncopy):
                fn(r)
            us = _elapsed_ms(fn, reps=max(args.kernel_reps, 2 * ncopy)) * 1e3
            gbps = bpw[p] * rows * cols / (us * 1e-6) / 1e9
            entry[p] = {"avg_launch_us": round(us, 2), "bytes_per_weight": round(bpw[p], 4),
                        "GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
                        "copies": ncopy}
            del sets
            torch.cuda.empty_cache()
        fb = entry["fwd"]["avg_launch_us"] + entry["bwd"]["avg_launch_us"]
        entry["fwd_bwd_weights_per_s"] = rows * cols / (fb * 1e-6)
        res[f"{n}:{m}"] = entry
        del w, L, G, out, dl, values, idx, dense
        torch.cuda.empty_cache()
    return {"metric": "per-pass throughput, general N:M on a 4096x11008 bf16 weight", "unit": "GB/s",
            "config": {"workload": "4096x11008 bf16, kappa=100, tau=1, logits N(0,1)"}, "results": res}


def workload_nemotron_pack(args):
    """Every Nemotron-15B-shaped matrix (32 layers x 6, bf16, logits N(0,1)): harden+pack and
    unpack, generated and timed layer by layer."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    t_pack = t_unpack = 0.0
    weights = 0
    for layer in range(nm_synth.LAYERS):
        mats = []
        for i, (name, rows, cols) in enumerate(nm_synth.NEMOTRON_15B_LAYER):
            seed = nm_synth.input_seed(4, layer, i)
            w, L, _ = nm_synth.matrix_inputs(rows, cols, N, M, torch.bfloat16, 0.015, seed,
                                             with_grad=False, device=dev)
            mats.append((w, L, cols, torch.empty((rows, cols // 2), dtype=w.dtype, device=dev),
                         torch.empty((rows, cols // 32), dtype=torch.int32, device=dev), torch.empty_like(w)))
            weights += rows * cols
        def pack(r):
            for w, L, c, v, ix, d in mats:
                S.nm_mask_harden_pack(w, L, N, M, out=(v, ix, None))

        def unpack(r):
            for w, L, c, v, ix, d in mats:
                S.nm_unpack(v, ix, c, N, M, out=d)

        pack(0)  # untimed: first touch of this layer's freshly allocated buffers
        unpack(0)
        t_pack += _elapsed_ms(pack)
        t_unpack += _elapsed_ms(unpack)
        del mats
    bpw = bytes_per_weight()
    res = {}
    for p, t in (("harden_pack", t_pack), ("unpack", t_unpack)):
        gbps = bpw[p] * weights / (t * 1e-3) / 1e9
        res[p] = {"ms": round(t, 3), "GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
    return {"metric": "harden+pack and unpack over every Nemotron-15B-shaped matrix", "unit": "GB/s",
            "config": {"workload": "32 layers x (q,k,v,o 6144x6144, up 24576x6144, down 6144x24576), "
                                   "14,495,514,624 bf16 weights, 2:4"}, "weights": weights, "results": res}


def workload_single256(args):
    """One 256x256 fp32 weight, 2:4, kappa 100, tau 4, seed 0: launch-latency-bound."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    w, L, G = nm_synth.matrix_inputs(256, 256, N, M, torch.float32, 0.02, nm_synth.input_seed(1, 0, 0))
    w, L, G = w.cuda(), L.cuda(), G.cuda()
    out, dl = torch.empty_like(w), torch.empty_like(L)
    v = torch.empty((256, 128), device="cuda")
    ix = torch.empty((256, 8), dtype=torch.int32, device="cuda")
    d = torch.empty_like(w)
    calls = {"fwd": lambda r: S.nm_mask_forward(w, L, N, M, 100.0, 4.0, 0, r, out=out),
             "bwd": lambda r: S.nm_mask_backward(w, L, G, N, M, 100.0, 4.0, 0, r, out=dl),
             "harden_pack": lambda r: S.nm_mask_harden_pack(w, L, N, M, out=(v, ix, None)),
             "unpack": lambda r: S.nm_unpack(v, ix, 256, N, M, out=d)}
    res = {}
    for p, fn in calls.items():
        fn(0)
        res[p] = {"avg_launch_us": round(_elapsed_ms(fn, reps=200) * 1e3, 2)}

    # the four passes captured into one HIP graph (same arguments on every replay), which takes
    # the host's per-call cost out of the step
    def step(r):
        for fn in calls.values():
            fn(0)
    res["step_eager_us"] = round(_elapsed_ms(step, reps=200) * 1e3, 2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(0)
    res["step_graph_replay_us"] = round(_elapsed_ms(lambda r: g.replay(), reps=200) * 1e3, 2)
    return {"metric": "launch latency, one 256x256 fp32 weight", "unit": "us", "results": res}


def workload_monitor(args):
    """Forward of one LLaMA-7B-shaped layer (2:4, kappa 100, tau 4, prior logits) with the fused
    convergence monitors, next to the plain forward: per call the one monitored kernel (its
    matrix-wide sums taken inside the launch); algorithmic bytes add the sample written and the previous sample read
    (1 byte per group each)."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    mats = make_layer(dev)
    for mt in mats:
        g = (mt["rows"], mt["cols"] // M)
        mt["prev"] = torch.zeros(g, dtype=torch.uint8, device=dev)
        mt["sample"] = torch.empty(g, dtype=torch.uint8, device=dev)
        mt["stats"] = torch.zeros(2, dtype=torch.float64, device=dev)
        mt["ws"] = torch.zeros(S.monitor_workspace_bytes(mt["rows"], mt["cols"], N, M), dtype=torch.uint8,
                               device=dev)
    weights = nm_synth.layer_weights(nm_synth.LLAMA2_7B_LAYER)

    def plain(r):
        for mt in mats:
            run_pass(S, mt, "fwd", r)

    def monitored(r):
        for mt in mats:
            S.nm_mask_forward_monitor(mt["w"], mt["L"], N, M, KAPPA, TAU, mt["seed"], r, prev_sample=mt["prev"],
                                      out=(mt["out"], mt["sample"], mt["stats"]), workspace=mt["ws"])
            mt["prev"], mt["sample"] = mt["sample"], mt["prev"]   # this step's sample is the next one's prev

    plain(0)
    monitored(0)
    res = {}
    for label, fn, bpw in (("fwd", plain, bytes_per_weight()["fwd"]),
                           ("fwd+monitors", monitored, bytes_per_weight()["fwd"] + 2 / M)):
        t = _elapsed_ms(fn, reps=args.kernel_reps)
        gbps = bpw * weights / (t * 1e-3) / 1e9
        res[label] = {"ms_per_pass": round(t, 4), "avg_call_us": round(t * 1e3 / len(mats), 2),
                      "bytes_per_weight": bpw, "GBps": round(gbps, 1),
                      "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
    res["overhead_pct"] = round(100 * (res["fwd+monitors"]["ms_per_pass"] / res["fwd"]["ms_per_pass"] - 1), 1)
    means = [(mt["stats"][0].item() / (mt["rows"] * mt["cols"] / M),
              mt["stats"][1].item() / (mt["rows"] * mt["cols"] / M)) for mt in mats]
    return {"metric": "forward with fused Fig. 5 monitors vs plain forward", "unit": "GB/s",
            "config": {"workload": "LLaMA-2-7B-shaped decoder layer, 7 matrices, 202,375,168 bf16 weights, "
                                   "2:4, kappa=100, tau=4, prior logits"},
            "results": res, "monitor_means_last_call": [[round(a, 6), round(b, 6)] for a, b in means]}


WREG_LAMBDA = -0.05


def workload_wreg(args):
    """Backward of one LLaMA-7B-shaped layer (2:4, kappa 100, tau 4, prior logits) with the fused
    weight regulariser lambda*sum(w_masked^2), next to the plain backward and to the unfused way
    of getting the same gradient (a torch pass forming G + 2*lambda*w_masked from the forward's
    output, then the plain backward).  Algorithmic bytes: the fused pass moves what the plain
    backward moves (16 B per weight; 14 without a task gradient, which is then not read)."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    mats = make_layer(dev)
    for mt in mats:
        run_pass(S, mt, "fwd", 0)
        mt["G2"] = torch.empty_like(mt["G"])
    weights = nm_synth.layer_weights(nm_synth.LLAMA2_7B_LAYER)

    def plain(r):
        for mt in mats:
            run_pass(S, mt, "bwd", 0)

    def fused(r):
        for mt in mats:
            S.nm_mask_backward_wreg(mt["w"], mt["L"], mt["G"], N, M, KAPPA, TAU, mt["seed"], 0, WREG_LAMBDA,
                                    out=mt["dl"])

    def alone(r):
        for mt in mats:
            S.nm_mask_backward_wreg(mt["w"], mt["L"], None, N, M, KAPPA, TAU, mt["seed"], 0, WREG_LAMBDA,
                                    out=mt["dl"])

    def unfused(r):
        for mt in mats:
            torch.add(mt["G"], mt["out"], alpha=2 * WREG_LAMBDA, out=mt["G2"])
            S.nm_mask_backward(mt["w"], mt["L"], mt["G2"], N, M, KAPPA, TAU, mt["seed"], 0, out=mt["dl"])

    bpw = bytes_per_weight()["bwd"]
    res = {}
    for label, fn, b in (("bwd", plain, bpw), ("bwd+wreg fused", fused, bpw),
                         ("wreg alone", alone, bpw - WB), ("bwd+wreg unfused (torch add + bwd)", unfused, bpw)):
        t = _elapsed_ms(fn, reps=args.kernel_reps)
        gbps = b * weights / (t * 1e-3) / 1e9
        res[label] = {"ms_per_pass": round(t, 4), "avg_call_us": round(t * 1e3 / len(mats), 2),
                      "bytes_per_weight": b, "GBps": round(gbps, 1),
                      "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
    res["fused_speedup_over_unfused"] = round(res["bwd+wreg unfused (torch add + bwd)"]["ms_per_pass"]
                                              / res["bwd+wreg fused"]["ms_per_pass"], 3)
    return {"metric": "backward with the fused weight regulariser vs plain and unfused", "unit": "GB/s",
            "config": {"workload": "LLaMA-2-7B-shaped decoder layer, 7 matrices, 202,375,168 bf16 weights, "
                                   f"2:4, kappa=100, tau=4, prior logits, lambda={WREG_LAMBDA}"},
            "results": res}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (no sparsity factor)


def workload_spmm(args):
    """Product of bf16 activations (4096 tokens) with each 2:4-packed matrix of one
    LLaMA-7B-shaped layer on the sparse matrix cores, next to torch's dense bf16 product with the
    unpacked weights (the library GEMM) for context.  Useful flops are the kept products:
    2 * tokens * out * in / 2; the dense-equivalent rate counts 2 * tokens * out * in."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    tokens = 4096
    mats = []
    for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
        seed = nm_synth.input_seed(2, 0, i)
        w, L, _ = nm_synth.matrix_inputs(rows, cols, N, M, torch.bfloat16, 0.02, seed, logits="prior", device=dev,
                                         prior=kernel_prior)
        values, indices = S.nm_mask_harden_pack(w, L, N, M)
        dense_t = S.nm_unpack(values, indices, cols, N, M).t().contiguous()  # [in, out], contiguous
        x = nm_synth.normal((tokens, cols), 1.0, seed + 7, torch.bfloat16, device=dev)
        y = torch.empty((tokens, rows), dtype=torch.bfloat16, device=dev)
        mats.append(dict(name=name, rows=rows, cols=cols, values=values, indices=indices, dense_t=dense_t, x=x, y=y))
        del w, L
    useful = sum(2.0 * tokens * mt["rows"] * mt["cols"] / 2 for mt in mats)
    # Consecutive calls take the layer's weights from three copies in turn (681 MB packed, 1.2 GB
    # dense), so every call reads its weights from HBM, as the layers of a model do, rather than
    # from the 256 MB last-level cache.
    layers = [mats] + [[dict(mt, values=mt["values"].clone(), indices=mt["indices"].clone(),
                             dense_t=mt["dense_t"].clone()) for mt in mats] for _ in range(2)]

    def sparse(r):
        for mt in layers[r % 3]:
            S.nm_sparse_matmul(mt["values"], mt["indices"], mt["x"], out=mt["y"])

    def dense(r):
        for mt in layers[r % 3]:
            torch.mm(mt["x"], mt["dense_t"], out=mt["y"])

    res = {}
    for label, fn in (("sparse_smfmac", sparse), ("dense_torch", dense)):
        t = _elapsed_ms(fn, reps=args.kernel_reps)
        res[label] = {"ms_per_layer": round(t, 4), "avg_call_us": round(t * 1e3 / len(mats), 2),
                      "useful_TFLOPs": round(useful / (t * 1e-3) / 1e12, 1),
                      "dense_equivalent_TFLOPs": round(2 * useful / (t * 1e-3) / 1e12, 1),
                      "pct_dense_bf16_peak_useful": round(100 * useful / (t * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1)}
    res["speedup_vs_dense"] = round(res["dense_torch"]["ms_per_layer"] / res["sparse_smfmac"]["ms_per_layer"], 3)

    # smaller batches, from decode (bound by reading the weights once: packed 1.125 B per
    # weight, dense bf16 2 B) through prefill sizes; HIP-event times per call include the host's
    # launch cost, which is of the order of the kernels at the smallest sizes (the rocprofv3
    # trace gives the kernels alone)
    weights = sum(mt["rows"] * mt["cols"] for mt in mats)
    batches = {}
    for tk in (1, 2, 4, 16, 64, 128, 256, 512, 1024, 2048):
        xd = [nm_synth.normal((tk, mt["cols"]), 1.0, 11 + tk, torch.bfloat16, device=dev) for mt in mats]
        yd = [torch.empty((tk, mt["rows"]), dtype=torch.bfloat16, device=dev) for mt in mats]
        # one workspace for the split k ranges of mid-size batches, allocated outside the timing
        need = max(S.sparse_matmul_workspace_bytes(mt["rows"], mt["cols"], tk) for mt in mats)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def sparse_d(r, split=True):
            for i, mt in enumerate(layers[r % 3]):
                S.nm_sparse_matmul(mt["values"], mt["indices"], xd[i], out=yd[i], workspace=ws, split=split)

        def dense_d(r):
            for i, mt in enumerate(layers[r % 3]):
                torch.mm(xd[i], mt["dense_t"], out=yd[i])

        reps = 10 * args.kernel_reps if tk <= 128 else 2 * args.kernel_reps
        ts, td = _elapsed_ms(sparse_d, reps=reps), _elapsed_ms(dense_d, reps=reps)
        u = weights * tk  # useful flops: 2 * tokens * (kept weights = weights / 2)
        batches[f"{tk}_tokens"] = {"sparse_ms_per_layer": round(ts, 4), "dense_ms_per_layer": round(td, 4),
                                   "sparse_useful_TFLOPs": round(u / (ts * 1e-3) / 1e12, 1),
                                   "sparse_weight_GBps": round(1.125 * weights / (ts * 1e-3) / 1e9, 1),
                                   "speedup_vs_dense": round(td / ts, 3)}
        if need > 0:  # the same batch on the tiles alone (nm_sparse_matmul, no k split)
            tn = _elapsed_ms(lambda r: sparse_d(r, split=False), reps=reps)
            batches[f"{tk}_tokens"]["sparse_no_split_ms_per_layer"] = round(tn, 4)
            batches[f"{tk}_tokens"]["split_speedup"] = round(tn / ts, 3)
    res["batches"] = batches
    return {"metric": "2:4 sparse x dense product on the packed weights vs dense bf16 GEMM", "unit": "TFLOP/s",
            "config": {"workload": "LLaMA-2-7B-shaped layer (7 matrices) packed 2:4, three copies of its "
                                   "weights cycled, X 4096 tokens bf16, Y bf16, fp32 accumulation"},
            "roofline": {"bound": "mfma", "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "achieved": res["sparse_smfmac"]["useful_TFLOPs"],
                         "frac": round(res["sparse_smfmac"]["useful_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4)},
            "results": res}


def workload_prior_init(args):
    """Magnitude-prior logit initialisation of every matrix of one LLaMA-7B-shaped layer (2:4,
    alpha 3) and of a 4096x11008 matrix for 2:8 and 4:8: read w, write the K logits of each group
    (and the one-byte prior index where noted)."""
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S
    dev = torch.device("cuda:0")
    res = {}
    cases = [("2:4 layer", 2, 4, nm_synth.LLAMA2_7B_LAYER, False),
             ("2:4 layer +idx", 2, 4, nm_synth.LLAMA2_7B_LAYER, True),
             ("2:8 4096x11008", 2, 8, [("down", 4096, 11008)], False),
             ("4:8 4096x11008", 4, 8, [("down", 4096, 11008)], False)]
    for label, n, m, shapes, with_idx in cases:
        k = S.num_candidates(n, m)
        mats = []
        for i, (name, rows, cols) in enumerate(shapes):
            w = nm_synth.normal((rows, cols), 0.02, 3 * nm_synth.input_seed(2, 0, i), torch.bfloat16, device=dev)
            mats.append((w, torch.empty((rows, cols // m, k), device=dev),
                         torch.empty((rows, cols // m), dtype=torch.uint8, device=dev) if with_idx else None))
        weights = sum(w.numel() for w, _, _ in mats)

        def run(r):
            for w, L, ix in mats:
                S.nm_prior_init(w, n, m, 3.0, out=(L, ix))

        run(0)
        t = _elapsed_ms(run, reps=args.kernel_reps)
        bpw = WB + 4 * k / m + (1 / m if with_idx else 0)
        gbps = bpw * weights / (t * 1e-3) / 1e9
        res[label] = {"ms_per_pass": round(t, 4), "avg_launch_us": round(t * 1e3 / len(mats), 2),
                      "bytes_per_weight": bpw, "GBps": round(gbps, 1),
                      "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
        del mats
    return {"metric": "magnitude-prior logit initialisation", "unit": "GB/s",
            "config": {"workload": "LLaMA-2-7B-shaped layer (202,375,168 bf16 weights) at 2:4; "
                                   "4096x11008 bf16 at 2:8 and 4:8; alpha=3"}, "results": res}


def main():
    args = parse()
    if args.workload != "llama7b_layer":
        import torch
        torch.cuda.set_device(0)
        fn = {"sweep32": workload_sweep32, "general_nm": workload_general_nm,
              "nemotron_pack": workload_nemotron_pack, "single256": workload_single256,
              "prior_init": workload_prior_init, "monitor": workload_monitor,
              "spmm": workload_spmm, "wreg": workload_wreg}[args.workload]
        out = fn(args)
        out.update({"n_gpus": 1, "data": "synthetic, seeded, generated on the GPU", "dtype": "f32"})
        print(json.dumps(out), flush=True)
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return
    if args.summarize_pmc:
        print(json.dumps(write_traffic(*args.summarize_pmc, os.path.join(ROOT, "profiles", "traffic.json")),
                         indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the layer is independent "
              "per group and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch

    import nm_synth
    import semi_structured_sparsity_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy_gbps = copy_ceiling(dev)
    mats = make_layer(dev)
    torch.cuda.synchronize()
    weights = nm_synth.layer_weights(nm_synth.LLAMA2_7B_LAYER)
    bpw = bytes_per_weight()

    for s in range(args.warmup):
        step_all(S, mats, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(PASSES) + 1)] for _ in range(args.steps)]
    e0.record()
    for s in range(args.steps):
        step_all(S, mats, args.warmup + s, marks[s])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    step_ms_wall = wall * 1e3 / args.steps
    ms_per_step = max(step_ms, step_ms_wall)
    # the metric: forward + backward of every matrix, timed inside each of the K whole-path steps
    fb_ms_per_step = sum(m[0].elapsed_time(m[PASSES.index("bwd") + 1]) for m in marks) / args.steps
    # each pass inside the timed steps, per launch (the passes below time each pass on its own,
    # one kernel launched over and over)
    in_step_us = {p: round(sum(m[i].elapsed_time(m[i + 1]) for m in marks) / args.steps * 1e3 / len(mats), 2)
                  for i, p in enumerate(PASSES)}

    # per-kernel timing: each pass over the seven matrices, HIP events on the launch stream
    passes = {}
    for p in PASSES:
        for mt in mats:
            run_pass(S, mt, p, 0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(args.kernel_reps):
            for mt in mats:
                run_pass(S, mt, p, r)
        b.record()
        torch.cuda.synchronize()
        launches = args.kernel_reps * len(mats)
        avg_us = a.elapsed_time(b) * 1e3 / launches
        alg_bytes = bpw[p] * weights / len(mats)  # per launch, averaged over the matrices
        passes[p] = {"avg_launch_us": round(avg_us, 2), "launches_per_step": len(mats),
                     "bytes_per_weight": bpw[p],
                     "GBps": round(alg_bytes / (avg_us * 1e-6) / 1e9, 1),
                     "pct_hbm_peak": round(100 * alg_bytes / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
                     "pct_of_copy": round(100 * alg_bytes / (avg_us * 1e-6) / 1e9 / copy_gbps, 1)}
    fb_us = (passes["fwd"]["avg_launch_us"] + passes["bwd"]["avg_launch_us"]) * len(mats)
    fwd_bwd = {"weights_per_s": weights / (fb_us * 1e-6),
               "GBps": round((bpw["fwd"] + bpw["bwd"]) * weights / (fb_us * 1e-6) / 1e9, 1)}
    fwd_bwd["pct_hbm_peak"] = round(100 * fwd_bwd["GBps"] / HBM_PEAK_GBPS, 1)
    # the target's pass set: forward + backward + harden/pack
    fbp_us = fb_us + passes["harden_pack"]["avg_launch_us"] * len(mats)
    fwd_bwd_pack = {"weights_per_s": weights / (fbp_us * 1e-6),
                    "GBps": round((bpw["fwd"] + bpw["bwd"] + bpw["harden_pack"]) * weights / (fbp_us * 1e-6) / 1e9, 1)}
    fwd_bwd_pack["pct_hbm_peak"] = round(100 * fwd_bwd_pack["GBps"] / HBM_PEAK_GBPS, 1)
    dom = max(PASSES, key=lambda p: passes[p]["avg_launch_us"])
    dom_bytes = bpw[dom] * weights / len(mats)
    achieved = dom_bytes / (passes[dom]["avg_launch_us"] * 1e-6) / 1e9
    traffic = stored_traffic(dom)
    step_bytes = sum(bpw.values()) * weights
    result = {
        "metric": METRIC,
        "value": weights / (fb_ms_per_step * 1e-3),
        "value_is": "forward + backward weights per second: HIP events on the launch stream around the "
                    "forward and backward passes of the seven matrices inside each of the K timed steps",
        "unit": "weights/s",
        "fwd_bwd_ms_per_step": round(fb_ms_per_step, 4),
        "fwd_bwd_GBps": round((bpw["fwd"] + bpw["bwd"]) * weights / (fb_ms_per_step * 1e-3) / 1e9, 1),
        "fwd_bwd_pct_hbm_peak": round(100 * (bpw["fwd"] + bpw["bwd"]) * weights / (fb_ms_per_step * 1e-3) / 1e9
                                      / HBM_PEAK_GBPS, 1),
        "step_weights_per_s": weights / (ms_per_step * 1e-3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_events": round(step_ms, 4),
        "step_ms_wall": round(step_ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded Gaussian bf16 weights N(0,0.02) and grads N(0,1); fp32 logits "
                "3*onehot(magnitude prior, from nm_prior_init) + N(0,0.1); generated on the GPU",
        "config": {"workload": "LLaMA-2-7B-shaped decoder layer, 7 matrices, 202,375,168 weights, "
                               "2:4, bf16 weights, fp32 logits, kappa=100, tau=4",
                   "passes_per_step": "fwd+bwd+harden_pack+unpack (value: fwd+bwd)",
                   "global_batch": 1, "parallelism": "single GPU"},
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_pct_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
        "copy_ceiling": {"GBps": round(copy_gbps, 1), "kernel": "k_debug_copy",
                         "what": "flat 16-byte-per-thread copy of 1 GiB, read + write bytes"},
        "fwd_bwd": fwd_bwd,
        "fwd_bwd_pack": fwd_bwd_pack,
        "passes": passes,
        "passes_in_step_avg_launch_us": in_step_us,
        "roofline": {"bound": "hbm", "kernel": KERNELS[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(dom_bytes, 0),
                     "avg_launch_us": passes[dom]["avg_launch_us"]},
    }
    if not args.no_sweep:
        # the target's workload: 32 layers x 10 annealed steps of fwd + bwd + harden_pack
        del mats
        torch.cuda.empty_cache()
        sw = workload_sweep32(args)
        result["sweep32"] = {k: sw[k] for k in ("metric", "value", "unit", "ms_per_step", "GBps", "pct_hbm_peak",
                                                 "forward_pack_in_one_call", "config")}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
