"""Throughput of the N:M mask layer on one MI355X.

One step = the whole hot path over one LLaMA-2-7B-shaped decoder layer (q, k, v, o 4096x4096;
gate, up 11008x4096; down 4096x11008; 202,375,168 bf16 weights, fp32 logits, 2:4, kappa = 100,
tau = 4, logits from the magnitude prior): forward (soft mask times frozen weights), backward to
the logits, hard-mask extraction with compressed pack, and unpack, for all seven matrices.
Inputs are synthetic, seeded, generated on the GPU and resident in HBM before timing starts.

Prints one JSON line.  `value` is masked weights per second of whole steps; the per-pass
breakdown, the roofline of the dominant kernel (HIP-event timing, algorithmic bytes) and the
oracle's CPU baseline on a bounded sample are added alongside.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--kernel-reps", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="least CPU time of the baseline")
    p.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                   help="print the path kernels' average durations from rocprofv3 --stats output")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run 4 plain 1 GiB device copies (counter calibration under a profiler)")
    return p.parse_args()


def make_layer(dev):
    import torch

    import nm_synth
    mats = []
    for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
        seed = nm_synth.input_seed(2, 0, i)
        w, L, G = nm_synth.matrix_inputs(rows, cols, N, M, torch.bfloat16, 0.02, seed,
                                         logits="prior", device=dev)
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


def step_all(S, mats, step):
    # pass-major, as in a training step (all forwards, then all backwards, ...): each pass moves
    # >= 2 GB across the seven matrices, so no pass finds a matrix's data left in the 256 MB
    # last-level cache by the previous pass over the same matrix
    for p in PASSES:
        for mt in mats:
            run_pass(S, mt, p, step)


def cpu_baseline(min_seconds=10.0, max_passes=8):
    """The oracle over the same layer (same shapes, generators and parameters, CPU copies):
    forward, backward, pack and unpack of all seven matrices, repeated over successive steps
    until at least `min_seconds` of CPU time has been spent.  Returns weights/s of whole steps."""
    import torch

    import nm_synth
    import oracle
    threads = min(16, os.cpu_count() or 1)
    mats = []
    for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
        seed = nm_synth.input_seed(2, 0, i)
        w = nm_synth.normal((rows, cols), 0.02, 3 * seed, torch.bfloat16)
        mats.append((seed, cols, w, nm_synth.prior_logits(w, N, M, 3 * seed + 1),
                     nm_synth.normal((rows, cols), 1.0, 3 * seed + 2, torch.bfloat16)))
    total_w, elapsed, passes = 0, 0.0, 0
    while passes < max_passes and (passes == 0 or elapsed < min_seconds):
        for seed, cols, w, L, G in mats:
            t0 = time.perf_counter()
            oracle.forward(w, L, N, M, KAPPA, TAU, seed, passes, nthreads=threads)
            oracle.backward(w, L, G, N, M, KAPPA, TAU, seed, passes, nthreads=threads)
            v, idx, _ = oracle.pack(w, L, N, M, nthreads=threads)
            oracle.unpack(v, idx, cols, N, M, nthreads=threads)
            elapsed += time.perf_counter() - t0
            total_w += w.numel()
        passes += 1
    return {"value": total_w / elapsed, "unit": "weights/s", "cores": oracle.threads_used(threads),
            "kind": "oracle",
            "sample": f"{passes} step(s) of the whole layer ({total_w} weight-passes): "
                      f"fwd+bwd+harden_pack+unpack in binary64 on {threads} threads, {elapsed:.1f} s"}


# ---------------------------------------------------------------------------------------------
# rocprofv3 summaries (run on the CSV output of the commands printed in profiles/)

KERNELS = {"fwd": "k_forward<2, 4, nm::BF16, 0>", "bwd": "k_backward<2, 4, nm::BF16>",
           "harden_pack": "k_pack_bytes<2, nm::BF16>", "unpack": "k_unpack_bytes<2, nm::BF16>"}
COPY_BYTES = 1 << 30  # the --copy-calibration copies


def kernel_source_hash():
    """Hash of the HIP sources, so stored counter readings can be matched to the kernels."""
    import hashlib
    import semi_structured_sparsity_amd.build as b
    h = hashlib.sha256()
    for path in sorted(b.SOURCES + b.HEADERS):
        h.update(open(path, "rb").read())
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


def main():
    args = parse()
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
    mats = make_layer(dev)
    torch.cuda.synchronize()
    weights = nm_synth.layer_weights(nm_synth.LLAMA2_7B_LAYER)
    bpw = bytes_per_weight()

    for s in range(args.warmup):
        step_all(S, mats, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(args.steps):
        step_all(S, mats, args.warmup + s)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    step_ms_wall = wall * 1e3 / args.steps
    ms_per_step = max(step_ms, step_ms_wall)

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
                     "pct_hbm_peak": round(100 * alg_bytes / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)}
    fb_us = (passes["fwd"]["avg_launch_us"] + passes["bwd"]["avg_launch_us"]) * len(mats)
    fwd_bwd = {"weights_per_s": weights / (fb_us * 1e-6),
               "GBps": round((bpw["fwd"] + bpw["bwd"]) * weights / (fb_us * 1e-6) / 1e9, 1)}
    fwd_bwd["pct_hbm_peak"] = round(100 * fwd_bwd["GBps"] / HBM_PEAK_GBPS, 1)
    dom = max(PASSES, key=lambda p: passes[p]["avg_launch_us"])
    dom_bytes = bpw[dom] * weights / len(mats)
    achieved = dom_bytes / (passes[dom]["avg_launch_us"] * 1e-6) / 1e9
    traffic = stored_traffic(dom)
    step_bytes = sum(bpw.values()) * weights
    result = {
        "metric": METRIC,
        "value": weights / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded Gaussian bf16 weights N(0,0.02) and grads N(0,1); fp32 logits "
                "3*onehot(magnitude prior) + N(0,0.1); generated on the GPU",
        "config": {"workload": "LLaMA-2-7B-shaped decoder layer, 7 matrices, 202,375,168 weights, "
                               "2:4, bf16 weights, fp32 logits, kappa=100, tau=4",
                   "passes_per_step": "fwd+bwd+harden_pack+unpack",
                   "global_batch": 1, "parallelism": "single GPU"},
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_pct_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
        "fwd_bwd": fwd_bwd,
        "passes": passes,
        "roofline": {"bound": "hbm", "kernel": KERNELS[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(dom_bytes, 0),
                     "avg_launch_us": passes[dom]["avg_launch_us"]},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
