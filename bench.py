#!/usr/bin/env python3
"""Benchmark of the gradient-aggregation hot path on one MI355X.

Default workload: AlexNet-shaped, W=128 workers x P=60,965,224 parameters,
binary16 gradients, coarse-grained sparse communication with 32768-element
chunks keeping 10% of them per worker (k=187 of 1861), the residual carried in
deferred form (written every depth+1 steps and re-formed in between from the
previous `depth` gradient batches and selection masks, which are kept), and
momentum SGD on binary32 master weights.

One step = lazy-allreduce fusion of the W*16 per-layer gradient tensors read
with zero copy through the layer table, together with the chunk norms and the
residual (k_norm_hist), top-k chunk selection (k_topk), and the gather-reduce
of the selected chunks fused with the mean and the SGD update (k_gather_hist,
or k_gather_wave with --residual lazy), over one batch of gradients already
resident in HBM (six gradient batches are cycled so that consecutive steps
see fresh inputs).

Prints one JSON line:
  value            algorithmic GB/s of the whole step, B_alg / step time, where
                   B_alg = W*P*(2 + 4 + 4) + 16*P bytes (binary16 gradient read,
                   residual read and write, w and v read and write)
  roofline         the dominant kernel (k_chunk_norm): 10*W*P bytes per launch
                   over its mean launch time from HIP events on its stream,
                   against the 8 TB/s HBM peak
  cpu_baseline     the oracle timed on the host cores over whole steps
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
import types

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "aggregated gradient GB/s and % of HBM peak, W workers × P params"


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 24 for the sparse workload, a whole number of store periods "
                         "at depth 0-3; 200 for a dense one)")
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--workload", default="alexnet128_sparse")
    ap.add_argument("--batches", type=int, default=6, help="distinct gradient batches cycled over steps")
    ap.add_argument("--source", choices=["layers", "bucket"], default="layers",
                    help="gradients as per-layer tensors fused with zero copy (default) or a packed bucket")
    ap.add_argument("--residual", choices=["deferred", "lazy"], default="deferred",
                    help="sparse workload: the deferred residual (written every depth+1 steps, re-formed from the "
                         "held gradients in between) or the lazy-zero sequence of the boundary's calls")
    ap.add_argument("--depth", type=int, default=2,
                    help="deferred residual: earlier gradient batches held (the residual is stored every depth+1 "
                         "steps)")
    ap.add_argument("--order", choices=["tree", "server", "ring"], default="tree",
                    help="dense workloads: summation order (parameter server, ring) for comparison")
    ap.add_argument("--wire", choices=["f32", "f16"], default="f32",
                    help="dense workloads: binary16 wire (every value sent between workers rounded)")
    ap.add_argument("--no-extras", dest="extras", action="store_false", default=True,
                    help="skip the extra measurements of the default run (the step protocol and the lazy-zero "
                         "sequence of the sparse workload, and the dense workloads)")
    ap.add_argument("--cpu-baseline", dest="cpu_baseline", action="store_true", default=True)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy (one-layer pack) of known size, for counter calibration")
    ap.add_argument("--overlap", action="store_true",
                    help="dense workloads: time a stand-in backward pass (one weight-gradient GEMM per layer, "
                         "last layer first) with the multi-bucket reduction overlapped on a second stream")
    ap.add_argument("--bucket-mb", default="1,4,16,100000",
                    help="--overlap: bucket thresholds to compare, MiB per worker")
    ap.add_argument("--reduce-workgroups", default="0,512",
                    help="--overlap: grid caps of the bucket reductions to compare (0: full grid)")
    ap.add_argument("--cu-split", default="",
                    help="--overlap: also run the overlapped schedule with the compute units partitioned: the "
                         "reductions on a stream confined to CUs 0..N-1, the producer on a stream with the others "
                         "(comma-separated multiples of 32)")
    ap.add_argument("--producer", choices=["gemm", "dense", "copy"], default="gemm",
                    help="--overlap: each layer's gradients come from its weight-gradient GEMM (gemm), from "
                         "the same flops as square 4096^3 GEMMs plus a copy of a staged gradient (dense), or "
                         "from the copy alone (copy)")
    ap.add_argument("--producer-batch", type=int, default=64,
                    help="--overlap gemm: samples per worker; a layer's weight-gradient GEMM reduces over "
                         "batch x output positions")
    ap.add_argument("--split", type=int, default=0,
                    help="time the two per-GPU kernels of the dense step split across this many GPUs (W/G "
                         "workers each): one GPU's partial tree sum and one owner's combine of G partials")
    ap.add_argument("--traffic", default=None, help="JSON file with measured HBM bytes per launch of the "
                                                    "dominant kernel (from rocprofv3 counters); default: "
                                                    "profiles/traffic_<workload>.json")
    return ap.parse_args()


def host_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def copy_calibration():
    """A plain copy of 2 GiB through the pack kernel (W=1, one layer)."""
    import torch
    import gradient_aggregation_amd as ga
    n = 1 << 30                              # binary16 elements = 2 GiB
    plan = ga.Plan(1, [n], True)
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = plan.empty_bucket()
    ptrs = torch.tensor([src.data_ptr()], dtype=torch.int64, device="cuda")
    for _ in range(5):
        plan.bucket_pack(ptrs, dst)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    plan.bucket_pack(ptrs, dst)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * plan.ld, "ms": ms,
                      "GBps": (2 * n + 2 * plan.ld) / ms / 1e6}), flush=True)


def load_batches(wl, plan, nb, layers_src, thr, keep_host_first):
    """nb gradient batches generated on the host and made resident in HBM:
    per-layer tensors (a layer table per batch) or packed [W][ld] buckets.
    Returns (sources, kept layer tensors, first batch on the host or None)."""
    import torch
    import workloads
    P, ld, W = wl.P, plan.ld, wl.W
    seg = workloads.segments(wl)
    gdt = torch.float16 if wl.fp16 else torch.float32
    offs = np.cumsum([0] + wl.numels)
    sources, keep = [], []
    row = np.empty(P, np.uint16 if wl.fp16 else np.float32)
    pinned = torch.empty(P, dtype=gdt).pin_memory()
    host_first = np.zeros((W, ld), row.dtype) if keep_host_first else None
    t0 = time.time()
    for bi in range(nb):
        if layers_src:
            tensors = [[torch.empty(n, dtype=gdt, device="cuda") for n in wl.numels] for _ in range(W)]
        else:
            bucket = torch.zeros((W, ld), dtype=gdt, device="cuda")
        for w in range(W):
            workloads.grad_row(wl, bi + 1, w, seg, out=row, threads=thr)
            pinned.numpy().view(row.dtype)[:] = row
            if layers_src:
                for l in range(len(wl.numels)):
                    tensors[w][l].copy_(pinned[offs[l]:offs[l + 1]], non_blocking=False)
            else:
                bucket[w, :P].copy_(pinned, non_blocking=False)
            if bi == 0 and host_first is not None:
                host_first[w, :P] = row
        if layers_src:
            keep.append(tensors)
            sources.append(torch.tensor([t.data_ptr() for tw in tensors for t in tw], dtype=torch.int64,
                                        device="cuda"))
        else:
            sources.append(bucket)
        log("%s: gradient batch %d resident (%.1fs)" % (wl.name, bi + 1, time.time() - t0))
    return sources, keep, host_first


def time_steps(step, n_warm, n_timed, n_kernels):
    """Run n_warm + n_timed steps (step(t, events) records one event after each
    of its n_kernels launches).  Returns (host ms per timed step, GPU-event ms
    per timed step, [per timed step: [ms of each kernel]], [per timed step:
    what step() returned])."""
    import torch
    stream = torch.cuda.current_stream()
    n = n_warm + n_timed
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_kernels + 1)] for _ in range(n)]
    ret = [None] * n

    def one(t):
        ev[t][0].record(stream)
        ret[t] = step(t, ev[t][1:])

    for t in range(n_warm):
        one(t)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for t in range(n_warm, n):
        one(t)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [[ev[t][j].elapsed_time(ev[t][j + 1]) for j in range(n_kernels)] for t in range(n)]
    return wall * 1e3 / n_timed, t_start.elapsed_time(t_end) / n_timed, per, ret


def sparse_stepper(plan, wl, sources, state, mode, depth, layers_src):
    """A step function for time_steps over the sparse workload, and the object
    holding its residual.  mode "deferred": the history form at `depth`;
    "lazy": the lazy-zero sequence of the boundary's calls."""
    import torch
    import gradient_aggregation_amd as ga
    nb = len(sources)
    wd, vd = state
    if mode == "deferred":
        dr = ga.DeferredResidual(plan, depth)

        def step(t, ev):
            return dr.step(sources[t % nb], None, wd, vd, wl.lr, wl.mu, events=ev)
        return step, dr
    W = plan.W
    holder = types.SimpleNamespace(
        resid=plan.empty_residual(), keys=plan.empty_keys(),
        idx=torch.empty((W, max(plan.k, 1)), dtype=torch.int32, device="cuda"),
        mask=torch.zeros((W, plan.mask_words), dtype=torch.int32, device="cuda"), t0=None)

    def step(t, ev):
        b = sources[t % nb]
        first = holder.t0 is None
        if first:
            holder.t0 = t
        prev = None if first else holder.mask
        if layers_src:
            plan.chunk_norm_layers(b, holder.resid, holder.keys, prev)
        else:
            plan.chunk_norm(b, holder.resid, holder.keys, prev)
        ev[0].record()
        plan.chunk_topk(holder.keys, holder.idx, holder.mask)
        ev[1].record()
        plan.sparse_gather_reduce(holder.resid, holder.mask, False, None, wd, vd, wl.lr, wl.mu)
        ev[2].record()
        return True
    return step, holder


def kernel_stats(per, timed, names, stored=None):
    out = {}
    for j, nm in enumerate(names):
        d = [per[t][j] for t in timed]
        out[nm] = {"mean_ms": float(np.mean(d)), "min_ms": float(np.min(d)), "max_ms": float(np.max(d))}
        if stored is not None and not all(stored[t] for t in timed):
            for kind, want in (("storing", True), ("other", False)):
                dk = [per[t][j] for t in timed if bool(stored[t]) == want]
                if dk:
                    out[nm]["mean_ms_%s_steps" % kind] = round(float(np.mean(dk)), 4)
    return out


def sparse_protocol(plan, wl, sources, w_init, mode, depth, layers_src, reps=5, steps=3):
    """The step timing of the sparse workload's own protocol: `steps` steps from
    a zero residual and fresh state, repeated `reps` times with the state reset
    outside the timed region; per step, the median over the repetitions of the
    whole step and of its two halves (norms + top-k | gather + SGD)."""
    import torch
    P, W = wl.P, wl.W
    b_alg = W * P * ((2 if wl.fp16 else 4) + 8) + 16 * P
    times = [[] for _ in range(steps)]
    halves = [[] for _ in range(steps)]
    for rep in range(reps):
        wd = torch.from_numpy(w_init).cuda()
        vd = torch.zeros(P, dtype=torch.float32, device="cuda")
        step, holder = sparse_stepper(plan, wl, sources, (wd, vd), mode, depth, layers_src)
        holder.resid.zero_()
        torch.cuda.synchronize()
        _, _, per, _ = time_steps(step, 0, steps, 3)
        for t in range(steps):
            times[t].append(sum(per[t]))
            halves[t].append((per[t][0] + per[t][1], per[t][2]))
        del step, holder, wd, vd
        torch.cuda.empty_cache()
    med = [float(np.median(x)) for x in times]
    return {
        "steps": steps, "repetitions": reps, "reset": "zero residual, fresh w and v, outside the timed region",
        "step_ms_median": [round(x, 4) for x in med],
        "norm_topk_ms_median": [round(float(np.median([h[0] for h in halves[t]])), 4) for t in range(steps)],
        "gather_sgd_ms_median": [round(float(np.median([h[1] for h in halves[t]])), 4) for t in range(steps)],
        "median_step_ms": round(float(np.median(med)), 4),
        "alg_GBps_at_median_step": round(b_alg / (float(np.median(med)) * 1e-3) / 1e9, 1),
        "pct_hbm_peak_alg_at_median_step": round(100.0 * b_alg / (float(np.median(med)) * 1e-3) / 1e9 /
                                                 HBM_PEAK_GBPS, 2),
        "mean_of_steps_ms": round(float(np.mean(med)), 4),
        "note": "step 1 reads only the gradient (the residual is zero: described by an all-ones mask in the "
                "deferred form, read from the zeroed buffer in the lazy form)",
    }


def dense_summary(thr, steps=200):
    """The dense workloads (NiN W=32 binary32, GoogLeNet W=128 and AlexNet W=16
    binary16), each from per-layer tensors read with zero copy: ms per step of
    the fused tree + mean + SGD, algorithmic GB/s and % of peak, the fusion
    copy (ga_bucket_pack) rate and the end-to-end time with that copy."""
    import torch
    import gradient_aggregation_amd as ga
    import workloads
    out = {}
    for name in ("nin", "googlenet", "alexnet16"):
        wl = workloads.WORKLOADS[name]
        plan = ga.Plan(wl.W, wl.numels, wl.fp16)
        sources, keep, _ = load_batches(wl, plan, 2, True, thr, False)
        w_init = workloads.weights(wl, threads=thr)
        states = [(torch.from_numpy(w_init).cuda(), torch.zeros(wl.P, dtype=torch.float32, device="cuda"))
                  for _ in range(2)]

        def step(t, ev):
            wd, vd = states[t % 2]
            plan.tree_reduce_layers(sources[t % 2], None, wd, vd, wl.lr, wl.mu)
            ev[0].record()

        ms, gms, per, _ = time_steps(step, 20, steps, 1)
        b_in = 2 if wl.fp16 else 4
        b_alg = wl.W * wl.P * b_in + 16 * wl.P
        pack = time_pack(plan, wl, sources[-1], keep[-1], torch.cuda.current_stream())
        kms = float(np.mean([per[t][0] for t in range(20, 20 + steps)]))
        out[name] = {"W": wl.W, "P": wl.P, "grad_dtype": "f16" if wl.fp16 else "f32", "steps": steps,
                     "ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                     "alg_GBps": round(b_alg / (ms * 1e-3) / 1e9, 1),
                     "pct_hbm_peak_alg": round(100.0 * b_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                     "bytes_alg_per_step": b_alg, "pack_GBps": pack["GBps"], "pack_ms": pack["mean_ms"],
                     "end_to_end_ms_with_pack": round(ms + pack["mean_ms"], 4)}
        log("dense %s: %.4f ms/step (%.1f%% of peak)" % (name, ms, out[name]["pct_hbm_peak_alg"]))
        del sources, keep, states
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the W workers are simulated as W buffers in one GPU's HBM, "
              "so --gpus %d is not supported (use --gpus 1)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import gradient_aggregation_amd as ga
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.overlap:
        run_overlap(args)
        return
    if args.split:
        run_split(args)
        return

    wl = workloads.WORKLOADS[args.workload]
    sparse = wl.mode == "sparse"
    if args.steps is None:
        args.steps = 24 if sparse else 200
    variant = args.order != "tree" or args.wire != "f32"
    if variant:
        if sparse:
            print("--order/--wire apply to the dense workloads", file=sys.stderr)
            sys.exit(2)
        args.source = "bucket"      # the comparison schemes read a packed bucket
    plan = ga.Plan(wl.W, wl.numels, wl.fp16, chunk=wl.chunk, keep_ratio=wl.rho)
    P, ld, W = wl.P, plan.ld, wl.W
    thr = host_threads()
    log("workload %s: W=%d P=%d ld=%d fp16=%s chunk=%d k=%d n_c=%d" % (
        wl.name, W, P, ld, wl.fp16, plan.chunk, plan.k, plan.n_chunks))
    layers_src = args.source == "layers"
    nb = max(1, args.batches)
    deferred = False
    if sparse:
        deferred = args.residual == "deferred" and layers_src and plan.chunk % 256 == 0
        if args.residual == "deferred" and not deferred:
            log("the deferred form needs per-layer tensors and a chunk size that is a multiple of 256; "
                "timing the lazy-zero sequence")
        if deferred and nb < args.depth + 1:
            print("--depth %d needs at least %d gradient batches" % (args.depth, args.depth + 1), file=sys.stderr)
            sys.exit(2)

    # ---- inputs: generated on the host, made resident in HBM before timing ----
    # Default: every worker's gradient arrives as its own per-layer tensors (as
    # a backward pass leaves them) and the step fuses them with zero copy by
    # reading through the layer table.  --source bucket feeds a pre-packed
    # [W][ld] bucket instead.
    t0 = time.time()
    sources, keep, host_first = load_batches(wl, plan, nb, layers_src, thr, args.cpu_baseline)
    w_init = workloads.weights(wl, threads=thr)
    # Dense workloads: the w/v state (at most 0.5 GB) alternates between two
    # replicas, so the 256 MB Infinity Cache cannot serve a step's w and v
    # from the step before (each replica is last touched two steps earlier,
    # with a whole gradient batch streamed in between).  The sparse workload's
    # state is far larger than the cache.
    n_state = 1 if sparse else 2
    states = [(torch.from_numpy(w_init).cuda(), torch.zeros(P, dtype=torch.float32, device="cuda"))
              for _ in range(n_state)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    stream = torch.cuda.current_stream()
    if sparse:
        names = ["chunk_norm", "topk", "gather_sgd"]
        step, holder = sparse_stepper(plan, wl, sources, states[0], "deferred" if deferred else "lazy",
                                      args.depth, layers_src)
    else:
        names = ["tree_sgd"]

        def step(t, ev):
            b = sources[t % nb]
            wd, vd = states[t % n_state]
            if variant:
                plan.reduce_variant(b, args.order, args.wire == "f16", None, wd, vd, wl.lr, wl.mu)
            elif layers_src:
                plan.tree_reduce_layers(b, None, wd, vd, wl.lr, wl.mu)
            else:
                plan.tree_reduce(b, None, wd, vd, wl.lr, wl.mu)
            ev[0].record()
            return True

    ms_step, gpu_ms_step, per, stored = time_steps(step, args.warmup, args.steps, len(names))
    n_steps = args.warmup + args.steps
    timed = range(args.warmup, n_steps)
    first_step = {nm: round(per[0][j], 4) for j, nm in enumerate(names)}
    per_kernel = kernel_stats(per, timed, names, stored if sparse else None)
    log("timed %d steps: %.3f ms/step (GPU events %.3f ms/step); %s" % (
        args.steps, ms_step, gpu_ms_step,
        ", ".join("%s %.3f ms" % (k, v["mean_ms"]) for k, v in per_kernel.items())))

    b_in = 2 if wl.fp16 else 4
    sel_stats = None
    if sparse and deferred:
        sel_stats = selection_stats(plan, holder.masks[(holder.next - 2) % len(holder.masks)],
                                    holder.masks[(holder.next - 1) % len(holder.masks)], P)
    elif sparse:
        sel_stats = selection_stats(plan, None, holder.mask, P)

    pack = time_pack(plan, wl, sources[-1], keep[-1] if layers_src else None, stream)

    if sparse:
        b_alg = W * P * (b_in + 4 + 4) + 16 * P
        dom, dom_bytes = "chunk_norm", W * P * (b_in + 4 + 4)
    else:
        b_alg = W * P * b_in + 16 * P
        dom, dom_bytes = "tree_sgd", b_alg
    value = b_alg / (ms_step * 1e-3) / 1e9
    # algorithmic bytes and rate of every kernel of the step
    if sparse:
        kbytes = {"chunk_norm": W * P * (b_in + 4 + 4),
                  "topk": W * plan.n_chunks * 8,
                  "gather_sgd": W * plan.k * plan.chunk * 4 + 16 * P}
    else:
        kbytes = {"tree_sgd": b_alg}
    for nm, kb in kbytes.items():
        per_kernel[nm]["bytes_alg"] = kb
        per_kernel[nm]["GBps_alg"] = round(kb / (per_kernel[nm]["mean_ms"] * 1e-3) / 1e9, 1)
        per_kernel[nm]["frac_hbm_peak"] = round(per_kernel[nm]["GBps_alg"] / HBM_PEAK_GBPS, 4)
    dom_ms = per_kernel[dom]["mean_ms"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    if sparse:
        dom_kernel = "k_norm_hist" if (deferred or layers_src) else "k_chunk_norm"
    elif variant:
        dom_kernel = "k_variant_" + ("tree" if args.order == "tree" else "seq")
    else:
        dom_kernel = "k_tree_layers" if layers_src else "k_tree"
    traffic_key = dom_kernel if not variant else "%s_order_%s_wire_%s" % (dom_kernel, args.order, args.wire)
    step_key = None
    if sparse:
        traffic_key = "%s_%s" % (dom_kernel, ("depth%d" % args.depth) if deferred else "lazy")
        step_key = "step_%s" % (("depth%d" % args.depth) if deferred else "lazy")
    tpath = args.traffic or os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    traffic = measured_traffic(tpath, traffic_key)
    step_traffic = measured_traffic(tpath, step_key) if step_key else None
    moved = None if traffic is None else traffic["bytes_per_launch"] / (dom_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "gpu_ms_per_step": round(gpu_ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "W": W, "P": P, "grad_dtype": "f16" if wl.fp16 else "f32",
            "accumulate": "f32 fixed binary tree", "keys": "f64" if sparse else None,
            "chunk": plan.chunk or None, "keep_ratio": wl.rho if sparse else None,
            "k": plan.k if sparse else None, "n_chunks": plan.n_chunks if sparse else None,
            "residual_mode": (("deferred, depth %d (stored every %d steps)" % (args.depth, args.depth + 1))
                              if deferred else "lazy-zero") if sparse else None,
            "gradient_batches": nb,
            "fusion": "zero-copy read of %d per-layer tensors" % (W * len(wl.numels)) if layers_src
                      else "pre-packed bucket",
            "order": args.order, "wire": args.wire,
            "parallelism": "1 GPU, W workers as HBM buffers",
            "state_replicas": n_state,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "bytes_alg_per_step": b_alg,
        "grad_elements_per_s": W * P / (ms_step * 1e-3),
        "grad_input_GBps": round(W * P * b_in / (ms_step * 1e-3) / 1e9, 2),
        "kernels": per_kernel,
        "first_step_ms": first_step if sparse else None,
        "selection_last_step": sel_stats,
        "roofline": {
            "kernel": dom_kernel,
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            # the bytes the kernel moves (counters) over its time, beside the
            # algorithmic figure above
            "moved_GBps": None if moved is None else round(moved, 1),
            "moved_frac": None if moved is None else round(moved / HBM_PEAK_GBPS, 4),
            "traffic_source": None if traffic is None else traffic["summary"],
            "bytes_per_launch": dom_bytes, "mean_launch_ms": round(dom_ms, 4),
            # the same chip's plain-copy rate in this run (the fusion copy of the
            # per-layer tensors, below): the measured ceiling for mixed read/write
            "vs_plain_copy": round(achieved / pack["GBps"], 3) if pack.get("GBps") else None,
        },
        # the whole step by the counters: HBM bytes all its kernels move per
        # step (averaged over the step kinds) over the step time
        "step_moved": None if step_traffic is None else {
            "bytes_per_step": step_traffic["bytes_per_launch"],
            "GBps": round(step_traffic["bytes_per_launch"] / (ms_step * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * step_traffic["bytes_per_launch"] / (ms_step * 1e-3) / 1e9 /
                                  HBM_PEAK_GBPS, 2),
            "source": step_traffic["summary"]},
        "pack": pack,
        "ms_per_step_with_pack": round(ms_step + pack["mean_ms"], 4),
        "input_generation_s": round(gen_s, 1),
    }
    if sparse:
        del step, holder
        torch.cuda.empty_cache()
    if sparse and args.extras:
        # the same workload under its own timing protocol (3 steps from a zero
        # residual, repeated with a reset), and the lazy-zero
        # sequence of the boundary's calls, on the same resident batches
        result["protocol"] = {"deferred_depth%d" % args.depth if deferred else "lazy":
                              sparse_protocol(plan, wl, sources, w_init, "deferred" if deferred else "lazy",
                                              args.depth, layers_src)}
        if deferred:
            result["protocol"]["lazy"] = sparse_protocol(plan, wl, sources, w_init, "lazy", 0, layers_src)
            lstep, lholder = sparse_stepper(plan, wl, sources, (torch.from_numpy(w_init).cuda(),
                                                                torch.zeros(P, dtype=torch.float32, device="cuda")),
                                            "lazy", 0, layers_src)
            lms, lgms, lper, _ = time_steps(lstep, args.warmup, args.steps, 3)
            result["lazy_sequence"] = {
                "calls": "chunk_norm_layers -> chunk_topk -> sparse_gather_reduce (zero_selected=0)",
                "ms_per_step": round(lms, 4), "alg_GBps": round(b_alg / (lms * 1e-3) / 1e9, 1),
                "pct_hbm_peak_alg": round(100.0 * b_alg / (lms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                "kernels": {k: round(v["mean_ms"], 4) for k, v in
                            kernel_stats(lper, range(args.warmup, args.warmup + args.steps), names).items()}}
            log("lazy-zero sequence: %.3f ms/step" % lms)
            del lstep, lholder
        log("protocol: %s" % {k: v["step_ms_median"] for k, v in result["protocol"].items()})
    if args.cpu_baseline:
        result["cpu_baseline"], ostate = cpu_baseline(wl, plan, host_first, w_init, thr)
        del host_first
        if not variant:
            result["parity_full_size"] = full_size_parity(
                plan, wl, sources[0], w_init, "deferred" if deferred else "lazy", args.depth, layers_src, ostate)
            log("full-size parity: %s" % result["parity_full_size"])
        del ostate
    if args.extras:
        del sources, keep, states
        torch.cuda.empty_cache()
        result["dense_workloads"] = dense_summary(thr)
    print(json.dumps(result), flush=True)


def run_overlap(args):
    """Multi-bucket lazy allreduce overlapped with a stand-in backward pass.

    The producer writes every layer's gradients for all W workers, last layer
    first, each layer as one batched GEMM dW[w] = dY[w] X[w] of the layer's
    [out, in] weight shape (in = fan-in; 1 for a bias) whose reduction length
    K is the per-worker batch times the layer's output positions (AlexNet:
    55x55, 27x27 and 13x13 for conv1, conv2 and conv3-5, 1 for the fully
    connected layers; other workloads: 1), the weight-gradient half of a
    backward pass.  With --producer dense the same flops run as square
    4096 x 4096 x 4096 GEMMs (compute-bound, little HBM traffic) followed by a
    copy of a staged gradient into the layer; with --producer copy only the
    copy runs.  The reduction runs per bucket on a second
    stream, each bucket waiting on the event the producer records once the
    bucket's layers are written.  Times (HIP events, mean over --steps):
      T_prod     producer alone
      T_red      the one-launch zero-copy reduction alone (+ SGD)
      T_serial   producer, then the one-launch reduction, on one stream
      T_overlap  producer and per-bucket reductions on two streams
    (median over --steps rounds that run the five in turn).
    overlap efficiency = (T_serial - T_overlap) / min(T_prod, T_red): 1 when
    the shorter of the two is hidden entirely, 0 when nothing overlaps."""
    import torch
    import gradient_aggregation_amd as ga
    import workloads
    # CU-partitioned stream pairs for --cu-split, made before anything else
    # runs: for N in the list (a multiple of 32), one stream confined to CUs
    # 0 .. N-1 and one to the others.  (On the runtime used here a mask that
    # spreads the CUs over the chip, every 16th, was refused with error 2.)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    hip = None
    cu_streams = {}
    if args.cu_split:
        import ctypes
        # the HIP runtime this process already uses (torch's copy): a second
        # copy loaded by name would be a separate runtime
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        hip = ctypes.CDLL(path)
        words = (n_cu + 31) // 32
        for ncu in [int(x) for x in args.cu_split.split(",") if x]:
            if ncu % 32 or not 0 < ncu < n_cu:
                raise ValueError("--cu-split values must be multiples of 32 below %d" % n_cu)
            red_set = set(range(ncu))
            pair = []
            for want in (True, False):
                m = (ctypes.c_uint32 * words)()
                for c in range(n_cu):
                    if (c in red_set) == want:
                        m[c >> 5] |= 1 << (c & 31)
                h = ctypes.c_void_p()
                rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), m)
                if rc != 0:
                    raise RuntimeError("hipExtStreamCreateWithCUMask(%d CUs) returned %d" % (
                        len(red_set) if want else n_cu - len(red_set), rc))
                pair.append(h)
            cu_streams[ncu] = (red_set, pair)
    wl = workloads.WORKLOADS[args.workload if args.workload != "alexnet128_sparse" else "alexnet16"]
    if wl.mode != "dense":
        print("--overlap applies to the dense workloads", file=sys.stderr)
        sys.exit(2)
    W, P, L = wl.W, wl.P, len(wl.numels)
    gdt = torch.float16 if wl.fp16 else torch.float32
    esz = 2 if wl.fp16 else 4
    plan = ga.Plan(W, wl.numels, wl.fp16)
    torch.manual_seed(1)
    shapes = []
    for shp in wl.layers:
        out = int(shp[0])
        inn = int(np.prod(shp[1:])) if len(shp) > 1 else 1
        shapes.append((out, inn))
    positions = [1] * L
    if list(wl.layers) == list(workloads.ALEXNET_LAYERS):
        positions = [55 * 55] * 2 + [27 * 27] * 2 + [13 * 13] * 6 + [1] * 6
    Ks = [args.producer_batch * p for p in positions]
    # layer l of all workers: one [W, ldl] tensor, rows 16-byte aligned
    lds = [(n + 7) // 8 * 8 for n in wl.numels]
    layer_t = [torch.zeros((W, ld), dtype=gdt, device="cuda") for ld in lds]
    ptrs = torch.tensor([layer_t[l].data_ptr() + w * lds[l] * esz for w in range(W) for l in range(L)],
                        dtype=torch.int64, device="cuda")
    if args.producer == "gemm":
        A, B = [], []
        for l, (o, i) in enumerate(shapes):
            sc = 1.0 / np.sqrt(Ks[l])
            A.append(torch.empty((W, o, Ks[l]), dtype=gdt, device="cuda").uniform_(-sc, sc))
            B.append(torch.empty((W, Ks[l], i), dtype=gdt, device="cuda").uniform_(-1e-2, 1e-2))
        tmp = [None if lds[l] == wl.numels[l] else torch.empty((W,) + shapes[l], dtype=gdt, device="cuda")
               for l in range(L)]
        flops = float(sum(2.0 * Ks[l] * W * wl.numels[l] for l in range(L)))
    else:
        stage = [torch.randn((W, ld), device="cuda").mul_(1e-3).to(gdt) for ld in lds]
        flops = 0.0
        reps_l = [0] * L
        if args.producer == "dense":
            n = 4096
            X = torch.empty((n, n), dtype=gdt, device="cuda").uniform_(-0.02, 0.02)
            Y = torch.empty((n, n), dtype=gdt, device="cuda").uniform_(-0.02, 0.02)
            Z = torch.empty((n, n), dtype=gdt, device="cuda")
            reps_l = [int(round(2.0 * Ks[l] * W * wl.numels[l] / (2.0 * n ** 3))) for l in range(L)]
            flops = float(sum(reps_l)) * 2.0 * n ** 3

    def produce(l):
        if args.producer == "gemm":
            o, i = shapes[l]
            if tmp[l] is None:
                torch.bmm(A[l], B[l], out=layer_t[l].view(W, o, i))
            else:
                torch.bmm(A[l], B[l], out=tmp[l])
                layer_t[l][:, :wl.numels[l]].copy_(tmp[l].view(W, -1))
        else:
            for _ in range(reps_l[l]):
                torch.mm(X, Y, out=Z)
            layer_t[l].copy_(stage[l])

    wd = torch.from_numpy(workloads.weights(wl)).cuda()
    vd = torch.zeros(P, dtype=torch.float32, device="cuda")
    main = torch.cuda.current_stream()
    s_prod, s_red = torch.cuda.Stream(), torch.cuda.Stream()
    lr, mu = wl.lr, wl.mu

    def timed_interleaved(fns, reps):
        """Median time of each function, the functions run in turn so that
        clock and power drift affect them alike."""
        for _ in range(args.warmup):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
              for _ in range(reps)]
        for r in range(reps):
            for j, fn in enumerate(fns):
                ev[r][j][0].record(main)
                fn()
                ev[r][j][1].record(main)
        torch.cuda.synchronize()
        return [float(np.median([ev[r][j][0].elapsed_time(ev[r][j][1]) for r in range(reps)]))
                for j in range(len(fns))]

    def prod_all():
        for l in range(L - 1, -1, -1):
            produce(l)

    def red_all():
        plan.tree_reduce_layers(ptrs, None, wd, vd, lr, mu)

    def serial():
        prod_all()
        red_all()

    reps = args.steps or 20
    rows = []
    caps = [int(x) for x in args.reduce_workgroups.split(",") if x]
    for mb in [float(x) for x in args.bucket_mb.split(",") if x]:
        bk = ga.Buckets(plan, int(mb * (1 << 20)))
        first_to_bucket = {r[0]: i for i, r in enumerate(bk.ranges)}
        ready = [torch.cuda.Event() for _ in range(bk.count)]
        start_ev, done_p, done_r = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()
        for cap in caps:
            def overlapped():
                start_ev.record(main)
                s_prod.wait_event(start_ev)
                s_red.wait_event(start_ev)
                with torch.cuda.stream(s_prod):
                    for l in range(L - 1, -1, -1):
                        produce(l)
                        if l in first_to_bucket:
                            ready[first_to_bucket[l]].record(s_prod)
                    done_p.record(s_prod)
                with torch.cuda.stream(s_red):
                    for b in range(bk.count):
                        bk.reduce_layers(b, ptrs, ready[b], None, wd, vd, lr, mu, max_workgroups=cap)
                    done_r.record(s_red)
                main.wait_event(done_p)
                main.wait_event(done_r)

            def buckets_alone():
                for b in range(bk.count):
                    bk.reduce_layers(b, ptrs, None, None, wd, vd, lr, mu, max_workgroups=cap)

            t_prod, t_red, t_bk, t_serial, t_ov = timed_interleaved(
                [prod_all, red_all, buckets_alone, serial, overlapped], reps)
            eff = (t_serial - t_ov) / min(t_prod, t_red)
            rows.append({"bucket_mib": mb, "buckets": bk.count, "max_workgroups": cap,
                         "T_prod_ms": round(t_prod, 4), "T_red_ms": round(t_red, 4),
                         "T_red_buckets_ms": round(t_bk, 4), "T_serial_ms": round(t_serial, 4),
                         "T_overlap_ms": round(t_ov, 4), "hidden_ms": round(t_prod + t_red - t_ov, 4),
                         "efficiency": round(eff, 3)})
            log("bucket %g MiB (%d buckets), grid cap %d: T_prod %.3f, T_red %.3f (buckets %.3f), T_serial %.3f, "
                "T_overlap %.3f ms; hidden %.3f ms; efficiency %.2f" % (
                    mb, bk.count, cap, t_prod, t_red, t_bk, t_serial, t_ov, t_prod + t_red - t_ov, eff))
        for ncu in [int(x) for x in args.cu_split.split(",") if x]:
            # partitioned compute units: the reductions on CUs 0 .. ncu-1,
            # the producer on the rest
            red_set, streams = cu_streams[ncu]
            m_red, m_prod = (torch.cuda.ExternalStream(h.value) for h in streams)

            def overlapped_cu():
                start_ev.record(main)
                m_prod.wait_event(start_ev)
                m_red.wait_event(start_ev)
                with torch.cuda.stream(m_prod):
                    for l in range(L - 1, -1, -1):
                        produce(l)
                        if l in first_to_bucket:
                            ready[first_to_bucket[l]].record(m_prod)
                    done_p.record(m_prod)
                with torch.cuda.stream(m_red):
                    for b in range(bk.count):
                        bk.reduce_layers(b, ptrs, ready[b], None, wd, vd, lr, mu)
                    done_r.record(m_red)
                main.wait_event(done_p)
                main.wait_event(done_r)

            def prod_part():
                start_ev.record(main)
                m_prod.wait_event(start_ev)
                with torch.cuda.stream(m_prod):
                    prod_all()
                    done_p.record(m_prod)
                main.wait_event(done_p)

            def red_part():
                start_ev.record(main)
                m_red.wait_event(start_ev)
                with torch.cuda.stream(m_red):
                    for b in range(bk.count):
                        bk.reduce_layers(b, ptrs, None, None, wd, vd, lr, mu)
                    done_r.record(m_red)
                main.wait_event(done_r)

            t_prod, t_red, t_pp, t_rp, t_serial, t_ov = timed_interleaved(
                [prod_all, red_all, prod_part, red_part, serial, overlapped_cu], reps)
            eff = (t_serial - t_ov) / min(t_prod, t_red)
            rows.append({"bucket_mib": mb, "buckets": bk.count, "cu_split": ncu, "reduction_cus": len(red_set),
                         "T_prod_ms": round(t_prod, 4), "T_red_ms": round(t_red, 4),
                         "T_prod_on_rest_ms": round(t_pp, 4), "T_red_on_split_ms": round(t_rp, 4),
                         "T_serial_ms": round(t_serial, 4), "T_overlap_ms": round(t_ov, 4),
                         "hidden_ms": round(t_prod + t_red - t_ov, 4), "efficiency": round(eff, 3)})
            log("bucket %g MiB (%d buckets), reductions on %d CUs: T_prod %.3f (on the rest %.3f), T_red %.3f "
                "(on %d CUs %.3f), T_serial %.3f, T_overlap %.3f ms; efficiency %.2f" % (
                    mb, bk.count, len(red_set), t_prod, t_pp, t_red, len(red_set), t_rp, t_serial, t_ov, eff))
            torch.cuda.synchronize()
            del m_red, m_prod
        bk.close()
    for _, streams in cu_streams.values():
        for h in streams:
            hip.hipStreamDestroy(h)
    best = max(rows, key=lambda r: r["efficiency"])
    b_alg = W * P * esz + 16 * P
    result = {
        "metric": "computation/aggregation overlap efficiency (T_serial - T_overlap) / min(T_prod, T_red)",
        "value": best["efficiency"], "unit": "fraction", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": best["T_overlap_ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "W": W, "P": P, "grad_dtype": "f16" if wl.fp16 else "f32",
                   "producer": args.producer,
                   "producer_batch": args.producer_batch if args.producer != "copy" else None,
                   "producer_tflop": round(flops / 1e12, 4), "parallelism": "1 GPU, W workers as HBM buffers"},
        "T_red_GBps": round(b_alg / (best["T_red_ms"] * 1e-3) / 1e9, 1),
        "buckets": rows,
    }
    print(json.dumps(result), flush=True)


def run_split(args):
    """The per-GPU kernels of the dense step split across G GPUs, at their
    real shapes: ga_tree_partial over one GPU's W/G workers (all P elements)
    and ga_tree_combine over the G partial rows of one owner's slice of
    ceil(P/G) elements (mean and SGD included).  The exchange between them
    (a reduce-scatter of P*4 bytes per GPU) is not run; its bytes are given."""
    import torch
    import gradient_aggregation_amd as ga
    import workloads
    wl = workloads.WORKLOADS[args.workload]
    W, G, P = wl.W, args.split, wl.P
    m = W // G if G > 0 else 0
    if G < 1 or m * G != W or m & (m - 1):
        print("--split G needs W/G a power of two (W=%d)" % W, file=sys.stderr)
        sys.exit(2)
    gdt = torch.float16 if wl.fp16 else torch.float32
    torch.manual_seed(3)
    grp = ga.Plan(m, wl.numels, wl.fp16)
    bucket = (torch.randn((m, grp.ld), device="cuda") * 1e-3).to(gdt)
    part_out = torch.empty(P, dtype=torch.float32, device="cuda")
    Q = ((P + G - 1) // G + 63) // 64 * 64
    own = ga.Plan(G, [Q], False)
    partials = torch.randn((G, own.ld), device="cuda") * 1e-3
    g = torch.empty(Q, dtype=torch.float32, device="cuda")
    w = torch.randn(Q, device="cuda") * 0.05
    v = torch.zeros(Q, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    steps = args.steps or 200

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    t_part = timed(lambda: grp.tree_partial(bucket, part_out))
    t_comb = timed(lambda: own.tree_combine(partials, W, None, w, v, wl.lr, wl.mu))
    b_in = 2 if wl.fp16 else 4
    part_bytes = m * P * b_in + 4 * P
    comb_bytes = G * Q * 4 + 16 * Q
    xchg = (G - 1) * ((P + G - 1) // G) * 4
    print(json.dumps({
        "metric": "per-GPU kernels of the dense step split across GPUs", "workload": wl.name, "W": W, "G": G,
        "workers_per_gpu": m, "P": P, "slice": Q, "steps": steps,
        "partial_ms": round(t_part, 4), "partial_GBps": round(part_bytes / (t_part * 1e-3) / 1e9, 1),
        "combine_ms": round(t_comb, 4), "combine_GBps": round(comb_bytes / (t_comb * 1e-3) / 1e9, 1),
        "exchange_bytes_per_gpu": xchg,
        "exchange_ms_at_7_links_153GBps": round(xchg / (7 * 153e9) * 1e3, 4),
        "data": "synthetic"}), flush=True)


def time_pack(plan, wl, src, layer_tensors, stream):
    """Lazy-allreduce fusion as a copy, measured on its own: the W*L layer
    tensors of one gradient batch are packed into a fresh bucket by
    ga_bucket_pack (context for producers that need a materialized bucket)."""
    import torch
    offs = np.cumsum([0] + wl.numels)
    if layer_tensors is not None:
        table = src
    else:
        esz = src.element_size()
        table = torch.tensor([src.data_ptr() + (w * plan.ld + int(offs[l])) * esz
                              for w in range(wl.W) for l in range(len(wl.numels))], dtype=torch.int64,
                             device="cuda")
    dst = plan.empty_bucket()
    for _ in range(2):
        plan.bucket_pack(table, dst)
    reps = 5
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        plan.bucket_pack(table, dst)
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    d = [ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]
    ok = True
    for w in (0, wl.W - 1):
        ref = torch.cat(layer_tensors[w]) if layer_tensors is not None else src[w, :wl.P]
        ok = ok and bool(torch.equal(dst[w, :wl.P], ref))
    del dst
    esz = 2 if wl.fp16 else 4
    moved = 2 * wl.W * wl.P * esz
    return {"kernel": "k_pack", "layers": len(wl.numels), "tensors": wl.W * len(wl.numels),
            "mean_ms": round(float(np.mean(d)), 4), "GBps": round(moved / (np.mean(d) * 1e-3) / 1e9, 1),
            "bytes": moved, "matches_source": ok}


def selection_stats(plan, prev, cur, P):
    """Chunk counts of one step's selection (cur) against the previous step's
    (prev, or None): (worker, chunk) pairs sent, sent again, newly sent, and
    the chunks some worker sent."""
    import torch
    n_c = plan.n_chunks
    sh = torch.arange(32, device=cur.device, dtype=torch.int32)

    def bits(m):
        return (((m.unsqueeze(-1) >> sh) & 1) != 0).reshape(m.shape[0], -1)[:, :n_c]

    bc = bits(cur)
    bp = bits(prev) if prev is not None else torch.zeros_like(bc)
    return {"pairs_sent": int(bc.sum()), "pairs_sent_again": int((bp & bc).sum()),
            "pairs_newly_sent": int((bc & ~bp).sum()), "chunks_sent_by_any_worker": int(bc.any(dim=0).sum()),
            "n_chunks": int(n_c)}


def code_digest(texts):
    """SHA-256 of C/C++ sources with comments and all whitespace removed: a
    change to the code changes it, a change to a comment or to the layout of
    the lines does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for t in texts:
        t = t.replace("\\\n", "")   # continued lines spliced first, as C does
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(re.sub(r"\s+", "", t).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic(path, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    or None when there is none or the code of the kernel's sources changed since it
    was taken (comments aside)."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    texts = []
    for src in rec["sources"]:
        path_src = os.path.join(ROOT, src)
        if not os.path.exists(path_src):
            return None
        with open(path_src) as f:
            texts.append(f.read())
    return rec if code_digest(texts) == rec.get("code_sha256") else None


def cpu_baseline(wl, plan, host_bucket, w_init, thr, min_s=10.0, max_steps=5):
    """The oracle, as it is, timed on the host cores: whole steps of the
    workload (all W workers) on the first gradient batch, repeated until at
    least `min_s` seconds of work (at most `max_steps` steps); the sparse
    residual and the w, v state carry over from step to step.  Returns the
    record and the oracle's final state (steps, w, v, residual or None)."""
    import oracle
    P = wl.P
    b_in = 2 if wl.fp16 else 4
    sparse = wl.mode == "sparse"
    w = w_init.copy()
    v = np.zeros(P, np.float32)
    r = np.zeros(host_bucket.shape, np.float32) if sparse else None
    steps = 0
    t0 = time.time()
    while True:
        if sparse:
            oracle.sparse_step(host_bucket, P, wl.fp16, wl.chunk, plan.k, r, wl.lr, wl.mu, w, v,
                               want_keys=False, want_gbar=False, threads=thr)
        else:
            oracle.dense_step(host_bucket, P, wl.fp16, wl.lr, wl.mu, w, v, want_gbar=False, threads=thr)
        steps += 1
        if time.time() - t0 >= min_s or steps >= max_steps:
            break
    total = time.time() - t0
    t = total / steps
    b_alg = wl.W * P * ((b_in + 8) if sparse else b_in) + 16 * P
    log("cpu baseline: %d oracle steps over all %d workers in %.2fs on %d threads" % (steps, wl.W, total, thr))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rec = {"value": round(b_alg / t / 1e9, 3), "unit": "GB/s", "cores": thr, "kind": "oracle",
           "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
           "sample": "%d consecutive whole %s steps of the workload (all %d workers, P=%d) on the first "
                     "gradient batch, oracle threads=%d, %.2f s in all, %.2f s per step"
                     % (steps, wl.mode, wl.W, P, thr, total, t)}
    return rec, (steps, w, v, r)


def full_size_parity(plan, wl, src0, w_init, mode, depth, layers_src, ostate):
    """The timed path run on the first gradient batch for as many steps as the
    oracle ran in cpu_baseline, from the same initial state, and compared with
    the oracle's final w, v and residual (every worker, every element, on the
    device one worker row at a time).  The deferred form gets one layer table
    per step (copies of the first batch's table: the same tensors, unchanged,
    as its history requires) and is flushed; in the lazy-zero form the chunks
    of the last mask are +0.  Bit patterns are compared; +0 against -0 would
    show as a difference."""
    import torch
    steps, w_ref, v_ref, r_ref = ostate
    P, W = wl.P, wl.W
    wd = torch.from_numpy(w_init).cuda()
    vd = torch.zeros(P, dtype=torch.float32, device="cuda")
    if r_ref is None:
        for _ in range(steps):
            if layers_src:
                plan.tree_reduce_layers(src0, None, wd, vd, wl.lr, wl.mu)
            else:
                plan.tree_reduce(src0, None, wd, vd, wl.lr, wl.mu)
        resid, mask = None, None
    else:
        srcs = [src0.clone() for _ in range(steps)] if layers_src else [src0] * steps
        step, holder = sparse_stepper(plan, wl, srcs, (wd, vd), mode, depth, layers_src)
        ev = [torch.cuda.Event() for _ in range(3)]
        for t in range(steps):
            step(t, ev)
        if mode == "deferred":
            resid, mask = holder.flush(), None
        else:
            resid, mask = holder.resid, holder.mask
    torch.cuda.synchronize()

    def same(a, ref):
        return torch.equal(a.view(torch.int32), torch.from_numpy(ref).cuda().view(torch.int32))

    out = {"steps": steps, "form": ("deferred, depth %d" % depth) if mode == "deferred" and r_ref is not None
           else ("lazy-zero" if r_ref is not None else "dense tree"),
           "against": "the oracle's state after the cpu_baseline steps",
           "w": "bitwise" if same(wd, w_ref) else "differs",
           "v": "bitwise" if same(vd, v_ref) else "differs"}
    if r_ref is not None:
        C = plan.chunk
        cid = torch.arange(P, device="cuda") // C
        bad = 0
        for wk in range(W):
            row = resid[wk, :P]
            if mask is not None:
                bits = (mask[wk][cid >> 5] >> (cid & 31)) & 1
                row = torch.where(bits.bool(), torch.zeros_like(row), row)
            ref = torch.from_numpy(r_ref[wk, :P]).cuda()
            bad += int((row.view(torch.int32) != ref.view(torch.int32)).sum())
        out["residual"] = "bitwise, all %d workers" % W if bad == 0 else "%d elements differ" % bad
        del cid, holder, step, srcs
    del wd, vd, resid
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
