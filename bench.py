"""Benchmark of the tree-verify MLA-absorb attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload kimi] [--no-cpu-baseline]
                    [--cold-steps C] [--attn-event-every E] [--staged]

A step is one pass of the whole path over one synthetic batch already resident in HBM:
ancestor bitmasks from the parent array, the ragged plan, the attention and the split combine.
For one request of bf16 inputs (the Kimi shape, decode, small trees, chains and prefill chunks)
the masks and the plan are made inside the attention launch (kdt_tree_verify_prepare_attend):
two launches per step; several requests, fp32 inputs, and --staged, run masks + plan as a launch
of their own.  The default workload is
the Kimi/DeepSeekV3-shape request (H = 64 heads, latent 512 + rope 64, bf16, committed cache
4096 tokens, a 64-node best-first draft tree).

One JSON line is printed.  `value` is algorithmic TFLOP/s of the whole step;
`roofline` rates the attention launch alone (HIP events around its launches in every E-th
step of the timed region, on the stream it runs on, recorded without a system-scope cache
fence so that timing does not add cache write-backs to the step) against the roof that binds it (bf16 MFMA peak, or
HBM bandwidth when the algorithmic intensity is below the ridge point), with `traffic` the HBM
bytes per launch from the committed rocprofv3 counter summary (null when the kernel sources
changed since it was taken); `cpu_baseline` times the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBPS = 8000.0

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Timing events of the HIP runtime the process already runs (torch's), created with
    hipEventDisableSystemFence: recording one does not write back and invalidate the caches
    (a default event's system-scope fence does, which between two kernels of a step costs
    several microseconds, most of it writing back the split partials).  The timestamps still
    follow the completion of the work recorded before them."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        # by soname: dlopen returns the runtime torch has loaded, not a second copy
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.flags = HIP_EVENT_DISABLE_SYSTEM_FENCE
        self.events = []

    def create(self):
        ev = self.ct.c_void_p()
        err = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.flags)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        err = self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        err = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return float(ms.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def tree_depth_sum(parents: np.ndarray) -> np.ndarray:
    """Sum over nodes of the root-to-node path length (= visible tree keys), per request."""
    B, N = parents.shape
    depth = np.zeros((B, N), np.int64)
    for b in range(B):
        for i in range(N):
            p = parents[b, i]
            depth[b, i] = 1 + (depth[b, p] if p >= 0 else 0)
    return depth.sum(axis=1)


def algorithmic_work(inp: workloads.Inputs):
    """(flops, bytes, cache_bytes) that the method must do: cache pairs plus visible tree pairs."""
    sp = inp.spec
    D, dc = sp.d_latent + sp.d_rope, sp.d_latent
    e = 2 if sp.dtype == "bf16" else 4
    R = sp.nodes * sp.heads
    lens = inp.cache_lens.numpy().astype(np.int64)
    vis_tree = tree_depth_sum(inp.parents.numpy())
    flops = float(np.sum(2 * R * lens * (D + dc)) + np.sum(2 * sp.heads * (D + dc) * vis_tree))
    W = (sp.nodes + 63) // 64
    cache_bytes = float(lens.sum() * D * e)
    by = cache_bytes + sp.batch * R * D * e + sp.batch * sp.nodes * D * e + sp.batch * sp.nodes * W * 8 \
        + sp.batch * R * dc * 4
    return flops, by, cache_bytes


def run(args):
    import tree_verify_mla_02_amd as kdt

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = workloads.make_inputs(args.workload, seed=args.seed)
    sp = inp.spec
    flops, nbytes, cache_bytes = algorithmic_work(inp)

    parents = inp.parents.to(dev)
    lens = inp.cache_lens.to(dev)
    q_lat, q_rope = inp.q_lat.to(dev), inp.q_rope.to(dev)
    kv, tkv = inp.kv_cache.to(dev), inp.tree_kv.to(dev)
    dc = sp.d_latent
    ckv, krope, tckv, tkrope = kv[:, :dc], kv[:, dc:], tkv[:, :, :dc], tkv[:, :, dc:]
    maxL, total = int(inp.cache_lens.max()), inp.total_len
    desc = kdt.make_desc(q_lat, q_rope, ckv, krope, tckv, tkrope, maxL, total)
    ws = kdt.alloc_workspace(desc, dev)
    masks = torch.empty((sp.batch, sp.nodes, (sp.nodes + 63) // 64), dtype=torch.int64, device=dev)
    out = torch.empty((sp.batch, sp.nodes, sp.heads, dc), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # masks, plan and attention in one launch where the batch allows (one bf16 request), else
    # prepare and attend; --staged times the three launches everywhere
    one_launch = not getattr(args, "staged", False) and kdt.prepare_attend_launches(desc) == 1

    def prep():
        if not one_launch:
            kdt.prepare(parents, lens, desc, ws, masks_out=masks, dev_status=status, stream=stream)

    def attend():
        if one_launch:
            kdt.prepare_attend(parents, lens, q_lat, q_rope, ckv, krope, tckv, tkrope, inp.scale, out, desc, ws,
                               masks_out=masks, dev_status=status, stream=stream)
        else:
            kdt.attend(q_lat, q_rope, ckv, krope, tckv, tkrope, masks, inp.scale, out, desc, ws, stream=stream)

    def step():
        prep()
        attend()
        kdt.combine(out, desc, ws, stream=stream)

    step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())} on the benchmark inputs")
    # the outputs of a first step against the oracle before anything is timed: masks bit for
    # bit, attention rows within the tolerance (every row up to ~40 GFLOP of oracle work, else
    # one row of every 32-row group of every request plus random rows).  The warm-up comes after
    # it: the GPU clock falls while the host runs the oracle, and from idle it takes some 50 ms
    # of back-to-back steps to settle (the Kimi step runs about 10 % slower before that).
    check = check_outputs(inp, masks, out)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())} on the benchmark inputs")

    # ---- timed region: K whole steps; the attention launches of every E-th step are bracketed
    # by events on the stream they run on (the same stream as the rest of the step).  Each
    # recorded event is a command-processor round trip between two kernels (a few microseconds
    # of a 60-microsecond step when every step records two), so they are recorded on a sample
    # of the timed steps.
    he = HipEvents()
    every = max(1, args.attn_event_every)
    sampled = [i for i in range(args.steps) if i % every == 0]
    evs = {i: (he.create(), he.create()) for i in sampled}

    def timed_step(i):
        prep()
        if i in evs:
            he.record(evs[i][0], stream)
        attend()
        if i in evs:
            he.record(evs[i][1], stream)
        kdt.combine(out, desc, ws, stream=stream)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = he.create(), he.create()
    he.record(ev0, stream)
    for i in range(args.steps):
        timed_step(i)
    host_ms = (time.perf_counter() - t0) * 1e3
    he.record(ev1, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = he.elapsed_ms(ev0, ev1) / args.steps
    attn_each = np.array([he.elapsed_ms(*evs[i]) for i in sampled])
    attn_ms = float(attn_each.mean())

    # ---- cold caches: before each of a few steps, write a 512 MiB scratch buffer (twice the
    # 256 MB Infinity Cache) so the step starts with cold L2 and MALL; the attention launch and
    # the whole step are timed
    cold, cold_step = [], []
    if args.cold_steps:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for _ in range(args.cold_steps):
            scratch.fill_(1)
            s0, a0, a1, s1 = he.create(), he.create(), he.create(), he.create()
            he.record(s0, stream)
            prep()
            he.record(a0, stream)
            attend()
            he.record(a1, stream)
            kdt.combine(out, desc, ws, stream=stream)
            he.record(s1, stream)
            torch.cuda.synchronize()
            cold.append(he.elapsed_ms(a0, a1))
            cold_step.append(he.elapsed_ms(s0, s1))
        del scratch
    he.close()

    # the roof that binds: MFMA when the algorithmic intensity is above the ridge point
    mfma_peak = PEAK_BF16_TFLOPS if sp.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBPS * 1e9)
    hbm_bound = flops / nbytes < ridge
    if hbm_bound:
        bound, peak, unit_r = "hbm", PEAK_HBM_GBPS, "GB/s"
        achieved = nbytes / (attn_ms * 1e-3) / 1e9
    else:
        bound, peak, unit_r = "mfma", mfma_peak, "TFLOP/s"
        achieved = flops / (attn_ms * 1e-3) / 1e12

    def frac(ms):
        """Fraction of the binding roof reached by a region of `ms` milliseconds."""
        if ms is None:
            return None
        rate = nbytes / (ms * 1e-3) / 1e9 if hbm_bound else flops / (ms * 1e-3) / 1e12
        return round(rate / peak, 4)
    cold_ms = float(np.median(cold)) if cold else None
    cold_step_ms = float(np.median(cold_step)) if cold_step else None
    value = flops / (step_ms * 1e-3) / 1e12
    line = {
        "metric": "tree-verify attn TFLOP/s + cache GB/s, % of MI355X roofline, Kimi-shape N=64 tree",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic (seeded N(0,1) inputs, best-first draft tree)",
        "config": {
            "workload": f"{sp.name}: B={sp.batch} requests, N={sp.nodes} tree nodes, H={sp.heads} heads, "
                        f"d_latent={sp.d_latent}, d_rope={sp.d_rope}, cache={maxL} tokens, {sp.dtype}",
            "batch": sp.batch, "nodes": sp.nodes, "heads": sp.heads, "cache_len": maxL,
            "total_cache_tokens": total, "tree": sp.tree, "splits": kdt.num_splits(desc),
        },
        "cache_gbps": round(cache_bytes / (step_ms * 1e-3) / 1e9, 2),
        "alg_gflop_per_step": round(flops / 1e9, 4),
        "alg_mbytes_per_step": round(nbytes / 1e6, 4),
        # the attention launch: with one_launch it also makes the masks and the plan (no
        # prepare launch in the step)
        "launches_per_step": (2 if one_launch else 3) if kdt.num_splits(desc) > 1 else (1 if one_launch else 2),
        "attn_launch": "masks + plan + attention" if one_launch else "attention",
        "attn_kernel_ms": round(attn_ms, 5),
        "attn_kernel_samples": len(sampled),
        "attn_kernel_ms_p10_p50_p90": [round(float(np.percentile(attn_each, q)), 5) for q in (10, 50, 90)],
        "attn_kernel_cold_ms_median": round(cold_ms, 5) if cold else None,
        "step_cold_ms_median": round(cold_step_ms, 5) if cold_step else None,
        # the binding roof's fraction over other regions: the attention launch with cold caches,
        # and the whole step (masks + plan, attention, combine), hot and cold
        "frac_attn_cold": frac(cold_ms),
        "frac_step_hot": frac(step_ms),
        "frac_step_cold": frac(cold_step_ms),
        "output_check": check,
        "arith_intensity_flop_per_byte": round(flops / nbytes, 1),
        "kernel_source_hash": kernel_source_hash(),
        "wall_ms_timed_region": round(wall_ms, 3),
        "host_launch_ms_per_step": round(host_ms / args.steps, 5),
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": unit_r,
            "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(sp.name),
        },
    }
    return line, inp


def check_outputs(inp, masks, out):
    """Compare the device masks and outputs of a finished step with the fp64 oracle; exits
    with an error when they differ.  Returns a short description of what was compared."""
    import oracle
    sp = inp.spec
    ref_masks, _ = oracle.visibility(inp.parents.numpy())
    if not np.array_equal(masks.cpu().numpy().view(np.uint64), ref_masks):
        raise SystemExit("masks differ from the oracle on the benchmark inputs")
    flops, _, _ = algorithmic_work(inp)
    R = sp.nodes * sp.heads
    total = sp.batch * R
    if flops <= 40e9:
        rows = None
    else:
        rng = np.random.default_rng(12345)
        per_group = [b * R + np.minimum(np.arange(0, R, 32) + rng.integers(0, 32, size=(R + 31) // 32), R - 1)
                     for b in range(sp.batch)]
        rows = np.unique(np.concatenate(per_group + [rng.integers(0, total, size=256)]))
    cores = len(os.sched_getaffinity(0))
    ref = oracle.run(inp, rows=rows, threads=cores)[1].reshape(-1, sp.d_latent)
    got = out.reshape(-1, sp.d_latent)
    if rows is not None:
        got = got[torch.from_numpy(rows).to(out.device)]
    got = got.cpu().double().numpy()
    err = float(np.abs(got - ref).max())
    tol = 2e-3 if sp.dtype == "bf16" else 1e-5
    if not np.isfinite(got).all() or err > tol:
        raise SystemExit(f"attention max-abs error {err} above {tol} on the benchmark inputs")
    what = f"all {total} rows" if rows is None else f"{rows.size} of {total} rows (one per 32-row group + random)"
    return {"masks": "bit-exact", "rows": what, "max_abs_err": float(f"{err:.3e}"), "tol": tol}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, min_seconds=10.0, max_seconds=30.0):
    """The fp64 oracle on the host cores: whole steps (masks + every output row) of the same
    workload, repeated until about min_seconds of CPU work (at most max_seconds)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    flops, _, _ = algorithmic_work(inp)
    oracle.build()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run(inp, threads=cores)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt * (reps + 1) / reps > max_seconds:
            break
    rows = inp.spec.batch * inp.spec.nodes * inp.spec.heads
    return {"value": round(reps * flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} whole step(s) of the same workload (masks + all {rows} rows, fp64) "
                      f"in {dt:.2f} s on {cores} threads", "cpu_model": cpu_model()}


def accept_inputs(inp, seed):
    """Drafted tokens (distinct among siblings) and target predictions that follow a random
    root-to-leaf walk (its first step always, each later one with probability 0.85), for the
    workload's trees."""
    par = inp.parents.numpy()
    B, N = par.shape
    rng = np.random.default_rng([seed, 77])
    tok = rng.permutation(B * N * 4)[: B * N].reshape(B, N).astype(np.int32)
    nxt, root = guided_predictions(par, tok, rng)
    return par.astype(np.int32), tok, nxt, root


def run_next_row(args):
    """The greedy tree-accept or the KV compaction kernel alone: K launches bracketed by
    fence-free events, each launch on the same inputs (both kernels are idempotent)."""
    import tree_verify_mla_02_amd as kdt
    from oracle import accept as oracle_accept
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = workloads.make_inputs(args.workload, seed=args.seed)
    sp = inp.spec
    par, tok, nxt, root = accept_inputs(inp, args.seed)
    B, N = par.shape
    d_par, d_tok, d_nxt, d_root = (torch.from_numpy(x).to(dev) for x in (par, tok, nxt, root))
    stream = torch.cuda.current_stream(dev)
    path, acc, bonus = kdt.tree_accept(d_par, d_tok, d_nxt, d_root, stream=stream)
    torch.cuda.synchronize()
    he = HipEvents()
    if args.row == "accept":
        def launch():
            kdt.tree_accept(d_par, d_tok, d_nxt, d_root, path, acc, bonus, stream=stream)
        # bytes the walk must touch: the three [B, N] arrays and root_next, the outputs
        nbytes = B * N * 12 + B * 4 + B * N * 4 + B * 8
        work = B
    else:
        dc = sp.d_latent
        kv, tkv = inp.kv_cache.to(dev), inp.tree_kv.to(dev)
        lens_np = inp.cache_lens.numpy().astype(np.int64)
        T = int(lens_np.sum())
        acc_np = acc.cpu().numpy().astype(np.int64)
        rows = T + int(acc_np.sum())
        out = torch.empty((rows, kv.shape[1]), dtype=kv.dtype, device=dev)
        q_lat = torch.empty((B, N, 1, dc), dtype=kv.dtype, device=dev)
        q_rope = torch.empty((B, N, 1, kv.shape[1] - dc), dtype=kv.dtype, device=dev)
        desc = kdt.make_desc(q_lat, q_rope, kv[:, :dc], kv[:, dc:], tkv[:, :, :dc], tkv[:, :, dc:],
                             int(lens_np.max()), T)
        d_lens = inp.cache_lens.to(dev)
        new_lens = torch.empty(B, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def launch():
            kdt.kv_compact(kv[:, :dc], kv[:, dc:], d_lens, tkv[:, :, :dc], tkv[:, :, dc:], path, acc, desc,
                           out[:, :dc], out[:, dc:], new_lens=new_lens, capacity_rows=rows, dev_status=status,
                           stream=stream)
        e = kv.element_size()
        nbytes = 2 * rows * kv.shape[1] * e          # every new row read once and written once
        work = rows
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    if args.row == "compact" and int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())} on the benchmark inputs")
    evs = [(he.create(), he.create()) for _ in range(args.steps)]
    ev0, ev1 = he.create(), he.create()
    he.record(ev0, stream)
    for i in range(args.steps):
        he.record(evs[i][0], stream)
        launch()
        he.record(evs[i][1], stream)
    he.record(ev1, stream)
    torch.cuda.synchronize()
    step_ms = he.elapsed_ms(ev0, ev1) / args.steps
    each = np.array([he.elapsed_ms(a, b) for a, b in evs])
    he.close()
    k_ms = float(each.mean())
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    line = {
        "metric": "greedy tree-accept requests/s" if args.row == "accept" else "post-verify KV compaction GB/s",
        "value": round(work / (step_ms * 1e-3), 3) if args.row == "accept" else round(nbytes / (step_ms * 1e-3) / 1e9, 3),
        "unit": "requests/s" if args.row == "accept" else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32" if args.row == "accept" else sp.dtype,
        "data": "synthetic (seeded tokens and target predictions on the workload's draft trees)",
        "config": {"workload": f"{args.row} on {sp.name}: B={B} requests, N={N} nodes"
                               + (f", {int(inp.cache_lens.sum())} committed + {work - int(inp.cache_lens.sum())}"
                                  f" accepted rows of {(sp.d_latent + sp.d_rope)} {sp.dtype}" if args.row == "compact" else ""),
                   "batch": B, "nodes": N},
        "kernel_ms": round(k_ms, 5),
        "kernel_ms_p10_p50_p90": [round(float(np.percentile(each, q)), 5) for q in (10, 50, 90)],
        "kernel_source_hash": kernel_source_hash("tree_accept" if args.row == "accept" else "kv_compact"),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": recorded_traffic(sp.name, "kv_compact") if args.row == "compact" else None},
    }
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        reps, t0 = 0, time.perf_counter()
        while True:
            if args.row == "accept":
                oracle_accept.tree_accept(par, tok, nxt, root)
            else:
                oracle_accept.kv_compact(inp.kv_cache[:, :dc].view(torch.int16).numpy(),
                                         inp.kv_cache[:, dc:].view(torch.int16).numpy(), lens_np,
                                         inp.tree_kv[:, :, :dc].view(torch.int16).numpy(),
                                         inp.tree_kv[:, :, dc:].view(torch.int16).numpy(),
                                         path.cpu().numpy(), acc_np)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or dt * (reps + 1) / reps > 30.0:
                break
        line["cpu_baseline"] = {
            "value": round(reps * work / dt, 3) if args.row == "accept" else round(reps * nbytes / dt / 1e9, 3),
            "unit": line["unit"], "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole launch(es) of the same inputs in {dt:.2f} s (plain Python / numpy, one thread)"}
    return line


def run_tree_row(args):
    """The best-first tree builder alone on the workload's tree shape (requests, nodes, depth,
    top-k): K launches bracketed by fence-free events on the same drafter log probabilities."""
    import tree_verify_mla_02_amd as kdt
    from oracle import tree_build as oracle_tree
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sp = workloads.SPECS[args.workload]
    B, N = sp.batch, sp.nodes
    D, K = (sp.depth, sp.topk) if sp.tree == "bestfirst" else (8, 8)
    rng = np.random.default_rng([args.seed, 91])
    lp = np.stack([workloads.drafter_logprobs(rng, D, K) for _ in range(B)]).astype(np.float32)
    cand = rng.integers(0, 160000, size=(B, D, K)).astype(np.int32)
    d_lp, d_cand = torch.from_numpy(lp).to(dev), torch.from_numpy(cand).to(dev)
    stream = torch.cuda.current_stream(dev)
    outs = kdt.build_tree(d_lp, d_cand, N, stream=stream)
    torch.cuda.synchronize()
    want = oracle_tree.best_first_tree(lp, cand, N)
    for g, w in zip(outs, want):
        if not np.array_equal(g.cpu().numpy(), w):
            raise SystemExit("tree builder output differs from the oracle on the benchmark inputs")

    def launch():
        kdt.build_tree(d_lp, d_cand, N, *outs, stream=stream)
    he = HipEvents()
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    evs = [(he.create(), he.create()) for _ in range(args.steps)]
    ev0, ev1 = he.create(), he.create()
    he.record(ev0, stream)
    for i in range(args.steps):
        he.record(evs[i][0], stream)
        launch()
        he.record(evs[i][1], stream)
    he.record(ev1, stream)
    torch.cuda.synchronize()
    step_ms = he.elapsed_ms(ev0, ev1) / args.steps
    each = np.array([he.elapsed_ms(a, b) for a, b in evs])
    he.close()
    k_ms = float(each.mean())
    line = {
        "metric": "best-first draft-tree build requests/s", "value": round(B / (step_ms * 1e-3), 3),
        "unit": "requests/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded drafter log probabilities, logits N(0, 2^2), sorted per depth)",
        "config": {"workload": f"tree on {sp.name}: B={B} requests, N={N} nodes, depth<={D}, top-{K}",
                   "batch": B, "nodes": N, "depth": D, "topk": K},
        "kernel_ms": round(k_ms, 5),
        "kernel_ms_p10_p50_p90": [round(float(np.percentile(each, q)), 5) for q in (10, 50, 90)],
        "kernel_source_hash": kernel_source_hash("tree_build"),
        # the pops of one request form one dependent chain: the bound is its latency per node
        "roofline": {"bound": "latency", "achieved": round(k_ms * 1e6 / N, 2), "peak": None,
                     "unit": "ns per node (serial pops of one request)", "frac": None, "traffic": None},
    }
    if not args.no_cpu_baseline:
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle_tree.best_first_tree(lp, cand, N)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or dt * (reps + 1) / reps > 30.0:
                break
        line["cpu_baseline"] = {
            "value": round(reps * B / dt, 3), "unit": "requests/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole launch(es) of the same inputs in {dt:.2f} s (plain Python heapq, one thread)"}
    return line


def guided_predictions(par, tok, rng, hit=0.85):
    """Synthetic target predictions for a batch of trees: the target's greedy tokens follow a
    random root-to-leaf walk (its first step always, each later one with probability `hit`),
    anything else elsewhere; the verify kernels never see them, only the accept step does."""
    B, N = par.shape
    nxt = rng.integers(0, 1 << 20, size=(B, N)).astype(np.int32)
    root = rng.integers(0, 1 << 20, size=B).astype(np.int32)
    for b in range(B):
        kids = {}
        for j in range(N):
            kids.setdefault(int(par[b, j]), []).append(j)
        cur = -1
        while kids.get(cur) and (cur < 0 or rng.random() < hit):
            j = int(rng.choice(kids[cur]))
            if cur < 0:
                root[b] = tok[b, j]
            else:
                nxt[b, cur] = tok[b, j]
            cur = j
    return nxt, root


def run_step_row(args):
    """One whole speculative verify step on the GPU, stream-ordered with no host sync between
    its stages: best-first tree build -> masks + plan -> attention -> combine -> greedy accept
    -> KV compaction.  Checked once against the oracle chain, then K steps timed with
    fence-free events between the stages."""
    import dataclasses

    import oracle
    import tree_verify_mla_02_amd as kdt
    from oracle import accept as oracle_accept
    from oracle import tree_build as oracle_tree
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = workloads.make_inputs(args.workload, seed=args.seed)
    sp = inp.spec
    B, N, H, dc = sp.batch, sp.nodes, sp.heads, sp.d_latent
    D, K = (sp.depth, sp.topk) if sp.tree == "bestfirst" else (8, 8)
    rng = np.random.default_rng([args.seed, 93])
    lp = np.stack([workloads.drafter_logprobs(rng, D, K) for _ in range(B)]).astype(np.float32)
    cand = rng.permutation(1 << 20)[: B * D * K].reshape(B, D, K).astype(np.int32)   # distinct token ids
    par_ref, tok_ref, _, _ = oracle_tree.best_first_tree(lp, cand, N)
    if (par_ref < -1).any():
        raise SystemExit(f"depth {D} x top-{K} has fewer than {N} paths")
    nxt, root = guided_predictions(par_ref, tok_ref, rng)
    inp = dataclasses.replace(inp, parents=torch.from_numpy(par_ref.copy()))

    d_lp, d_cand = torch.from_numpy(lp).to(dev), torch.from_numpy(cand).to(dev)
    d_nxt, d_root = torch.from_numpy(nxt).to(dev), torch.from_numpy(root).to(dev)
    lens = inp.cache_lens.to(dev)
    q_lat, q_rope = inp.q_lat.to(dev), inp.q_rope.to(dev)
    maxL, T = int(inp.cache_lens.max()), inp.total_len
    # the cache buffer has room for N more rows per request; one request compacts in place
    # (only its accepted rows move), a batch into a second buffer
    in_place = B == 1
    cap = T + B * N
    kv = torch.empty((cap, inp.kv_cache.shape[1]), dtype=inp.kv_cache.dtype, device=dev)
    kv[:T] = inp.kv_cache.to(dev)
    tkv = inp.tree_kv.to(dev)
    ckv, krope, tckv, tkrope = kv[:, :dc], kv[:, dc:], tkv[:, :, :dc], tkv[:, :, dc:]
    desc = kdt.make_desc(q_lat, q_rope, ckv, krope, tckv, tkrope, maxL, T)
    ws = kdt.alloc_workspace(desc, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    parents, tokens, depth, rank = (torch.empty((B, N), **i32) for _ in range(4))
    masks = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=dev)
    out = torch.empty((B, N, H, dc), dtype=torch.float32, device=dev)
    path, acc, bonus, new_lens = torch.empty((B, N), **i32), torch.empty(B, **i32), torch.empty(B, **i32), \
        torch.empty(B, **i32)
    kv_out = kv if in_place else torch.empty((cap, kv.shape[1]), dtype=kv.dtype, device=dev)
    status = torch.zeros(1, **i32)
    stream = torch.cuda.current_stream(dev)
    one_launch = not getattr(args, "staged", False) and kdt.prepare_attend_launches(desc) == 1

    def step(rec=None):
        mark = (lambda k: rec(k)) if rec else (lambda k: None)
        mark(0)
        kdt.build_tree(d_lp, d_cand, N, parents, tokens, depth, rank, stream=stream)
        mark(1)
        if not one_launch:
            kdt.prepare(parents, lens, desc, ws, masks_out=masks, dev_status=status, stream=stream)
        mark(2)
        if one_launch:
            kdt.prepare_attend(parents, lens, q_lat, q_rope, ckv, krope, tckv, tkrope, inp.scale, out, desc, ws,
                               masks_out=masks, dev_status=status, stream=stream)
        else:
            kdt.attend(q_lat, q_rope, ckv, krope, tckv, tkrope, masks, inp.scale, out, desc, ws, stream=stream)
        mark(3)
        kdt.combine(out, desc, ws, stream=stream)
        mark(4)
        kdt.tree_accept(parents, tokens, d_nxt, d_root, path, acc, bonus, stream=stream)
        mark(5)
        kdt.kv_compact(ckv, krope, lens, tckv, tkrope, path, acc, desc, kv_out[:, :dc], kv_out[:, dc:],
                       new_lens=new_lens, capacity_rows=cap, dev_status=status, stream=stream)
        mark(6)

    step()
    torch.cuda.synchronize()
    # ---- the chain against the oracle chain: integer stages bit for bit, attention sampled rows
    if int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())} on the benchmark inputs")
    if not (np.array_equal(parents.cpu().numpy(), par_ref) and np.array_equal(tokens.cpu().numpy(), tok_ref)):
        raise SystemExit("tree differs from the oracle")
    ref_masks, _ = oracle.visibility(par_ref)
    if not np.array_equal(masks.cpu().numpy().view(np.uint64), ref_masks):
        raise SystemExit("masks differ from the oracle")
    R = N * H
    rows = np.unique(np.concatenate([b * R + np.array([0, R - 1]) for b in range(B)] +
                                    [rng.integers(0, B * R, size=64)]))
    ref_out = oracle.run(inp, rows=rows)[1].reshape(-1, dc)
    err = float(np.abs(out.reshape(-1, dc)[torch.from_numpy(rows).to(dev)].cpu().double().numpy() - ref_out).max())
    tol = 2e-3 if sp.dtype == "bf16" else 1e-5
    if err > tol:
        raise SystemExit(f"attention max-abs error {err} above {tol}")
    w_path, w_acc, w_bonus = oracle_accept.tree_accept(par_ref, tok_ref, nxt, root)
    if not (np.array_equal(path.cpu().numpy(), w_path) and np.array_equal(acc.cpu().numpy(), w_acc)
            and np.array_equal(bonus.cpu().numpy(), w_bonus)):
        raise SystemExit("accept differs from the oracle")
    as_i16 = (lambda t: t.view(torch.int16).numpy()) if sp.dtype == "bf16" else (lambda t: t.view(torch.int32).numpy())
    wc, wr, wl = oracle_accept.kv_compact(as_i16(inp.kv_cache[:, :dc]), as_i16(inp.kv_cache[:, dc:]),
                                          inp.cache_lens.numpy().astype(np.int64), as_i16(inp.tree_kv[:, :, :dc]),
                                          as_i16(inp.tree_kv[:, :, dc:]), w_path.astype(np.int64),
                                          w_acc.astype(np.int64))
    n_new = int(wl.sum())
    got = kv_out[:n_new].cpu()
    if not (np.array_equal(as_i16(got[:, :dc]), wc) and np.array_equal(as_i16(got[:, dc:]), wr)
            and np.array_equal(new_lens.cpu().numpy(), wl)):
        raise SystemExit("compaction differs from the oracle")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    he = HipEvents()
    evs = [[he.create() for _ in range(7)] for _ in range(args.steps)]
    ev0, ev1 = he.create(), he.create()
    he.record(ev0, stream)
    for i in range(args.steps):
        step(lambda k, i=i: he.record(evs[i][k], stream))
    he.record(ev1, stream)
    torch.cuda.synchronize()
    step_ms = he.elapsed_ms(ev0, ev1) / args.steps
    names = ["tree_build", "prepare", "attend", "combine", "accept", "compact"]
    stage = {n: float(np.mean([he.elapsed_ms(e[k], e[k + 1]) for e in evs])) for k, n in enumerate(names)}
    he.close()
    flops, nbytes, cache_bytes = algorithmic_work(inp)
    mfma_peak = PEAK_BF16_TFLOPS if sp.dtype == "bf16" else PEAK_F32_TFLOPS
    if flops / nbytes < mfma_peak * 1e12 / (PEAK_HBM_GBPS * 1e9):
        bound, peak, unit_r, achieved = "hbm", PEAK_HBM_GBPS, "GB/s", nbytes / (stage["attend"] * 1e-3) / 1e9
    else:
        bound, peak, unit_r, achieved = "mfma", mfma_peak, "TFLOP/s", flops / (stage["attend"] * 1e-3) / 1e12
    line = {
        "metric": "DDTree verify step (tree build, masks + plan, attention, combine, accept, compaction) requests/s",
        "value": round(B / (step_ms * 1e-3), 3), "unit": "requests/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sp.dtype,
        "data": "synthetic (seeded drafter log probabilities, N(0,1) queries and cache, guided target predictions)",
        "config": {"workload": f"step on {sp.name}: B={B} requests, N={N} nodes (depth<={D}, top-{K}), H={H} heads, "
                               f"cache={maxL} tokens, {sp.dtype}", "batch": B, "nodes": N, "heads": H,
                   "cache_len": maxL, "splits": kdt.num_splits(desc),
                   "compaction": "in place" if in_place else "into a second buffer"},
        "stage_us": {n: round(v * 1e3, 2) for n, v in stage.items()},
        "attend_stage": "masks + plan + attention (prepare_us is 0)" if one_launch else "attention",
        "accepted_tokens": int(w_acc.sum()), "attention_max_abs_err_sampled": err,
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit_r,
                     "frac": round(achieved / peak, 4), "traffic": None},
    }
    if not getattr(args, "no_cpu_baseline", True):
        # the oracle chain on the host cores: tree, masks + attention rows, accept, compaction.
        # Steps above ~40 GFLOP run the attention on a random sample of rows and scale it to
        # every row (the oracle's cost is linear in the rows).
        cores = len(os.sched_getaffinity(0))
        oracle.build()
        total_rows = B * R
        sample = total_rows if flops <= 40e9 else max(64, int(total_rows * 40e9 / flops))
        srows = None if sample == total_rows else np.sort(rng.choice(total_rows, size=sample, replace=False))
        reps, t_attn, t_rest = 0, 0.0, 0.0
        t0 = time.perf_counter()
        while True:
            a = time.perf_counter()
            p_ref = oracle_tree.best_first_tree(lp, cand, N)[0]
            b_ = time.perf_counter()
            oracle.run(dataclasses.replace(inp, parents=torch.from_numpy(p_ref)), rows=srows, threads=cores)
            c = time.perf_counter()
            a_path, a_acc, _ = oracle_accept.tree_accept(p_ref, tok_ref, nxt, root)
            oracle_accept.kv_compact(as_i16(inp.kv_cache[:, :dc]), as_i16(inp.kv_cache[:, dc:]),
                                     inp.cache_lens.numpy().astype(np.int64), as_i16(inp.tree_kv[:, :, :dc]),
                                     as_i16(inp.tree_kv[:, :, dc:]), a_path.astype(np.int64), a_acc.astype(np.int64))
            d_ = time.perf_counter()
            t_attn += c - b_
            t_rest += (b_ - a) + (d_ - c)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or dt * (reps + 1) / reps > 30.0:
                break
        step_s = (t_rest + t_attn * total_rows / sample) / reps
        line["cpu_baseline"] = {
            "value": round(B / step_s, 3), "unit": "requests/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} step(s) of the same workload in {dt:.2f} s: tree, masks, "
                      + (f"all {total_rows} attention rows" if srows is None else
                         f"{sample} of {total_rows} attention rows (scaled to all)")
                      + f" in fp64 on {cores} threads, accept, compaction"}
    return line


# HBM traffic of the attention kernel per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# summarised under profiles/.  The summary records a hash of the code the kernel is built from;
# when that code has changed since, the figure no longer describes this kernel and `traffic` is
# reported as null.  The hash covers each kernel's own sources, the C-ABI layer that sets its
# launch geometry (split policy, tile sizes, workspace layout) and the public header, and the
# compiler flags of the build.
_ABI = ["tree_verify_mla_02_amd/csrc/api.cpp", "include/kdt.h", "tree_verify_mla_02_amd/csrc/kdt_internal.h"]
KERNEL_SOURCES = {
    "verify_attn": ["tree_verify_mla_02_amd/csrc/verify_attn.hip",
                    "tree_verify_mla_02_amd/csrc/visibility_rows.h"] + _ABI,
    "kv_compact": ["tree_verify_mla_02_amd/csrc/accept.hip"] + _ABI,
    "tree_accept": ["tree_verify_mla_02_amd/csrc/accept.hip"] + _ABI,
    "tree_build": ["tree_verify_mla_02_amd/csrc/tree_build.hip"] + _ABI,
}


def kernel_source_hash(kernel: str = "verify_attn") -> str:
    """Hash of the code a kernel is compiled from (its sources with comments, blank lines and
    trailing blanks removed, so that an edit of a comment leaves it unchanged) and of the build
    flags."""
    import hashlib
    import re

    from tree_verify_mla_02_amd import build as kbuild
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        code = "\n".join(ln for ln in lines if ln.strip())
        h.update(name.encode() + b"\0" + code.encode())
    h.update(b"flags\0" + " ".join(kbuild.FLAGS).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str = "verify_attn"):
    """HBM bytes per launch from profiles/<kernel>_<workload>_hbm_traffic.md, or None when
    there is no summary or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--attn-event-every", type=int, default=5,
                    help="bracket the attention launch of every E-th timed step with events (1: every step)")
    ap.add_argument("--workload", default="kimi", choices=sorted(workloads.SPECS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--staged", action="store_true",
                    help="time prepare, attend and combine as three launches also where one launch makes the "
                         "masks, the plan and the attention")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="attention launches timed after flushing L2 and MALL (0 to skip)")
    ap.add_argument("--row", default="verify", choices=["verify", "accept", "compact", "tree", "step"],
                    help="verify: the tree-verify attention step (default); accept / compact / tree: the greedy "
                         "tree-accept, the KV compaction or the best-first tree builder kernel alone, on the "
                         "workload's trees and lengths; step: a whole verify step, all of them chained")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.attn_event_every < 1:
        ap.error("--steps and --attn-event-every must be >= 1 and --warmup >= 0")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X with no sharding "
              "(the design notes describe how it would shard); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_direction": n, "launches": args.steps}), flush=True)
        return
    if args.row == "tree":
        print(json.dumps(run_tree_row(args)), flush=True)
        return
    if args.row == "step":
        print(json.dumps(run_step_row(args)), flush=True)
        return
    if args.row != "verify":
        print(json.dumps(run_next_row(args)), flush=True)
        return
    line, inp = run(args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
