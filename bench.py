"""Benchmark: KPage block-sparse attention forward + backward on one MI355X.

One step is the whole hot path on one batch: kpage_attn_fwd then kpage_attn_bwd on
the 3D-padded video layout (21 x 30 x 52 tokens in 4 x 4 x 8 tiles -> 336 blocks of
128 rows, 43008 physical rows, 40 heads, d = 128, bf16; window (1,2,2) plus 4 random
blocks per query block; --workload 4 / 5 time the 21 x 45 x 80 top-87 and the
independent-partition workloads instead).
Planning (page tables, routes, owners) is built once before the timed region and reused,
as the method intends.

Reported value: useful TFLOP/s of the step = 14 * d * (valid query-key pairs) / time
(2 forward GEMMs + 5 backward GEMMs per valid pair), with the step time the median of
the timed steps (mean, minimum and maximum beside it); the forward alone is reported
beside it with 4 * d * pairs.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0
METRIC = "useful TFLOP/s (4·d·valid pairs) fwd & fwd+bwd; % bf16 MFMA peak"
WORKLOAD = 3  # the 3D-padded fwd + fwd+bwd configuration the metric's target is stated for
# the fwd+bwd configurations bench.py can time (--workload); the default is the metric's
WORKLOADS = {
    1: ("tiny 3d layout 5x6x10 (4x4x8 tiles, 8 blocks, 1024 rows), 2 heads, d=64, diagonal + "
        "Bernoulli(0.5) blocks, fwd+bwd", 5 * 6 * 10, (0, 1)),
    2: ("padding-free 16x32x32 (4x4x8 tiles, 128 full blocks, 16384 rows), 24 heads, d=128, "
        "window (1,1,1), fwd+bwd", 16 * 32 * 32, (0,)),
    3: ("3d-padded 21x30x52 (4x4x8 tiles, 336 blocks, 43008 rows), 40 heads, d=128, "
        "window (1,2,2) + 4 random blocks, fwd+bwd", 21 * 30 * 52, (0, 1)),
    4: ("vsa-style 21x45x80 (4x4x8 tiles, 720 blocks, 92160 rows), 40 heads, d=128, "
        "per-head top-87 blocks by mean-pooled q.k, fwd+bwd", 21 * 45 * 80, (0,)),
    5: ("svg2-style independent partitions of 75600 tokens (k-means 200 Q / 600 K clusters, top-p 0.9), "
        "40 heads, d=128, fwd+bwd", 21 * 45 * 80, (0,)),
}


def _device_plan_ms(K, problem, reps=3):
    """Host wall time of kpage_plan_device on a selected graph, synchronised: one untimed
    call first (first-use allocations), then the median of `reps` calls."""
    import torch
    K.kpage_plan_device(problem).close()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        plan = K.kpage_plan_device(problem)
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
        plan.close()
    return sorted(times)[len(times) // 2]


def _prelude(K, w, q, k, top_k=87, reps=5):
    """GPU block selection (mean pooling + top-k) on the workload's own layout, then the GPU
    planner on its graph: the selector and planner a dynamic-sparsity step would run before
    attention.  Timed with events on torch's current stream, which the calls launch on."""
    import torch
    dev = q.device
    qv = torch.as_tensor(w.q_valid[0], device=dev)
    kvv = torch.as_tensor(w.kv_valid[0], device=dev)
    ko = torch.as_tensor(w.kv_offset[0], device=dev)
    ws = torch.empty(K.kpage_select_workspace_size(q, k, qv, kvv, ko), dtype=torch.uint8, device=dev)
    ptr, idx = K.select_topk(q, k, qv, kvv, ko, top_k, workspace=ws)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ptr, idx = K.select_topk(q, k, qv, kvv, ko, top_k, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    sel_ms = e0.elapsed_time(e1) / reps
    plan_ms = _device_plan_ms(K, K.SelectedProblem(q, k, qv, kvv, ko, ptr, idx))
    BH = w.batch * w.heads
    rows_q, rows_k = int(w.q_valid[0].sum()), int(w.kv_valid[0].sum())
    # algorithmic bytes: the valid rows of Q and K read once, the graph written once
    nbytes = BH * (rows_q + rows_k) * w.head_dim * 2 + BH * (w.n_q * top_k * 4 + (w.n_q + 1) * 8)
    gbs = nbytes / (sel_ms * 1e-3) / 1e9
    return {"select_ms": round(sel_ms, 4), "plan_device_ms_median_incl_sync": round(plan_ms, 2), "top_k": top_k,
            "roofline": {"kernel": "kpage_select_topk (all kernels of one call)", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4),
                         "algorithmic": "Q and K valid rows read once + CSR graph written"}}


def _prelude_top_p(K, w, top_p=0.9, reps=5):
    """GPU cluster top-p selection (SVG2-style) from the workload's own clustering, then the
    GPU planner on its graph.  Timed with events on torch's current stream."""
    import numpy as np
    import torch
    dev = torch.device("cuda", 0)
    st = lambda key, dt: torch.as_tensor(np.stack([c[key] for c in w.clusters]), device=dev).to(dt).contiguous()
    args = [st("q_cent", torch.float32), st("k_cent", torch.float32), st("q_size", torch.int32),
            st("k_size", torch.int32), st("q_block_cluster", torch.int32), st("k_block_cluster", torch.int32)]
    scale = 1.0 / np.sqrt(w.head_dim)
    ptr, idx = K.select_top_p(w.batch, w.heads, *args, top_p=top_p, scale=scale)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ptr, idx = K.select_top_p(w.batch, w.heads, *args, top_p=top_p, scale=scale)
    e1.record()
    torch.cuda.synchronize()
    sel_ms = e0.elapsed_time(e1) / reps
    p = type("SelectedGraph", (), {})()
    for a in ("batch", "heads", "head_dim", "n_q", "n_kv", "seq_q", "seq_kv", "per_head", "q_valid", "kv_valid",
              "kv_offset"):
        setattr(p, a, getattr(w, a))
    p.q2k_ptr, p.q2k_idx = ptr, idx
    plan_ms = _device_plan_ms(K, p)
    return {"select_top_p_ms": round(sel_ms, 4), "plan_device_ms_median_incl_sync": round(plan_ms, 2), "top_p": top_p,
            "clusters": [int(args[0].shape[1]), int(args[1].shape[1])]}


def _cpu_baseline(workload, heads, runs=3):
    """The fp64 CPU oracle on a bounded sample: forward + backward of a few heads, the
    median wall time of `runs` runs."""
    from threadpoolctl import threadpool_info

    from oracle import oracle_bwd, oracle_plan
    from workloads import make_workload

    w = make_workload(workload, heads=list(heads), with_do=True)
    pairs = oracle_plan(w).stats["useful"]  # pair count of the sample, from the oracle planner
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle_bwd(w, w.q, w.k, w.v, w.do)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": round(14 * w.head_dim * pairs / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"oracle forward+backward (fp64 numpy) of {len(heads)} of the heads of the same workload, "
                  f"median of {runs} runs = {dt:.1f} s wall (runs {', '.join(f'{t:.1f}' for t in times)} s), "
                  f"scaled per valid pair",
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bwd_3d_padded_h40.json")


def _measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE counter
    summary (already scaled by the copy calibration), or None when the counters were taken
    on another workload or when the kernel's sources, or the host planner and launch-list
    code that decide its work, changed since they were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            full = json.load(f)
        rec = full["kernels"][kernel]
        if int(full["workload_id"]) != workload:
            return None
    except (OSError, KeyError, ValueError, TypeError):
        return None
    h = hashlib.sha256()
    for name in rec["sources"]:
        with open(os.path.join(ROOT, "block_sparse_attention_11_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return rec["bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def _route_pairs(w, K=None, plan=None):
    """Useful pairs of the work items of the M128 x N128 and M64 x N256 launches: blocks with
    c_q > 64 and the members of group items (up to four blocks of <= 32 rows run as one M128
    item), and the other blocks with 1 <= c_q <= 64."""
    import numpy as np
    BH = w.batch * w.heads
    slots = range(BH) if w.per_head else [0]
    grouped = set()
    if plan is not None:
        gptr = K.kpage_plan_export(plan, "group_ptr")
        mem = K.kpage_plan_export(plan, "group_members").reshape(-1, 4)
        for g in slots:
            for i in range(int(gptr[g]), int(gptr[g + 1])):
                grouped.update((g, int(q)) for q in mem[i] if q >= 0)
    out = {"q128": 0, "q64": 0}
    for g in slots:
        for q in range(w.n_q):
            cq = int(w.q_valid[g, q])
            if cq == 0:
                continue
            ks = w.q2k_idx[w.q2k_ptr[g, q]:w.q2k_ptr[g, q + 1]]
            pairs = cq * int(np.asarray(w.kv_valid[g])[ks].sum())
            out["q128" if cq > 64 or (g, q) in grouped else "q64"] += pairs
    if not w.per_head:
        out = {k: v * BH for k, v in out.items()}
    return out


def _route_split(K, plan, step, w, steps=5):
    """Forward and dQ launches split by route (timing mode 2), after the timed region: per-route
    time and useful TFLOP/s (4 d per pair for the forward, 6 d for the dQ pass); group items
    count with the M128 x N128 route, whose launch runs them."""
    K.kpage_timing_enable(plan, 2)
    for _ in range(steps):
        step()
    kern = {n: K.kpage_timing_read(plan, n) for n in K.KERNELS}
    K.kpage_timing_enable(plan, False)
    pairs = _route_pairs(w, K, plan)
    d = w.head_dim
    out = {}
    for name, key, route, per in (("fwd_q128", "fwd", "q128", 4), ("fwd_q64", "fwd_q64", "q64", 4),
                                  ("dq_q128", "bwd_dq", "q128", 6), ("dq_q64", "bwd_dq_q64", "q64", 6)):
        ms = kern[key][0] / max(kern[key][1], 1)
        out[name] = {"ms": round(ms, 4), "useful_pairs": pairs[route],
                     "useful_tflops": round(per * d * pairs[route] / (ms * 1e-3) / 1e12, 1) if ms > 0 else None}
    return out


def _copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reads": n, "writes": n}), flush=True)


def _dense_reference():
    """Context for the roofline fraction: what this GPU sustains on dense bf16 MFMA work
    with random data, through the vendor libraries behind PyTorch (hipBLASLt GEMMs and
    the flash-attention backend of scaled_dot_product_attention, forced so that no math
    fallback runs).  The kernels of this package are not involved."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    def timed(fn, iters, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    torch.manual_seed(0)
    out = {"peak_bf16_tflops": PEAK_BF16_TFLOPS}
    for n in (8192, 16384):
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        ms = timed(lambda: torch.matmul(a, b), 20, 5)
        out[f"gemm_bf16_{n}^3"] = {"ms": round(ms, 4), "tflops": round(2 * n ** 3 / ms / 1e9, 1)}
        del a, b
    h, s, d = 40, 16384, 128
    q, k, v, do = (torch.randn(1, h, s, d, device="cuda", dtype=torch.bfloat16) for _ in range(4))
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
        ms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v), 10, 3)
        out["flash_attention_fwd"] = {"shape": [1, h, s, d], "ms": round(ms, 4),
                                      "tflops": round(4 * s * s * d * h / ms / 1e9, 1)}
        qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))

        def fwd_bwd():
            torch.nn.functional.scaled_dot_product_attention(qg, kg, vg).backward(do)

        ms = timed(fwd_bwd, 5, 2)
        out["flash_attention_fwd_bwd"] = {"shape": [1, h, s, d], "ms": round(ms, 4),
                                          "tflops": round(14 * s * s * d * h / ms / 1e9, 1)}
    print(json.dumps({"dense_reference": out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-route-split", action="store_true",
                    help="skip the extra steps that time the forward and dQ launches per route (profiling runs)")
    ap.add_argument("--workload", type=int, default=WORKLOAD, choices=sorted(WORKLOADS),
                    help="configuration to time (default: the metric's 3D-padded fwd+bwd workload)")
    ap.add_argument("--q-group", type=int, default=0, metavar="N",
                    help="backward Q-group size in Q blocks (0: one group, the default)")
    ap.add_argument("--heads", type=int, default=0, metavar="N",
                    help="time only the first N heads of the workload (one GPU's share when the heads are "
                         "sharded over several GPUs; 0: all heads, the default)")
    ap.add_argument("--no-groups", action="store_true",
                    help="plan every query block as its own work item (no group items of small blocks)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the known-size kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--dense-reference", action="store_true",
                    help="only time dense bf16 GEMMs and dense flash attention through PyTorch's vendor "
                         "libraries (what this GPU sustains on dense MFMA work) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        _copy_calibration(args.copy_calibration)
        return
    if args.dense_reference:
        _dense_reference()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the attention shards by head with no exchange between GPUs, and this benchmark times one GPU's share.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_11_amd as K
    from workloads import make_workload

    dev = torch.device("cuda", 0)
    desc, tokens, cpu_heads = WORKLOADS[args.workload]
    w = make_workload(args.workload, heads=list(range(args.heads)) if args.heads > 0 else None, with_do=True)
    if args.heads > 0:
        desc += f"; first {w.heads} heads only"
    d = w.head_dim
    t0 = time.perf_counter()
    plan = K.kpage_plan(w, q_group=args.q_group, grouped=not args.no_groups)
    plan_ms = (time.perf_counter() - t0) * 1e3
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(K.kpage_bwd_workspace_size(plan), dtype=torch.uint8, device=dev)
    t0 = time.perf_counter()
    K.kpage_plan_upload(plan)
    K.kpage_attn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, ws, w.scale)  # builds the lazy backward plan
    torch.cuda.synchronize()
    bwd_plan_ms = (time.perf_counter() - t0) * 1e3
    stats = K.kpage_plan_stats(plan)
    # work items that run up to four small query blocks together (one per graph slot's group
    # and (batch, head) of the slot)
    n_groups = K.kpage_plan_export(plan, "group_members").size // 4
    n_group_items = n_groups if w.per_head else n_groups * w.batch * w.heads
    # the same plan built on the GPU (identical tables; the timed steps use the host-built one)
    K.kpage_plan_device(w).close()  # first use: kernel and allocator warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dplan = K.kpage_plan_device(w)
    dev_plan_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    K.kpage_attn_bwd(dplan, q, k, v, o, lse, do, dq, dk, dv, ws, w.scale)
    torch.cuda.synchronize()
    dev_bwd_plan_ms = (time.perf_counter() - t0) * 1e3
    dplan.close()

    def step():
        K.kpage_attn_fwd(plan, q, k, v, o, lse, w.scale)
        K.kpage_attn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, ws, w.scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K.kpage_timing_enable(plan, True)
    for name in K.KERNELS:
        K.kpage_timing_read(plan, name)
    # one event between consecutive steps on the stream the calls launch on: per-step times
    # whose median is the reported step time (the pages time the median of repeated runs)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    events[0].record()
    for i in range(args.steps):
        step()
        events[i + 1].record()
    torch.cuda.synchronize()
    step_ms = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    total_ms = events[0].elapsed_time(events[-1])
    kern = {name: K.kpage_timing_read(plan, name) for name in K.KERNELS}
    K.kpage_timing_enable(plan, False)
    ms_step = sorted(step_ms)[len(step_ms) // 2] if len(step_ms) % 2 else \
        0.5 * sum(sorted(step_ms)[len(step_ms) // 2 - 1:len(step_ms) // 2 + 1])
    ms_mean = total_ms / args.steps
    pairs = stats["useful"]
    fwd_ms = sum(kern[n][0] for n in ("fwd", "fwd_exact")) / args.steps
    bwd_ms = sum(kern[n][0] for n in ("bwd_pre", "bwd_zero", "bwd_kv", "bwd_reduce", "bwd_dq")) / args.steps
    value = 14 * d * pairs / (ms_step * 1e-3) / 1e12
    fwd_tflops = 4 * d * pairs / (fwd_ms * 1e-3) / 1e12

    # dominant kernel of the step, with its own algorithmic flops per launch over the useful pairs:
    # K/V-owned pass 4 GEMMs (S, dP, dV, dK) = 8 d; Q-owned dQ pass 3 GEMMs (S, dP, dQ) = 6 d;
    # forward (both routes) 2 GEMMs = 4 d
    cands = {"kpage_bwd_kv": (8, kern["bwd_kv"]), "kpage_bwd_dq": (6, kern["bwd_dq"]),
             "kpage_fwd": (4, (sum(kern[n][0] for n in ("fwd", "fwd_exact")), kern["fwd"][1]))}
    dom = max(cands, key=lambda n: cands[n][1][0])
    per_pair, (dom_ms, dom_n) = cands[dom]
    dom_avg = dom_ms / max(dom_n, 1)
    achieved = per_pair * d * pairs / (dom_avg * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": _measured_traffic(dom, args.workload), "traffic_unit": "HBM bytes per launch (counters)", "avg_ms": round(dom_avg, 4), "launches": dom_n,
                "algorithmic": f"{per_pair}*d*useful_pairs per launch"}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_statistic": "median of the timed steps",
        "ms_per_step_mean": round(ms_mean, 4),
        "ms_per_step_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc + (f", backward Q groups of {args.q_group} blocks" if args.q_group else "")
                   + (", no group items" if args.no_groups else ""),
                   "batch": 1, "heads": w.heads, "head_dim": d, "tokens": tokens,
                   "seq_physical": w.seq_q},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 4), "useful_tflops": round(fwd_tflops, 2),
                "pct_bf16_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2)},
        "bwd_ms": round(bwd_ms, 4),
        "kernel_ms_per_step": {n: round(kern[n][0] / args.steps, 4) for n in K.KERNELS},
        "pairs": {kk: stats[kk] for kk in ("useful", "whole_block", "paged_m128", "nominal", "scheduled",
                                             "bwd_physical")},
        "plan_ms": {"forward": round(plan_ms, 2), "backward_lazy_incl_first_call": round(bwd_plan_ms, 2),
                    "device_forward_incl_descriptor_upload": round(dev_plan_ms, 2),
                    "device_backward_lazy_incl_first_call": round(dev_bwd_plan_ms, 2)},
        "roofline": roofline,
        "group_items": n_group_items,
    }
    if not args.no_route_split:
        out["routes"] = _route_split(K, plan, step, w)
    if args.workload == 4:
        out["prelude"] = _prelude(K, w, q, k)
    if args.workload == 5:
        out["prelude"] = _prelude_top_p(K, w)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(args.workload, cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
