"""Benchmark of prefix-shared tree decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

One step = one pass of the hot path over the workload: the partial-attention
kernel (PAC) then the partial-output reduction (POR), with the tree index and
the plan built before the timed region and reused (plans are reused across
decode steps and layers).  Before every step a 1 GiB read of a buffer that is
never written evicts L2 and the last-level cache without leaving dirty lines
behind, so every step reads its KV from HBM and pays for no write-back of
the eviction.  A step is timed as one ``pst_decode_attn`` call (the library
enqueues PAC and POR back to back) between two HIP events recorded on the
stream it runs on; a second pass puts an event between the two kernels for
the per-kernel split (``pac_ms``, ``por_ms``; the roofline uses ``pac_ms``).
The output is in the input dtype, the library's default.  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Dense matrix-core peaks (no sparsity): bf16 2.5 PFLOP/s; float32 inputs run
# on the vector ALU (157.3 TFLOP/s).
COMPUTE_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
METRIC = "logical KV tokens attended/s and unique-KV HBM GB/s (% of MI355X peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: PAC settles after 30-40 cold steps (about 9 %% faster than the first "
                         "ones on the document-QA tree), which a decode loop reaches within its first milliseconds")
    ap.add_argument("--config", default="5-mha",
                    help="workload (default: the largest one that fits one GPU, the skewed MHA tree with ~38 GB "
                         "of K/V)")
    ap.add_argument("--no-gate", action="store_true",
                    help="skip the per-workload PAC + POR measurement of the document-QA, few-shot and "
                         "speculative trees that follows the main line")
    ap.add_argument("--gate-warmup", type=int, default=50,
                    help="untimed cold steps per workload of the gate measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baseline", action="store_true", help="skip the query-guided comparison")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm-cache timing (every PAC launch of the run is then cold, as under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="> 0: time a decode loop of this many steps (one token appended to every query's leaf per "
                         "step, paged pool) with the plan reused, re-planned every 16 steps and every step")
    ap.add_argument("--sweep", action="store_true",
                    help="tree-shape sweep (2T..5T k-ary trees and a degenerate tree; CoDec's shapes): tree path, "
                         "tree path without splitting, and the query-guided baseline per shape")
    ap.add_argument("--flatten-sweep", action="store_true",
                    help="partition comparison (DEFT-Node, DEFT-Node-Chunk and DEFT-Flatten at several chunk "
                         "lengths against the cost-model plan) on the large workloads and two tree shapes")
    ap.add_argument("--flatten", type=int, default=0,
                    help="> 0: time the DEFT-Flatten partition with chunks of this many tokens instead of the "
                         "cost-model plan")
    ap.add_argument("--page-size", type=int, default=0,
                    help="> 0: K/V in a paged pool of pages of this many tokens (scattered, with holes)")
    ap.add_argument("--page-order", choices=["scattered", "sequential"], default="scattered",
                    help="paged pool: pages drawn at random from a pool one eighth larger (scattered), or "
                         "numbered in order without holes (sequential)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "pac_traffic.json"),
                    help="rocprofv3 counter summary giving the PAC kernel's HBM bytes")
    return ap.parse_args()


def workload_stats(spec, tree):
    ix = tree.index()
    eb = 4 if spec.dtype == "f32" else 2
    tok_bytes = 2 * spec.num_kv_heads * spec.head_dim * eb
    live = ix["n_q"] > 0
    unique_tokens = int(spec.kv_len[live].astype("int64").sum())
    logical = int(ix["visible"].sum())
    per_query_tokens = int((ix["n_q"].astype("int64") * spec.kv_len).sum())
    return {
        "unique_kv_tokens": unique_tokens,
        "unique_kv_bytes": unique_tokens * tok_bytes,
        "logical_tokens": logical,
        "per_query_kv_bytes": per_query_tokens * tok_bytes,
        "flops": 4 * spec.head_dim * spec.num_q_heads * logical,
    }


def evict(pst, bufs):
    """Read 1 GiB that nothing writes: caches end up holding clean, unrelated lines."""
    pst.bench_read(bufs[0], bufs[1])


def time_steps(torch, pst, plan, q, k, v, out, lse, ws, evict_bufs, steps, warmup):
    """Cold steps on the current stream.  Pass 1: one ``pst_decode_attn``
    call (PAC then POR, enqueued back to back by the library) between two
    events: the step time.  Pass 2: events before PAC, between PAC and POR
    and after POR: the per-kernel split (each event on the stream adds a few
    microseconds, so the split sums to more than the step)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        evict(pst, evict_bufs)
        pst.decode_attn(plan, q, k, v, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evict(pst, evict_bufs)
        ev[i][0].record(stream)
        pst.decode_attn(plan, q, k, v, out=out, lse=lse, ws=ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [e[0].elapsed_time(e[1]) for e in ev]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        evict(pst, evict_bufs)
        ev[i][0].record(stream)
        pst.pac(plan, q, k, v, ws)
        ev[i][1].record(stream)
        pst.por(plan, out, lse, ws)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    pac_ms = [e[0].elapsed_time(e[1]) for e in ev]
    por_ms = [e[1].elapsed_time(e[2]) for e in ev]
    return step_ms, pac_ms, por_ms, wall


def time_warm(torch, pst, plan, q, k, v, out, lse, ws, steps):
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pst.decode_attn(plan, q, k, v, out=out, lse=lse, ws=ws)
    a.record(stream)
    for _ in range(steps):
        pst.decode_attn(plan, q, k, v, out=out, lse=lse, ws=ws)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def cpu_baseline(spec, q, k, v, out, budget_s):
    """The oracle as it stands, on a bounded sample of the workload's queries."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    order = np.random.default_rng(0).permutation(spec.num_queries)
    done, tokens, err = [], 0, 0.0
    t0 = time.perf_counter()
    for r in order:
        # The oracle gathers each query's path K/V from the device pools
        # itself (tens of GB never go to the host whole).
        O, _ = oracle.attend(spec, q, k, v, queries=[int(r)])
        tokens += len(oracle.visible_tokens(spec, int(r)))
        err = max(err, float(abs(out[int(r)].double().cpu().numpy() - O[0]).max()))
        done.append(int(r))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": tokens / dt, "unit": "logical KV tokens/s", "cores": threads, "kind": "oracle",
        "sample": f"{len(done)} of {spec.num_queries} queries (all heads, in a seeded random order), {tokens} "
                  f"logical tokens, {dt:.1f} s including the gather of each query's path K/V from device memory, "
                  f"float64 numpy on {os.cpu_count()} host CPUs ({model})",
        "parity_max_abs_on_sample": err,
    }


def shape_sweep(torch, pst, workloads, a):
    """CoDec's tree shapes (binary .. 5-ary trees, a degenerate tree), 4096
    tokens per query path, half of them in the shared root, GQA 32/8, d 128,
    bf16.  Per shape, cold-cache PAC + POR of: the tree path; the tree path
    with every node one piece (no workload partitioning); the query-guided
    (FlashDecoding-style) baseline, which reads shared KV once per query."""
    shapes = [workloads.kary_tree(2, 7), workloads.kary_tree(3, 5), workloads.kary_tree(4, 4),
              workloads.kary_tree(5, 4), workloads.degenerate_tree(64)]
    evict_bufs = (torch.empty(1 << 30, dtype=torch.uint8, device="cuda"),
                  torch.empty(4096, dtype=torch.float32, device="cuda"))
    rows = {}
    for spec in shapes:
        print(f"[bench] shape {spec.name}", file=sys.stderr, flush=True)
        q, k, v = workloads.make_tensors(spec, "cuda")
        tree = pst.Tree.from_spec(spec)
        st = workload_stats(spec, tree)
        out = torch.empty((spec.num_queries, spec.num_q_heads, spec.head_dim), device="cuda", dtype=q.dtype)
        lse = torch.empty((spec.num_queries, spec.num_q_heads), device="cuda", dtype=torch.float32)
        r = {"nodes": spec.num_nodes, "queries": spec.num_queries, "unique_kv_bytes": st["unique_kv_bytes"],
             "per_query_kv_bytes": st["per_query_kv_bytes"],
             "kv_read_ratio": st["per_query_kv_bytes"] / st["unique_kv_bytes"]}
        for name, kw in (("tree", {}), ("tree_no_split", {"no_split": True}), ("query_guided", {"query_guided": True})):
            plan = pst.Plan(tree, **kw)
            ws = pst.workspace(plan)
            steps, _, _, _ = time_steps(torch, pst, plan, q, k, v, out, lse, ws, evict_bufs, a.steps, a.warmup)
            r[name + "_ms"] = statistics.mean(steps)
            del ws, plan
        r["speedup_over_query_guided"] = r["query_guided_ms"] / r["tree_ms"]
        r["speedup_of_partitioning"] = r["tree_no_split_ms"] / r["tree_ms"]
        r["unique_kv_frac_of_peak"] = st["unique_kv_bytes"] / (r["tree_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        rows[spec.name] = r
        del q, k, v, tree
    print(json.dumps({
        "metric": "tree-shape sweep: PAC + POR ms per shape, tree path vs query-guided baseline",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic", "config": {"mode": "shape_sweep", "path_len": 4096, "shared_root": 0.5,
                                         "heads": "32/8", "head_dim": 128},
        "shapes": rows,
    }))


def flatten_sweep(torch, pst, workloads, a):
    """Partitions of the same tree (DEFT Table 6 and CoDec Fig. 10 analogs),
    cold-cache PAC + POR each: one piece per node (DEFT-Node), nodes cut
    into chunks of S_t tokens (DEFT-Node-Chunk), the depth-first flattening
    cut into chunks of S_t tokens with bit causal masks (DEFT-Flatten), and
    the cost-model plan."""
    chunks = (128, 256, 512, 1024)
    specs = [workloads.config("2"), workloads.config("3"), workloads.config("4"), workloads.config("5-mqa"),
             workloads.kary_tree(2, 7), workloads.degenerate_tree(64)]
    evict_bufs = (torch.empty(1 << 30, dtype=torch.uint8, device="cuda"),
                  torch.empty(4096, dtype=torch.float32, device="cuda"))
    rows = {}
    for spec in specs:
        print(f"[bench] partitions of {spec.name}", file=sys.stderr, flush=True)
        q, k, v = workloads.make_tensors(spec, "cuda")
        tree = pst.Tree.from_spec(spec)
        st = workload_stats(spec, tree)
        out = torch.empty((spec.num_queries, spec.num_q_heads, spec.head_dim), device="cuda", dtype=q.dtype)
        lse = torch.empty((spec.num_queries, spec.num_q_heads), device="cuda", dtype=torch.float32)
        variants = [("cost_model", {}), ("node", {"no_split": True})]
        variants += [(f"node_chunk_{c}", {"fixed_chunk": c}) for c in chunks]
        variants += [(f"flatten_{c}", {"flatten": c}) for c in chunks]
        r = {"queries": spec.num_queries, "nodes": spec.num_nodes, "unique_kv_bytes": st["unique_kv_bytes"]}
        # An untimed pass first (as many cold steps as each variant's
        # warm-up): the first variant timed after the inputs were made
        # otherwise reads up to 20 % slow.
        plan = pst.Plan(tree)
        ws = pst.workspace(plan)
        time_steps(torch, pst, plan, q, k, v, out, lse, ws, evict_bufs, 3, a.warmup)
        del ws, plan
        for name, kw in variants:
            plan = pst.Plan(tree, **kw)
            ws = pst.workspace(plan)
            steps, _, _, _ = time_steps(torch, pst, plan, q, k, v, out, lse, ws, evict_bufs, a.steps, a.warmup)
            r[name + "_ms"] = statistics.mean(steps)
            r[name + "_tasks"] = int(len(plan.view()["tasks"]))
            del ws, plan
        best = min((c for c in chunks), key=lambda c: r[f"flatten_{c}_ms"])
        r["flatten_best_chunk"] = best
        r["cost_model_over_best_flatten"] = r[f"flatten_{best}_ms"] / r["cost_model_ms"]
        r["unique_kv_frac_of_peak"] = st["unique_kv_bytes"] / (r["cost_model_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        rows[spec.name] = r
        del q, k, v, tree
    print(json.dumps({
        "metric": "partition comparison: PAC + POR ms per workload (DEFT-Node, -Node-Chunk, -Flatten, cost model)",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic", "config": {"mode": "flatten_sweep", "chunks": list(chunks)},
        "workloads": rows,
    }))


def decode_loop_bench(torch, pst, workloads, spec, a):
    """Multi-step decoding: per step, append one token to every query's leaf
    and run PAC + POR; wall time per step includes the host length update
    (and re-planning when due).  The same new K/V rows and queries feed
    every policy."""
    from prefix_shared_tree_amd.decode_loop import DecodeSession

    S = a.decode_steps
    P = a.page_size if a.page_size > 0 else 16
    print(f"[bench] decode loop on {spec.name}: {S} steps, {P}-token pages", file=sys.stderr, flush=True)
    q, k, v = workloads.make_tensors(spec, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    B, hkv, hq, d = spec.num_queries, spec.num_kv_heads, spec.num_q_heads, spec.head_dim
    dt = q.dtype
    kn = torch.randn((S, B, hkv, d), generator=g, device="cuda").to(dt)
    vn = torch.randn((S, B, hkv, d), generator=g, device="cuda").to(dt)
    qs = torch.randn((S, B, hq, d), generator=g, device="cuda").to(dt)
    out = torch.empty((B, hq, d), device="cuda", dtype=torch.float32)
    lse = torch.empty((B, hq), device="cuda", dtype=torch.float32)
    results = {}
    policies = (("reuse", 0, {}), ("replan_every_16", 16, {}), ("replan_every_step", 1, {}),
                ("flatten_256_replan_every_step", 0, {"flatten": 256}))
    for name, every, kw in policies:
        sess = DecodeSession(spec, k, v, page_size=P, max_new_tokens=S, replan_every=every, plan_kw=kw)
        torch.cuda.synchronize()
        gpu, dev = [], []
        t0 = time.perf_counter()
        for s in range(S):
            a0 = torch.cuda.Event(enable_timing=True)
            a0.record()
            sess.append(kn[s], vn[s])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sess.decode(qs[s], out=out, lse=lse)
            e1.record()
            gpu.append((e0, e1))
            dev.append((a0, e1))
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / S
        results[name] = {
            "wall_ms_per_step": wall * 1e3,
            "gpu_ms_per_step": statistics.mean(x.elapsed_time(y) for x, y in gpu),
            # the step's device span: the append (new K/V rows, lengths) and PAC + POR
            "device_ms_per_step": statistics.mean(x.elapsed_time(y) for x, y in dev),
            "replans": sess.replans,
            "replan_ms_each": sess.replan_s * 1e3 / sess.replans if sess.replans else 0.0,
        }
        del sess
    # The plan-reused loop again without the per-step events (each event is a
    # marker in the stream that costs device time of its own): wall only.
    sess = DecodeSession(spec, k, v, page_size=P, max_new_tokens=S)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(S):
        sess.append(kn[s], vn[s])
        sess.decode(qs[s], out=out, lse=lse)
    torch.cuda.synchronize()
    results["reuse"]["wall_ms_per_step_no_events"] = (time.perf_counter() - t0) * 1e3 / S
    del sess
    # Tree search: every 8 steps one query finishes and another forks in two,
    # so the batch keeps its size; each fork or finish rebuilds tree and plan.
    per = -(-(1 + S) // P)
    sess = DecodeSession(spec, k, v, page_size=P, max_new_tokens=S, extra_pages=per * (2 * (S // 8) + 2))
    torch.cuda.synchronize()
    gpu, topo = [], []
    t0 = time.perf_counter()
    for s in range(S):
        if s and s % 8 == 0:
            t1 = time.perf_counter()
            sess.prune(0)
            sess.branch(sess.num_queries - 1, kn[s][:2], vn[s][:2])
            torch.cuda.synchronize()
            topo.append(time.perf_counter() - t1)
        sess.append(kn[s], vn[s])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sess.decode(qs[s], out=out, lse=lse)
        e1.record()
        gpu.append((e0, e1))
    torch.cuda.synchronize()
    results["search_fork_finish_every_8"] = {
        "wall_ms_per_step": (time.perf_counter() - t0) * 1e3 / S,
        "gpu_ms_per_step": statistics.mean(x.elapsed_time(y) for x, y in gpu),
        "rebuilds": 2 * len(topo),
        "finish_plus_fork_ms_each": statistics.mean(topo) * 1e3 if topo else 0.0,
    }
    del sess
    print(json.dumps({
        "metric": "decode steps/s (append one token per query, PAC + POR, host length update and re-planning)",
        "value": 1e3 / results["reuse"]["wall_ms_per_step"], "unit": "steps/s", "n_gpus": 1, "steps": S,
        "higher_is_better": True, "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": spec.name, "kv_layout": f"paged, {P}-token pages", "mode": "decode_loop"},
        "policies": results,
    }))


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {a.gpus}); "
              "sharding across GPUs is a design, not code.", file=sys.stderr)
        sys.exit(2)
    import torch

    import prefix_shared_tree_amd as pst
    import workloads

    if a.sweep:
        shape_sweep(torch, pst, workloads, a)
        return
    if a.flatten_sweep:
        flatten_sweep(torch, pst, workloads, a)
        return
    spec = workloads.config(a.config)
    if a.decode_steps > 0:
        decode_loop_bench(torch, pst, workloads, spec, a)
        return
    print(f"[bench] workload {spec.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v = workloads.make_tensors(spec, "cuda")
    # The kernels read kk, vv (the contiguous pools, or a paged copy); the
    # oracle sample reads the contiguous k, v.
    kk, vv, paged = k, v, None
    if a.page_size > 0:
        paged, kk, vv = workloads.page_pools(spec, k, v, a.page_size, fill=0.0,
                                             scatter=a.page_order == "scattered")
    t0 = time.perf_counter()
    tree = pst.Tree.from_paged(spec, paged) if paged else pst.Tree.from_spec(spec)
    t_tree = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    plan = pst.Plan(tree, flatten=a.flatten) if a.flatten else pst.Plan(tree)
    t_plan = (time.perf_counter() - t0) * 1e3
    st = workload_stats(spec, tree)
    pv = plan.view()
    out = torch.empty((spec.num_queries, spec.num_q_heads, spec.head_dim), device="cuda", dtype=q.dtype)
    lse = torch.empty((spec.num_queries, spec.num_q_heads), device="cuda", dtype=torch.float32)
    ws = pst.workspace(plan)
    evict_bufs = (torch.empty(1 << 30, dtype=torch.uint8, device="cuda"), torch.empty(4096, dtype=torch.float32, device="cuda"))

    print(f"[bench] timing {a.steps} cold steps", file=sys.stderr, flush=True)
    step_ms, pac_ms, por_ms, wall = time_steps(torch, pst, plan, q, kk, vv, out, lse, ws, evict_bufs, a.steps,
                                               a.warmup)
    ms = statistics.mean(step_ms)
    pac_avg = statistics.mean(pac_ms)
    warm_ms = None if a.no_warm else time_warm(torch, pst, plan, q, kk, vv, out, lse, ws, a.steps)

    # Achievable streaming read bandwidth (same 128-bit loads, 2 GiB).
    rd = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")
    pst.bench_read(rd, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        pst.bench_read(rd, sink)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 5 * rd.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del rd

    result = {
        "metric": METRIC,
        "value": st["logical_tokens"] / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": statistics.median(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V rounded to bf16; tree shape of the named workload)",
        "config": {"workload": spec.name, "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "nodes": spec.num_nodes, "queries": spec.num_queries,
                   "unique_kv_tokens": st["unique_kv_tokens"], "logical_tokens": st["logical_tokens"],
                   "cache": "cold (1 GiB read of an unrelated buffer before each step)", "plan_reused": True,
                   "kv_layout": f"paged, {a.page_size}-token pages, {a.page_order}" if paged else "contiguous",
                   "partition": f"DEFT-Flatten, {a.flatten}-token chunks" if a.flatten else "cost model"},
        "unique_kv_GBps": st["unique_kv_bytes"] / (ms * 1e-3) / 1e9,
        "unique_kv_frac_of_peak": st["unique_kv_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "pac_ms": pac_avg,
        "por_ms": statistics.mean(por_ms),
        "warm_ms_per_step": warm_ms,
        "wall_ms_per_step_incl_evict": wall * 1e3 / a.steps,
        "stream_read_GBps": read_gbs,
        "tree_build_ms": t_tree,
        "plan_ms": t_plan,
        "plan": {"bins": pv["num_bins"], "tasks": int(pv["tasks"].shape[0]), "slots": int(pv["num_slots"]),
                 "estimated_makespan_us": pv["makespan"] / 1e3,
                 "cost_model": "fitted gfx950 table" if plan.cost is not None else "analytic fallback"},
    }
    traffic = traffic_for(a.traffic, spec.name) if not paged and not a.flatten else None
    # Algorithmic work of one PAC launch: the unique KV bytes, and 4 d H_q
    # FLOPs per logical (query, token) (QK^T and PV).  The bound is the larger
    # of the two floors; the other is reported beside it.
    flops = 4.0 * spec.head_dim * spec.num_q_heads * st["logical_tokens"]
    cpeak = COMPUTE_PEAK_TFLOPS[spec.dtype]
    hbm = {"bound": "hbm", "achieved": st["unique_kv_bytes"] / (pac_avg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
           "unit": "GB/s"}
    mfma = {"bound": "mfma" if spec.dtype == "bf16" else "alu", "achieved": flops / (pac_avg * 1e-3) / 1e12,
            "peak": cpeak, "unit": "TFLOP/s"}
    for r in (hbm, mfma):
        r["frac"] = r["achieved"] / r["peak"]
    compute_bound = flops / (cpeak * 1e12) > st["unique_kv_bytes"] / (HBM_PEAK_GBS * 1e9)
    main, other = (mfma, hbm) if compute_bound else (hbm, mfma)
    result["roofline"] = dict(main, traffic=traffic, kernel="pac_kernel",
                              algorithmic_bytes_per_launch=st["unique_kv_bytes"],
                              algorithmic_flops_per_launch=flops,
                              secondary={k: other[k] for k in ("bound", "achieved", "peak", "unit", "frac")})

    if not a.no_baseline:
        print("[bench] query-guided baseline (pst_decode_attn_baseline)", file=sys.stderr, flush=True)
        bws = torch.empty(max(pst.baseline_workspace_bytes(tree, plan.cost), 256), dtype=torch.uint8,
                          device="cuda")
        bms = time_baseline(torch, pst, tree, plan.cost, q, kk, vv, out, lse, bws, evict_bufs,
                            max(3, a.steps // 4), min(a.warmup, 10))
        result["baseline_query_guided"] = {
            "ms_per_step": bms, "speedup_of_tree_path": bms / ms,
            "kv_bytes_read": st["per_query_kv_bytes"],
            "kv_read_ratio": st["per_query_kv_bytes"] / st["unique_kv_bytes"],
        }
        del bws
        # The tree path's output is recomputed below for the parity sample.
    evict(pst, evict_bufs)
    pst.decode_attn(plan, q, kk, vv, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    if not a.no_cpu_baseline:
        print("[bench] oracle on a bounded sample (cpu_baseline)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(spec, q, k, v, out, a.cpu_seconds)
    if not a.no_gate and not paged and not a.flatten:
        del q, k, v, kk, vv, out, lse, ws, plan, tree
        torch.cuda.empty_cache()
        result["gate"] = gate(torch, pst, workloads, evict_bufs, a)
    print(json.dumps(result), flush=True)


def time_baseline(torch, pst, tree, cost, q, k, v, out, lse, ws, evict_bufs, steps, warmup):
    """Mean cold-cache time of one pst_decode_attn_baseline call (ms)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        evict(pst, evict_bufs)
        pst.decode_attn_baseline(tree, q, k, v, cost=cost, out=out, lse=lse, ws=ws)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evict(pst, evict_bufs)
        ev[i][0].record(stream)
        pst.decode_attn_baseline(tree, q, k, v, cost=cost, out=out, lse=lse, ws=ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return statistics.mean(e[0].elapsed_time(e[1]) for e in ev)


GATE_CONFIGS = ("2", "3", "4")


def gate(torch, pst, workloads, evict_bufs, a):
    """PAC + POR of the document-QA, few-shot and speculative trees, measured
    like the main line (cold caches, plan reused), against 8 TB/s on their
    unique K/V bytes; with each PAC launch's HBM traffic from the counter
    summary while it matches the kernel."""
    rows = {}
    for name in GATE_CONFIGS:
        spec = workloads.config(name)
        print(f"[bench] gate workload {spec.name}", file=sys.stderr, flush=True)
        q, k, v = workloads.make_tensors(spec, "cuda")
        tree = pst.Tree.from_spec(spec)
        plan = pst.Plan(tree)
        st = workload_stats(spec, tree)
        out = torch.empty((spec.num_queries, spec.num_q_heads, spec.head_dim), device="cuda", dtype=q.dtype)
        lse = torch.empty((spec.num_queries, spec.num_q_heads), device="cuda", dtype=torch.float32)
        ws = pst.workspace(plan)
        steps, pac, por, _ = time_steps(torch, pst, plan, q, k, v, out, lse, ws, evict_bufs, a.steps, a.gate_warmup)
        ms = statistics.mean(steps)
        rows[spec.name] = {
            "config": name, "ms_per_step": ms, "pac_ms": statistics.mean(pac), "por_ms": statistics.mean(por),
            "unique_kv_bytes": st["unique_kv_bytes"], "logical_tokens": st["logical_tokens"],
            "logical_tokens_per_s": st["logical_tokens"] / (ms * 1e-3),
            "unique_kv_GBps": st["unique_kv_bytes"] / (ms * 1e-3) / 1e9,
            "unique_kv_frac_of_peak": st["unique_kv_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "pac_unique_kv_frac_of_peak": st["unique_kv_bytes"] / (statistics.mean(pac) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "pac_traffic_bytes_per_launch": traffic_for(a.traffic, spec.name),
        }
        del q, k, v, tree, plan, ws, out, lse
        torch.cuda.empty_cache()
    return {"warmup": a.gate_warmup, "steps": a.steps, "workloads": rows}


def traffic_for(path, workload):
    """HBM bytes per PAC launch for this workload from the counter summary,
    if it was taken on the current kernel code (else None)."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    entries = tr.get("entries", [tr])
    sha = kernel_sha()
    for e in entries:
        if e.get("workload") == workload and e.get("kernel_source_sha") == sha:
            return e.get("hbm_bytes_per_launch")
    return None


def kernel_sha():
    """Hash of the PAC kernel's code (comments and blank lines removed, so a
    comment edit keeps the recorded traffic; any code change drops it)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in ("pac.hip", "pst_internal.h"):
        with open(os.path.join(ROOT, "prefix_shared_tree_amd", "csrc", name), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
