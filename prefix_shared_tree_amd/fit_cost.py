"""Fit the partial-attention cost table C_est(rows, len) on the GPU.

CoDec (CoDec: Prefix-Shared Decoding Kernel for LLMs), section 工作负载平衡,
profile-based cost estimation: before deployment, the partial-attention
kernel is profiled on the target hardware and head layout over a grid of KV
lengths n and query counts n_q; other shapes are interpolated.

Here one measurement times PAC launches over trees of identical nodes with
the plan forced to one piece per node and k nodes per bin: every workgroup of
a full-GPU launch runs k pieces of `rows` query rows and `len` tokens, on a
loaded GPU (shared HBM bandwidth included), caches flushed before every
launch.  The cost of a piece is the marginal time (T(k) - T(1)) / (k - 1), so
the launch itself, paid once per launch and not per piece, is left out.
Caches are emptied by reading 1 GiB of an unrelated buffer (reads leave no
dirty lines whose write-back would be charged to the measured launch).  The
table is made non-decreasing along both axes and written as JSON:

    python -m prefix_shared_tree_amd.fit_cost --q-heads 32 --kv-heads 8 --head-dim 128 --dtype bf16
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROWS_GRID = [1, 2, 4, 8, 16, 32, 64, 128, 256]
LEN_GRID = [16 << i for i in range(13)]  # 16 .. 65536


def table_path(hq, hkv, d, dtype):
    here = os.path.dirname(os.path.abspath(__file__))
    return os.path.join(here, "cost_tables", f"gfx950_{dtype}_q{hq}_kv{hkv}_d{d}.json")


def measure(pst, torch, hq, hkv, d, dtype, rows, length, bins, reps, flush, per_bin=1):
    g = hq // hkv
    nq = max(1, rows // g)
    n = bins * per_bin
    lens = np.full(n, length, dtype=np.int64)
    offs = np.arange(n, dtype=np.int64) * length
    parent = np.full(n, -1, dtype=np.int32)
    qnode = np.repeat(np.arange(n, dtype=np.int32), nq)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    tree = pst.Tree(parent, offs, lens, qnode, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                    out_dtype="f32")
    plan = pst.Plan(tree, num_bins=bins, no_split=True, max_rows=256 if dtype == "bf16" else 16,
                    use_fitted=False)
    tasks = plan.view()["tasks"]
    assert len(tasks) == n * -(-nq * g // (256 if dtype == "bf16" else 16))
    q = torch.randn((len(qnode), hq, d), device="cuda").to(tdt)
    k = torch.randn((hkv, n * length, d), device="cuda").to(tdt)
    v = torch.randn((hkv, n * length, d), device="cuda").to(tdt)
    ws = pst.workspace(plan)
    stream = torch.cuda.current_stream()
    times = []
    for i in range(reps + 1):
        pst.bench_read(flush[0], flush[1])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        pst.pac(plan, q, k, v, ws)
        b.record(stream)
        torch.cuda.synchronize()
        if i:
            times.append(a.elapsed_time(b) * 1e6)  # ns
    del q, k, v, ws
    return statistics.median(times), nq * g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--q-heads", type=int, default=32)
    ap.add_argument("--kv-heads", type=int, default=8)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--dtype", default="bf16")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--max-len", type=int, default=65536)
    ap.add_argument("--k", type=int, default=4, help="pieces per workgroup of the second launch")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    import torch

    import prefix_shared_tree_amd as pst

    hq, hkv, d = a.q_heads, a.kv_heads, a.head_dim
    g = hq // hkv
    cus, per = pst.device_info()
    bins = max(1, cus * per // hkv)
    flush = (torch.empty(1 << 30, dtype=torch.uint8, device="cuda"), torch.empty(4096, dtype=torch.float32, device="cuda"))
    rows_max = 256 if a.dtype == "bf16" else 16
    raw = {}
    launch = []
    t0 = time.time()
    for rows in ROWS_GRID:
        if rows > rows_max or rows < g:
            continue
        for length in LEN_GRID:
            if length > a.max_len:
                continue
            t1, _ = measure(pst, torch, hq, hkv, d, a.dtype, rows, length, bins, a.reps, flush, 1)
            tk, _ = measure(pst, torch, hq, hkv, d, a.dtype, rows, length, bins, a.reps, flush, a.k)
            ns = max(1.0, (tk - t1) / (a.k - 1))
            raw[(rows, length)] = ns
            launch.append(t1 - ns)
            print(f"rows {rows:4d} len {length:6d}: {ns / 1e3:10.2f} us per piece  (one piece per bin: {t1 / 1e3:.2f} us; "
                  f"{time.time() - t0:.0f} s)", flush=True)
    # Fill: rows below the GQA group take the group's value, rows above the
    # workgroup capacity the capacity's; lengths beyond max-len extrapolate.
    R = [r for r in ROWS_GRID]
    table = np.zeros((len(R), len(LEN_GRID)), dtype=np.int64)
    for i, rows in enumerate(R):
        rr = min(max(rows, g), rows_max)
        rr = next(x for x in ROWS_GRID if x >= rr)
        for j, length in enumerate(LEN_GRID):
            if (rr, length) in raw:
                table[i, j] = int(raw[(rr, length)])
            else:
                jj = max(jj for jj, L in enumerate(LEN_GRID) if (rr, L) in raw)
                j0 = jj - 1
                c1, c0 = raw[(rr, LEN_GRID[jj])], raw[(rr, LEN_GRID[j0])]
                table[i, j] = int(c1 + (c1 - c0) * (length - LEN_GRID[jj]) / (LEN_GRID[jj] - LEN_GRID[j0]))
    table = np.maximum.accumulate(np.maximum.accumulate(np.maximum(table, 1), axis=1), axis=0)
    out = a.out or table_path(hq, hkv, d, a.dtype)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    doc = {
        "arch": "gfx950", "dtype": a.dtype, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
        "bins": bins,
        "method": f"marginal per-piece time (T({a.k} pieces per workgroup) - T(1)) / {a.k - 1}, medians of PAC "
                  "launches over the whole GPU, cold caches",
        "launch_overhead_ns_median": float(np.median(launch)) if launch else 0.0,
        "rows_grid": R, "len_grid": LEN_GRID, "table_ns": table.tolist(),
        "raw_ns": {f"{r},{L}": v for (r, L), v in sorted(raw.items())},
    }
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
    print(f"wrote {out}", file=sys.stderr)


if __name__ == "__main__":
    main()
