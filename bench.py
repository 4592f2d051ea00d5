"""Benchmark: verified draft positions per second on one MI355X.

Default workload (the full combined verification step at the largest shape):
concurrency 32, block 16, Qwen3 vocabulary V = 151936, bf16 target logits,
K = 8 latent-mixture draft with greedy branches, DVL budget 256 (half of
32 x 16) from Beta(8, 2) survival estimates, T = 1.0, top-p 0.95, residual
and bonus sampling, Philox seeds advancing per step.  Synthetic seeded data
(synth.config(5)).  --config 1..4 runs the other workloads (1: 4 requests,
V 1024, fp32, dense draft; 2: conc 8, dense draft, full verification; 3: conc
32, dense draft, DVL 256; 4: conc 16, K 8 mixture, T 1.5, top-p 0.95, full
verification).  With --branch-T T_b > 0 the mixture workloads run with the
soft-branch drafter (each branch softmax(c / T_b)).

A timed step is the whole verification path on inputs resident in HBM:
dvl_alloc_pack (workloads with a budget), the rows launch (sv_verify_rows:
target-row statistics with top-p and the branch argmax over the component
rows; sv_verify_rows_dense: target and draft rows), sv_accept_sample
(category posterior, acceptance, residual / bonus draw).  The target forward
is outside the path; its output for each step (the packed rows for that
step's allocation) is prepared before the timed region in a buffer of its
own.  Tensors that every step re-reads (the component or draft rows, and the
target rows under full verification) are held in several device copies used
in turn, so that a step never reads what the steps before it left in the
256 MB Infinity Cache (--copies overrides the count).

Prints one JSON line.  `roofline` is for the dominant kernel (the rows
launch), timed live with HIP events on the stream the kernels run on;
`cpu_baseline` is the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20  # Infinity Cache of one MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--config", type=int, default=5, choices=(1, 2, 3, 4, 5),
                    help="5: conc 32 K=8 mixture with top-p and DVL (the headline workload); 1-4: the other "
                         "workloads")
    ap.add_argument("--graph", action="store_true",
                    help="also capture each step's calls as a HIP graph (one graph per step, same buffers) and time "
                         "the replays back to back (reported as graph_ms_per_step; value stays the eager rate)")
    ap.add_argument("--tree", action="store_true",
                    help="tree verification instead of a block: conc 32, depth 16, random draft trees of at most 64 "
                         "nodes (at most 4 children per node), V 151936 bf16, T 1, top-p 0.95")
    ap.add_argument("--branch-T", type=float, default=0.0,
                    help="soft-branch mixture: the drafter samples each branch from softmax(c / T_b) and "
                         "verification uses those branch distributions (0: greedy branches, the default)")
    ap.add_argument("--copies", type=int, default=0,
                    help="device copies of each re-read tensor, used in turn (0: enough that a step never re-reads "
                         "what the previous 768 MB of reads left in cache)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, one elementwise kernel that reads and writes MIB MiB: "
                         "the known-size reference that scales the HBM counters")
    ap.add_argument("--summarize-db", nargs="+", metavar="DB",
                    help="print a markdown summary (per-kernel mean duration, or mean counter values) of rocprofv3 "
                         "result databases (*_results.db) and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH", "WRITE"),
                    help="write the rows kernel's record in profiles/traffic.json from two rocprofv3 counter "
                         "outputs (counter_collection.csv or *_results.db: a FETCH_SIZE run, a WRITE_SIZE run, both "
                         "with --copy-calibration and the same --config) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- HBM traffic records
def rows_kernel(config: int) -> str:
    return "k_rows_mix" if config in (4, 5) else "k_rows_dense"


KERNEL_SOURCES = {
    "k_rows_mix": ("sv_mix.hip", "sv_rows_dev.hpp", "sv_device.hpp"),
    "k_rows_dense": ("sv_rows.hip", "sv_rows_dev.hpp", "sv_device.hpp"),
    "k_row_stats": ("sv_rows.hip", "sv_rows_dev.hpp", "sv_device.hpp"),
}
TREE_TRAFFIC_KEY = "tree:k_row_stats"  # the tree step's node-row statistics launch


def _code_only(text: str) -> str:
    """A source file's code: comments, trailing spaces and blank lines removed,
    so that a record stays tied to the code that was measured, not its comments."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "draft_verification_sv_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_key(config: int) -> str:
    return f"cfg{config}:{rows_kernel(config)}"


def load_traffic(config: int, key: str | None = None, kernel: str | None = None):
    """HBM traffic per launch of the rows kernel from committed rocprofv3 counter
    runs of this workload, if they were taken on the current kernel source; else None."""
    key = key or traffic_key(config)
    kernel = kernel or rows_kernel(config)
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(key)
    except (ValueError, AttributeError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(path: str, counter: str, grid: int | None = None):
    """(kernel name, value) per dispatch of one counter in a rocprofv3 CSV or result database
    (databases: only dispatches of `grid` threads when given)."""
    import csv

    per = {}
    if path.endswith(".db"):
        import sqlite3

        con = sqlite3.connect(path)
        for key, name, val, gs in con.execute("select dispatch_id, kernel_name, value, grid_size from "
                                              "counters_collection where counter_name = ?", (counter,)):
            if grid is not None and gs != grid and "neg_kernel" not in name:
                continue
            k0 = per.get(key)
            per[key] = (name, float(val) + (k0[1] if k0 else 0.0))
        return list(per.values())
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            name, val = row["Kernel_Name"], float(row["Counter_Value"])
            k0 = per.get(key)
            per[key] = (name, val + (k0[1] if k0 else 0.0))  # sum over instances of one dispatch
    return list(per.values())


def algorithmic_rows_bytes(config: int) -> float:
    """Algorithmic bytes of one rows launch: every target row (L_r + 1 per request)
    and every verified position's K component rows (dense: its draft row), each
    read once.  Workloads with a budget verify exactly `budget` positions (every
    survival score is positive)."""
    import synth

    w = synth.config(config, V=8, steps=1)  # the shapes only
    R, b, K = w.R, w.b, w.K
    V, esz = 151936 if config != 1 else 1024, 2 if config != 1 else 4
    pos = w.budget if w.budget is not None else R * b
    return float((pos + R) * V * esz + pos * max(K, 1) * V * esz)


def summarize_counters(config: int, fetch_csv: str, write_csv: str, copy_bytes: int, tree: bool = False):
    """Per-launch HBM traffic of the rows kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the calibration kernel
    (torch.neg over copy_bytes: copy_bytes read and copy_bytes written).  tree: the
    tree step's node-row statistics launch (k_row_stats over the node rows)."""
    import numpy as np

    kernel = "k_row_stats" if tree else rows_kernel(config)
    grid = None
    if tree:
        import synth

        sh = TREE_SHAPE
        tw = synth.tree("shape", R=sh["R"], b=sh["b"], V=synth.QWEN3_VOCAB, width=sh["width"], nodes=sh["nodes"],
                        T=sh["T"], top_p=sh["top_p"], seed=TREE_DATA_SEED, vseed=TREE_DATA_SEED_VERIFY)
        n_nodes = int(tw.node_off[-1])
        grid = n_nodes * 512  # one 512-thread block per node row

    def split(rows):
        copy = [v for n, v in rows if "neg_kernel" in n]
        kern = [v for n, v in rows if kernel in n]
        if not copy or not kern:
            raise SystemExit(f"counter file lacks the calibration copy or {kernel}: "
                             f"{sorted(set(n for n, _ in rows))}")
        return max(copy), kern

    algorithmic = float(n_nodes * 151936 * 2) if tree else algorithmic_rows_bytes(config)
    cf, kf = split(_counter_rows(fetch_csv, "FETCH_SIZE", grid))
    cw, kw = split(_counter_rows(write_csv, "WRITE_SIZE", grid))
    known_kib = copy_bytes / 1024.0
    sf, sw = known_kib / cf, known_kib / cw
    fetch_b = float(np.mean(kf)) * 1024.0 * sf
    write_b = float(np.mean(kw)) * 1024.0 * sw
    rec = {"source_sha": kernel_source_hash(kernel), "bytes_per_launch": round(fetch_b + write_b),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "fetch_kib_raw": float(np.mean(kf)), "write_kib_raw": float(np.mean(kw)),
           "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw, "copy_bytes": copy_bytes,
           "scale_fetch": sf, "scale_write": sw, "launches": [len(kf), len(kw)],
           "algorithmic_bytes": algorithmic, "traffic_over_algorithmic": (fetch_b + write_b) / algorithmic}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = {}
    if os.path.exists(path):
        try:
            allrec = json.load(open(path))
        except ValueError:
            allrec = {}
    allrec[TREE_TRAFFIC_KEY if tree else traffic_key(config)] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1)
    print(json.dumps(rec, indent=1))


# ---------------------------------------------------------------- the benchmark
def copies_for(per_step_bytes: float, override: int) -> int:
    """Copies of a tensor of which each step reads per_step_bytes, so that a copy
    is read again only after 3x the Infinity Cache's size of other reads."""
    if override > 0:
        return override
    return max(1, min(64, math.ceil(3 * MALL_BYTES / max(per_step_bytes, 1.0))))


def summarize_db(paths):
    """Markdown tables from rocprofv3 result databases: per kernel, the number of
    dispatches and mean duration (kernel traces), or the mean of each counter
    over its dispatches (counter runs)."""
    import collections
    import sqlite3

    def short(name):
        name = name.split("(")[0]
        return name[5:] if name.startswith("void ") else name

    for path in paths:
        con = sqlite3.connect(path)
        views = {r[0] for r in con.execute("select name from sqlite_master where type in ('table', 'view')")}
        print(f"### {os.path.basename(os.path.dirname(path))}/{os.path.basename(path)}\n")
        rows = list(con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection")) \
            if "counters_collection" in views else []
        if rows:
            per = collections.defaultdict(float)  # a counter's instances (per XCD, SE ...) summed per dispatch
            for did, name, counter, value in rows:
                per[(did, short(name), counter)] += float(value)
            acc = collections.defaultdict(lambda: collections.defaultdict(list))
            for (_, name, counter), value in per.items():
                acc[name][counter].append(value)
            counters = sorted({c for k in acc.values() for c in k})
            print("| kernel | dispatches | " + " | ".join(counters) + " |")
            print("|---|---|" + "---|" * len(counters))
            for k in sorted(acc):
                n = max(len(v) for v in acc[k].values())
                cells = [f"{sum(acc[k][c]) / len(acc[k][c]):.4g}" if acc[k].get(c) else "" for c in counters]
                print(f"| {k} | {n} | " + " | ".join(cells) + " |")
        else:
            print("| kernel | dispatches | mean us | total us |\n|---|---|---|---|")
            for name, calls, total, avg, _ in con.execute("select * from top_kernels"):
                print(f"| {short(name)} | {calls} | {avg:.2f} | {total:.1f} |")
        print()


def main():
    args = parse()
    if args.summarize_db:
        summarize_db(args.summarize_db)
        return
    if args.summarize_counters:
        summarize_counters(args.config, *args.summarize_counters, args.copy_calibration << 20, tree=args.tree)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path runs on a single GPU)",
              file=sys.stderr)
        sys.exit(2)
    if args.tree:
        main_tree(args)
        return
    import numpy as np
    import torch

    import draft_verification_sv_amd as sv
    import synth
    from draft_verification_sv_amd.step import pack_rows_device, row_pitch, to_device_rows

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    S = args.steps
    t_gen = time.time()
    bT = args.branch_T
    soft = bT > 0
    cfg = args.config
    if soft and cfg not in (4, 5):
        raise SystemExit("--branch-T applies to the mixture workloads (--config 4 or 5)")
    w = synth.config(cfg, steps=S, branch_T=bT)
    R, b, V, K, B = w.R, w.b, w.V, w.K, w.budget
    dense = K == 0
    dvl = B is not None
    print(f"[bench] data generated in {time.time() - t_gen:.1f}s: {w.name}", file=sys.stderr, flush=True)
    ld = row_pitch(V, w.dtype)
    esz = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    max_pos = min(B, R * b) if dvl else R * b
    max_rows = max_pos + R
    ws, nb = sv.make_workspace(R, b, K, V, dev)
    row_bytes = V * esz

    # proposal rows, in copies used in turn
    prop_host = w.draft if dense else w.comp
    prop_rows_per_step = max_pos * (1 if dense else K)
    n_prop = copies_for(prop_rows_per_step * row_bytes, args.copies)
    prop = [to_device_rows(prop_host, ld, dev) for _ in range(n_prop)]
    mix = None if dense else torch.from_numpy(w.mix.reshape(-1)).to(dev)
    a_all = torch.from_numpy(w.a.reshape(S, R * b)).to(dev) if dvl else None
    x_all = torch.from_numpy(w.x.reshape(S, R * b)).to(dev)
    seeds = torch.from_numpy(w.seeds.view(np.int64)).to(dev)
    T = torch.from_numpy(w.T).to(dev)
    top_p = None if w.top_p is None else torch.from_numpy(w.top_p).to(dev)
    budget = torch.tensor([B if dvl else 0], dtype=torch.int32, device=dev)
    branch_T = torch.full((R,), bT, dtype=torch.float32, device=dev) if soft else None

    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    z = lambda n, t: torch.zeros(n, dtype=t, device=dev)  # noqa: E731
    s_sc, L, pos_off, tgt_off = z(R * b, f32), z(R, i32), z(R + 1, i32), z(R + 1, i32)
    row_max, row_arg, row_lse, row_cut, row_kept = z(max_rows, f32), z(max_rows, i32), z(max_rows, f64), \
        z(max_rows, f32), z(max_rows, f64)
    branch_tok, post_w, q_at = z(max(R * K * b, 1), i32), z(max(R * b * K, 1), f64), z(R * b, f64)
    d_max, d_arg, d_lse = z(max_pos, f32), z(max_pos, i32), z(max_pos, f64)
    n_acc, token, is_bonus = z(R, i32), z(R, i32), z(R, i32)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    if args.copy_calibration > 0:  # known-size reference for the HBM counters (untimed)
        # an elementwise kernel that reads MIB MiB and writes MIB MiB once (a copy
        # through hipMemcpy would run on a DMA engine, outside the counters)
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- the target forward's output for every step, prepared before timing
    t_prep = time.time()
    full = to_device_rows(w.tgt, ld, dev)  # [R*(b+1), ld]: target rows for every position
    L_host = np.zeros((S, R), np.int32)
    if dvl:  # each step's packed rows in a buffer of its own
        packed = torch.empty((S, max_rows, ld), dtype=tdt, device=dev)
        for s in range(S):
            sv.dvl_alloc_pack(a_all[s], R, b, None, budget, s_sc, L, pos_off, tgt_off, ws, nb, sp)
            L_host[s] = L.cpu().numpy()
            pack_rows_device(full, L_host[s], b + 1, packed[s])
        del full
        n_tgt = S
    else:  # full verification: the same rows every step, in copies used in turn
        L_host[:] = b
        n_tgt = copies_for(max_rows * row_bytes, args.copies)
        packed = [full] + [full.clone() for _ in range(n_tgt - 1)]
        L.fill_(b)
        pos_off.copy_(torch.arange(R + 1, dtype=i32, device=dev) * b)
        tgt_off.copy_(torch.arange(R + 1, dtype=i32, device=dev) * (b + 1))
    torch.cuda.synchronize()
    print(f"[bench] target rows for {S} steps in {time.time() - t_prep:.1f}s; {n_tgt} target and {n_prop} "
          f"proposal copies", file=sys.stderr, flush=True)
    positions = L_host.sum(axis=1)  # verified positions per step

    def step(s, ev=None):
        sp = torch.cuda.current_stream(dev).cuda_stream  # the capture stream while a graph records
        tg = packed[s % n_tgt]
        pr = prop[s % n_prop]
        if dvl:
            sv.dvl_alloc_pack(a_all[s], R, b, None, budget, s_sc, L, pos_off, tgt_off, ws, nb, sp)
        if ev is not None:
            ev[0].record(stream)
        if dense:  # target-row and draft-row statistics in one launch
            sv.sv_verify_rows_dense(tg, dt, ld, V, tgt_off, R, max_rows, T, top_p, row_max, row_arg, row_lse,
                                    row_cut, row_kept, pr, dt, ld, b, pos_off, max_pos, x_all[s], d_max, d_arg,
                                    d_lse, ws, nb, sp)
        else:  # target rows (statistics, top-p) and component rows (branch argmax) in one launch
            sv.sv_verify_rows(tg, dt, ld, V, tgt_off, R, max_rows, T, top_p, row_max, row_arg, row_lse, row_cut,
                              row_kept, pr, ld, K, b, pos_off, max_pos, x_all[s], branch_T, ws, nb, sp)
        if ev is not None:
            ev[1].record(stream)
        # (mixture: category posterior), acceptance, residual / bonus draw
        if dense:
            sv.sv_accept_sample(tg, dt, ld, V, tgt_off, pos_off, R, b, T, row_arg, row_cut, row_kept, x_all[s],
                                sv.SV_Q_DENSE, pr, dt, ld, d_arg, d_lse, 0, None, None, 0, None, None, None, None,
                                seeds[s:s + 1], n_acc, token, is_bonus, None, None, None, ws, nb, sp)
        else:
            sv.sv_accept_sample(tg, dt, ld, V, tgt_off, pos_off, R, b, T, row_arg, row_cut, row_kept, x_all[s],
                                sv.SV_Q_MIXTURE, None, dt, 0, None, None, K, mix, pr if soft else None,
                                ld if soft else 0, branch_T, branch_tok, post_w, q_at,
                                seeds[s:s + 1], n_acc, token, is_bonus, None, None, None, ws, nb, sp)

    for k in range(args.warmup):
        step(k % S)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(S):
        step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    status = sv.sv_get_status(ws, sp)
    if status:
        print(f"[bench] device status {sv.decode_status(status)}", file=sys.stderr, flush=True)

    # ---- dominant kernel, timed with HIP events on the kernels' stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    nacc_hist = torch.zeros((S, R), dtype=torch.int32, device=dev)  # per-step accepted lengths (untimed pass)
    for s in range(S):
        step(s, evs[s])
        nacc_hist[s].copy_(n_acc)
    torch.cuda.synchronize()
    rejected = (nacc_hist.cpu().numpy() < L_host).sum(axis=1)  # requests drawing a residual, per step
    rows_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    # algorithmic bytes of the rows launch: every target row (L_r + 1 per request) and every verified
    # position's K component rows (dense: its draft row), each read once
    per_pos = 1 if dense else K
    rows_bytes = float(np.mean((positions + R) * row_bytes + positions * per_pos * row_bytes))
    achieved = rows_bytes / (rows_ms * 1e-3) / 1e9
    # step-aggregate algorithmic bytes: target rows, component (draft) rows, one sampled row per request
    # (dense draft or soft branches: a residual also reads the draft row, or the K branch rows, of its slot)
    step_bytes = (positions + R) * row_bytes + positions * per_pos * row_bytes + R * row_bytes
    if soft:
        step_bytes = step_bytes + rejected * K * row_bytes
    if dense:
        step_bytes = step_bytes + rejected * row_bytes
    ms_per_step = elapsed / S * 1e3
    value = float(positions.sum()) / elapsed

    graph_ms = None
    if args.graph:  # one HIP graph per step over the same buffers; replays timed back to back
        from draft_verification_sv_amd.step import capture_graph

        graphs = [capture_graph(lambda s=s: step(s)) for s in range(S)]
        for g in graphs[:min(S, args.warmup)]:
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg0) / S * 1e3
        del graphs

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds)

    traffic = None if soft else load_traffic(cfg)
    prop_desc = (f"K8 soft-branch mixture T_b {bT:g}" if soft else "K8 greedy-branch mixture") if not dense \
        else "independent (dense) draft"
    alloc = f"DVL budget {B}" if dvl else "full verification"
    tp = f"top-p{w.top_p[0]:g}" if w.top_p is not None else "no top-p"
    temps = "/".join(f"{t:g}" for t in sorted(set(w.T.tolist())))
    workload = (f"cfg{cfg}: conc{R} block{b} V{V} {w.dtype}, {prop_desc}, {alloc}, T{temps} {tp}, residual+bonus, "
                f"seeds advancing per step")
    kernel = rows_kernel(cfg) + (" (sv_verify_rows" + (", soft branches)" if soft else ")") if not dense
                                 else " (sv_verify_rows_dense: target rows + draft rows)")
    out = {
        "metric": "verified draft positions/sec at V=151936, conc 32; % of peak HBM GB/s",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Zipfian logits, Beta(8,2) survival estimates)" if cfg != 1
                else "synthetic (seeded N(0, 4) logits)",
        "config": {"workload": workload,
                   "requests": R, "block": b, "vocab": V, "K": K, "budget": B,
                   "copies": {"target": n_tgt if not dvl else "one per step", "proposal": n_prop},
                   **({"branch_T": bT} if soft else {})},
        "step_gbps": round(float(np.mean(step_bytes)) / (ms_per_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(float(np.mean(step_bytes)) / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "avg_launch_us": round(rows_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": rows_bytes},
        "cpu_baseline": cpu,
        "device_status": status,
    }
    if graph_ms is not None:
        out["graph_ms_per_step"] = round(graph_ms, 5)
    print(json.dumps(out), flush=True)


TREE_SHAPE = dict(R=32, b=16, width=4, nodes=64, T=1.0, top_p=0.95)
TREE_DATA_SEED = 3900        # trees and logits
TREE_DATA_SEED_VERIFY = 11   # verification seed of step 0 (advancing per step)


def main_tree(args):
    """Tree verification step: the node rows' statistics with top-p
    (sv_topp_threshold, row_off = node offsets), the drafter's rows'
    statistics (sv_softmax_stats), and sv_tree_verify (checks, residual
    masses, the walk, the draw).  The trees and logits are fixed; the
    verification seed advances per step.  A verified draft position is a
    draft node (every node but the roots)."""
    import numpy as np
    import torch

    import draft_verification_sv_amd as sv
    import synth
    from draft_verification_sv_amd.step import row_pitch, to_device_rows

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    S = args.steps
    t_gen = time.time()
    sh = TREE_SHAPE
    w = synth.tree("tree-conc32-d16-n64-w4-topp", R=sh["R"], b=sh["b"], V=synth.QWEN3_VOCAB, width=sh["width"],
                   nodes=sh["nodes"], T=sh["T"], top_p=sh["top_p"], seed=TREE_DATA_SEED, vseed=TREE_DATA_SEED_VERIFY)
    R, b, V = w.R, w.b, w.V
    n = int(w.node_off[-1])
    print(f"[bench] tree data generated in {time.time() - t_gen:.1f}s: {n} nodes, at most {w.max_kids} children",
          file=sys.stderr, flush=True)
    ld = row_pitch(V, "bf16")
    row_bytes = V * 2
    dt = sv.SV_BF16
    n_t = copies_for(n * row_bytes, args.copies)
    n_d = copies_for(R * b * row_bytes, args.copies)
    tg = [to_device_rows(w.tgt, ld, dev) for _ in range(n_t)]
    dr = [to_device_rows(w.draft.reshape(R * b, V), ld, dev) for _ in range(n_d)]
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    z = lambda k, t: torch.zeros(k, dtype=t, device=dev)  # noqa: E731
    T = torch.from_numpy(w.T).to(dev)
    tp = torch.from_numpy(w.top_p).to(dev)
    node_off = torch.from_numpy(w.node_off).to(dev)
    parent = torch.from_numpy(w.parent).to(dev)
    token = torch.from_numpy(w.token).to(dev)
    pos_off = torch.arange(R + 1, dtype=i32, device=dev) * b
    seeds = torch.arange(S, dtype=torch.int64, device=dev) + w.seed
    ws, nb = sv.make_workspace(R, b, 0, V, dev)
    st = [z(n, t) for t in (f32, i32, f64, f32, f64)]
    ds = [z(R * b, t) for t in (f32, i32, f64)]
    tb = sv.sv_tree_workspace_bytes(n, w.max_kids, V)
    tws = torch.zeros(tb, dtype=torch.uint8, device=dev)
    n_acc, path, stop, token_out, is_bonus = z(R, i32), z(R * b, i32), z(R, i32), z(R, i32), z(R, i32)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    if args.copy_calibration > 0:  # known-size reference for the HBM counters (untimed), as in main()
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step(s, ev=None):
        t, d = tg[s % n_t], dr[s % n_d]
        if ev is not None:
            ev[0].record(stream)
        sv.sv_topp_threshold(t, dt, ld, V, node_off, 0, R, n, T, tp, *st, ws, nb, sp)
        if ev is not None:
            ev[1].record(stream)
        sv.sv_softmax_stats(d, dt, ld, V, pos_off, b, R, R * b, T, *ds, ws, nb, sp)
        sv.sv_tree_verify(t, dt, ld, V, node_off, parent, token, R, b, n, w.max_kids, T, st[1], st[3], st[4], d, dt,
                          ld, ds[1], ds[2], seeds[s:s + 1], n_acc, path, stop, token_out, is_bonus, None, None, None,
                          ws, nb, tws, tb, sp)

    for k in range(args.warmup):
        step(k % S)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(S):
        step(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    status = sv.sv_get_status(ws, sp)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    acc = np.zeros(S)
    for s in range(S):
        step(s, evs[s])
        acc[s] = float(n_acc.sum().item())
    torch.cuda.synchronize()
    stats_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    ms_per_step = elapsed / S * 1e3
    positions = n - R
    stats_bytes = float(n * row_bytes)
    achieved = stats_bytes / (stats_ms * 1e-3) / 1e9
    # node rows and drafter rows read once, plus each request's drawn row (and, for a residual, its draft row)
    step_bytes = (n + R * b + 2 * R) * row_bytes
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_tree(w, args.cpu_seconds)
    out = {
        "metric": "verified draft positions/sec at V=151936, conc 32; % of peak HBM GB/s",
        "value": round(positions * S / elapsed, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Zipfian logits, random draft trees)",
        "config": {"workload": f"tree: conc{R} depth{b} V{V} bf16, random draft trees of at most {sh['nodes']} nodes "
                               f"(at most {sh['width']} children), {n} nodes ({positions} draft nodes) per step, "
                               f"T{sh['T']:g} top-p{sh['top_p']:g}, multi-round speculative sampling, seeds advancing "
                               f"per step",
                   "requests": R, "depth": b, "vocab": V, "nodes": n, "max_children": w.max_kids,
                   "copies": {"node_rows": n_t, "draft_rows": n_d}},
        "accepted_per_step": round(float(acc.mean()), 2),
        "step_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"kernel": "k_row_stats (sv_topp_threshold over the node rows)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": load_traffic(0, TREE_TRAFFIC_KEY, "k_row_stats"),
                     "avg_launch_us": round(stats_ms * 1e3, 2), "algorithmic_bytes_per_launch": stats_bytes},
        "cpu_baseline": cpu,
        "device_status": status,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_tree(w, seconds: float):
    """The CPU oracle's tree step on the same trees and rows, seeds advancing,
    until `seconds` pass (every OpenMP thread the oracle uses)."""
    import oracle

    import numpy as np

    n = int(w.node_off[-1])
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    k = 0
    while True:
        oracle.tree_step(tgt=w.tgt, tgt_row=np.arange(n), node_off=w.node_off, parent=w.parent, token=w.token, T=w.T,
                         b=w.b, seed=w.seed + k, draft=w.draft.reshape(w.R * w.b, w.V),
                         draft_row0=np.arange(w.R) * w.b, top_p=w.top_p)
        k += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(k * (n - w.R) / el, 2), "unit": "positions/s", "cores": min(threads, w.R), "kind": "oracle",
            "sample": f"{k} whole tree steps of the same workload ({k * (n - w.R)} draft nodes) in {el:.1f}s",
            "nproc": os.cpu_count(), "omp_threads": threads}


def cpu_baseline(w, seconds: float):
    """The CPU oracle as it stands, on a bounded sample of the same workload:
    whole steps (DVL when the workload has a budget, then the step: target
    statistics with top-p, proposal, acceptance, residual/bonus) on every
    OpenMP thread until `seconds` pass; then one step on a single thread."""
    import numpy as np

    import oracle

    R, b, V, K = w.R, w.b, w.V, w.K
    tgt = w.tgt.reshape(R * (b + 1), V)
    prop = dict(comp=w.comp.reshape(R * K * b, V), comp_row0=np.arange(R) * K * b, mix=w.mix, branch_T=w.branch_T) \
        if K > 0 else dict(draft=w.draft.reshape(R * b, V), draft_row0=np.arange(R) * b)

    def one(n):
        if w.budget is not None:
            Lr = oracle.dvl(w.a[n], w.budget)["L"]
        else:
            Lr = np.full(R, b, np.int32)
        oracle.step(tgt=tgt, tgt_row0=np.arange(R) * (b + 1), L=Lr, T=w.T, x=w.x[n], seed=int(w.seeds[n]),
                    top_p=w.top_p, **prop)
        return int(Lr.sum())

    threads = oracle.num_threads()
    t0 = time.perf_counter()
    pos = n = 0
    while n < w.steps:
        pos += one(n)
        n += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    one(0)
    single = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    return {"value": round(pos / el, 2), "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} whole steps of the same workload ({pos} verified positions) in {el:.1f}s",
            "nproc": os.cpu_count(), "omp_threads": threads, "single_thread_step_s": round(single, 3)}


if __name__ == "__main__":
    main()
