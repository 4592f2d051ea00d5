"""Benchmark: verified draft positions per second on one MI355X.

Workload (the full combined verification step at the largest shape):
concurrency 32, block 16, Qwen3 vocabulary V = 151936, bf16 target logits,
K = 8 latent-mixture draft with greedy branches, DVL budget 256 (half of
32 x 16) from Beta(8, 2) survival estimates, T = 1.0, top-p 0.95, residual
and bonus sampling, Philox seeds advancing per step.  Synthetic seeded data
(synth.config(5)).  With --branch-T T_b > 0 the same workload runs with the
soft-branch drafter (each branch softmax(c / T_b)), a variant measured
beside the headline line.

A timed step is the whole verification path on inputs resident in HBM:
dvl_alloc_pack, sv_verify_rows (target-row statistics with top-p and the
branch argmax over the component rows, one launch), sv_accept_sample
(category posterior, acceptance, residual / bonus draw).  The target forward is outside the path; its output for
each step (the packed rows for that step's allocation) is prepared before the
timed region in a buffer of its own, as the target model would have written it.

Prints one JSON line.  `roofline` is for the dominant kernel (k_rows_mix of
sv_verify_rows: target-row statistics and the branch argmax over the component
rows), timed live with HIP events on the stream the kernels run on; `cpu_baseline` is the CPU oracle on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--config", type=int, default=5, choices=(3, 5),
                    help="5: conc 32 K=8 mixture with top-p and DVL (the headline workload); 3: conc 32 dense "
                         "independent draft with DVL, no top-p")
    ap.add_argument("--branch-T", type=float, default=0.0,
                    help="soft-branch mixture: the drafter samples each branch from softmax(c / T_b) and "
                         "verification uses those branch distributions (0: greedy branches, the default)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, one elementwise kernel that reads and writes MIB MiB: "
                         "the known-size reference that scales the HBM counters")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 counter_collection.csv files "
                         "(FETCH_SIZE run, WRITE_SIZE run, both with --copy-calibration) and exit")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("sv_mix.hip", "sv_rows_dev.hpp", "sv_device.hpp"):
        h.update(open(os.path.join(ROOT, "draft_verification_sv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel)
    except (ValueError, AttributeError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


ROWS_KERNEL = "k_rows_mix"


def _counter_rows(path: str, counter: str):
    """(kernel name, value) per dispatch of one counter in a rocprofv3 CSV."""
    import csv

    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            name, val = row["Kernel_Name"], float(row["Counter_Value"])
            k0 = per.get(key)
            per[key] = (name, val + (k0[1] if k0 else 0.0))  # sum over instances of one dispatch
    return list(per.values())


def summarize_counters(fetch_csv: str, write_csv: str, copy_bytes: int, algorithmic: float):
    """Per-launch HBM traffic of the rows kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the calibration kernel
    (torch.neg over copy_bytes: copy_bytes read and copy_bytes written)."""
    import numpy as np

    def split(rows):
        copy = [v for n, v in rows if "neg_kernel" in n]
        kern = [v for n, v in rows if ROWS_KERNEL in n]
        if not copy or not kern:
            raise SystemExit(f"counter file lacks the calibration copy or {ROWS_KERNEL}: "
                             f"{sorted(set(n for n, _ in rows))}")
        return max(copy), kern

    cf, kf = split(_counter_rows(fetch_csv, "FETCH_SIZE"))
    cw, kw = split(_counter_rows(write_csv, "WRITE_SIZE"))
    known_kib = copy_bytes / 1024.0
    sf, sw = known_kib / cf, known_kib / cw
    fetch_b = float(np.mean(kf)) * 1024.0 * sf
    write_b = float(np.mean(kw)) * 1024.0 * sw
    rec = {"source_sha": kernel_source_hash(), "bytes_per_launch": round(fetch_b + write_b),
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
    allrec[ROWS_KERNEL] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    args = parse()
    if args.summarize_counters:
        # cfg5 verifies exactly `budget` positions every step (all survival scores > 0)
        pos, R, K, V = 256, 32, 8, 151936
        summarize_counters(*args.summarize_counters, args.copy_calibration << 20,
                           float((pos + R) * V * 2 + pos * K * V * 2))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path runs on a single GPU)",
              file=sys.stderr)
        sys.exit(2)
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
    dense = args.config == 3
    if dense and soft:
        raise SystemExit("--branch-T applies to the mixture workload (--config 5)")
    w = synth.config(args.config, steps=S, branch_T=bT)
    R, b, V, K, B = w.R, w.b, w.V, w.K, w.budget
    print(f"[bench] data generated in {time.time() - t_gen:.1f}s: {w.name}", file=sys.stderr, flush=True)
    ld = row_pitch(V, "bf16")
    max_pos = min(B, R * b)
    max_rows = max_pos + R
    dt = sv.SV_BF16
    ws, nb = sv.make_workspace(R, b, K, V, dev)

    full = to_device_rows(w.tgt, ld, dev)            # [R*(b+1), ld]: target rows for every position
    comp = None if dense else to_device_rows(w.comp, ld, dev)    # [R*K*b, ld]
    draft = to_device_rows(w.draft, ld, dev) if dense else None  # [R*b, ld]
    mix = None if dense else torch.from_numpy(w.mix.reshape(-1)).to(dev)
    a_all = torch.from_numpy(w.a.reshape(S, R * b)).to(dev)
    x_all = torch.from_numpy(w.x.reshape(S, R * b)).to(dev)
    seeds = torch.from_numpy(w.seeds.view(np.int64)).to(dev)
    T = torch.from_numpy(w.T).to(dev)
    top_p = None if w.top_p is None else torch.from_numpy(w.top_p).to(dev)
    budget = torch.tensor([B], dtype=torch.int32, device=dev)
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
    packed = torch.empty((S, max_rows, ld), dtype=torch.bfloat16, device=dev)
    L_host = np.zeros((S, R), np.int32)
    for s in range(S):
        sv.dvl_alloc_pack(a_all[s], R, b, None, budget, s_sc, L, pos_off, tgt_off, ws, nb, sp)
        L_host[s] = L.cpu().numpy()
        pack_rows_device(full, L_host[s], b + 1, packed[s])
    torch.cuda.synchronize()
    print(f"[bench] packed target rows for {S} steps in {time.time() - t_prep:.1f}s", file=sys.stderr, flush=True)
    positions = L_host.sum(axis=1)  # verified positions per step

    def step_dense(s, ev=None):
        sv.dvl_alloc_pack(a_all[s], R, b, None, budget, s_sc, L, pos_off, tgt_off, ws, nb, sp)
        if ev is not None:
            ev[0].record(stream)
        # target-row and draft-row statistics in one launch
        sv.sv_verify_rows_dense(packed[s], dt, ld, V, tgt_off, R, max_rows, T, top_p, row_max, row_arg, row_lse,
                                row_cut, row_kept, draft, dt, ld, b, pos_off, max_pos, d_max, d_arg, d_lse, ws, nb,
                                sp)
        if ev is not None:
            ev[1].record(stream)
        # acceptance, residual / bonus draw
        sv.sv_accept_sample(packed[s], dt, ld, V, tgt_off, pos_off, R, b, T, row_arg, row_cut, row_kept, x_all[s],
                            sv.SV_Q_DENSE, draft, dt, ld, d_arg, d_lse, 0, None, None, 0, None, None, None, None,
                            seeds[s:s + 1], n_acc, token, is_bonus, None, None, None, ws, nb, sp)

    def step(s, ev=None):
        if dense:
            return step_dense(s, ev)
        sv.dvl_alloc_pack(a_all[s], R, b, None, budget, s_sc, L, pos_off, tgt_off, ws, nb, sp)
        if ev is not None:
            ev[0].record(stream)
        # target rows (statistics, top-p) and component rows (branch argmax) in one launch
        sv.sv_verify_rows(packed[s], dt, ld, V, tgt_off, R, max_rows, T, top_p, row_max, row_arg, row_lse, row_cut,
                          row_kept, comp, ld, K, b, pos_off, max_pos, branch_T, ws, nb, sp)
        if ev is not None:
            ev[1].record(stream)
        # category posterior, acceptance, residual / bonus draw
        sv.sv_accept_sample(packed[s], dt, ld, V, tgt_off, pos_off, R, b, T, row_arg, row_cut, row_kept, x_all[s],
                            sv.SV_Q_MIXTURE, None, dt, 0, None, None, K, mix, comp if soft else None,
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
    mix_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    row_bytes = V * 2
    # algorithmic bytes of the timed statistics launch(es): every target row (L_r + 1 per request) and
    # every verified position's K component rows (dense: its draft row), each read once
    per_pos = 1 if dense else K
    mix_bytes = float(np.mean((positions + R) * row_bytes + positions * per_pos * row_bytes))
    achieved = mix_bytes / (mix_ms * 1e-3) / 1e9
    # step-aggregate algorithmic bytes: target rows, component (draft) rows, one sampled row per request
    # (dense draft or soft branches: a residual also reads the draft row, or the K branch rows, of its slot)
    step_bytes = (positions + R) * row_bytes + positions * per_pos * row_bytes + R * row_bytes
    if soft:
        step_bytes = step_bytes + rejected * K * row_bytes
    if dense:
        step_bytes = step_bytes + rejected * row_bytes
    ms_per_step = elapsed / S * 1e3
    value = float(positions.sum()) / elapsed

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds)

    traffic = None if (soft or dense) else load_traffic(ROWS_KERNEL)
    mixture = f"K8 soft-branch mixture T_b {bT:g}" if soft else "K8 greedy-branch mixture"
    if dense:
        workload = ("conc32 block16 V151936 bf16, independent (dense) draft, DVL budget 256, T1.0, no top-p, "
                    "residual+bonus, seeds advancing per step")
        kernel = "k_rows_dense (sv_verify_rows_dense: target rows + draft rows)"
    else:
        workload = (f"conc32 block16 V151936 bf16, {mixture}, DVL budget 256, T1.0 top-p0.95, residual+bonus, "
                    "seeds advancing per step")
        kernel = "k_rows_mix (sv_verify_rows" + (", soft branches)" if soft else ")")
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
        "dtype": "bf16",
        "data": "synthetic (seeded Zipfian logits, Beta(8,2) survival estimates)",
        "config": {"workload": workload,
                   "requests": R, "block": b, "vocab": V, "K": K, "budget": B,
                   **({"branch_T": bT} if soft else {})},
        "step_gbps": round(float(np.mean(step_bytes)) / (ms_per_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(float(np.mean(step_bytes)) / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "avg_launch_us": round(mix_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": mix_bytes},
        "cpu_baseline": cpu,
        "device_status": status,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, seconds: float):
    """The CPU oracle as it stands, on a bounded sample of the same workload:
    whole steps (DVL, then the step: target statistics with top-p, mixture
    argmax and posterior, acceptance, residual/bonus) until `seconds` pass."""
    import numpy as np

    import oracle

    R, b, V, K = w.R, w.b, w.V, w.K
    tgt = w.tgt.reshape(R * (b + 1), V)
    prop = dict(comp=w.comp.reshape(R * K * b, V), comp_row0=np.arange(R) * K * b, mix=w.mix, branch_T=w.branch_T) \
        if K > 0 else dict(draft=w.draft.reshape(R * b, V), draft_row0=np.arange(R) * b)
    t0 = time.perf_counter()
    pos = n = 0
    while n < w.steps:
        dv = oracle.dvl(w.a[n], w.budget)
        oracle.step(tgt=tgt, tgt_row0=np.arange(R) * (b + 1), L=dv["L"], T=w.T, x=w.x[n], seed=int(w.seeds[n]),
                    top_p=w.top_p, **prop)
        pos += int(dv["L"].sum())
        n += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(pos / el, 2), "unit": "positions/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} whole steps of the same workload ({pos} verified positions) in {el:.1f}s"}


if __name__ == "__main__":
    main()
