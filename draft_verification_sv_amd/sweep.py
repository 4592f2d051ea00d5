"""Accepted draft length against target sampling temperature, for latent-mixture
drafts with K = 1 and K = 8 greedy branches and a category temperature ZT.

"Pith review of DBLAST", Figure 1 and "What carries the argument": accepted
length of block drafts as the entropy of the target sampling distribution
rises, and the latent mixture as the dependent proposal; "Assumptions & free
parameters": the inference category temperature ZT, picked from
{0, 0.2, ..., 1.4}.  Reading: ZT is the temperature of the category prior at
inference; the drafter draws z from softmax(mix / ZT) (ZT = 0: the argmax
category), and verification uses that same prior, so the caller hands libsv
the mixing logits mix / ZT (ZT = 0: 0 at the argmax and -inf elsewhere).

Synthetic analogue only: the rows are seeded Zipfian logits (synth), fixed for
every prefix, so no trained drafter or dataset is involved and the numbers do
not reproduce the pages' figures.  Every step runs the library's fused path
(sv_verify_rows, sv_accept_sample) under full verification (L_r = b); host
code here only prepares inputs and summarises outputs (mean accepted length,
mean target entropy over a row sample).

    python -m draft_verification_sv_amd.sweep [--V 151936] [--R 32] [--steps 8]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

TEMPS = (0.0, 0.5, 1.0, 1.5, 2.0)
ZTS = (0.0, 0.6, 1.0, 1.4)


def mix_at(mix: np.ndarray, ZT: float) -> np.ndarray:
    """Mixing logits of the category prior at temperature ZT."""
    mix = np.asarray(mix, np.float32)
    if ZT == 0.0:
        out = np.full_like(mix, -np.inf)
        out[np.arange(mix.shape[0]), np.argmax(mix, axis=1)] = 0.0
        return out
    return (mix / np.float32(ZT)).astype(np.float32)


def workload(K: int, ZT: float, *, V: int, R: int, steps: int, seed: int = 3000) -> synth.Workload:
    """Zipfian target rows (block 16, bf16), K greedy-branch components, the
    drafter's category drawn at ZT, no top-p, full verification.  The target
    rows depend on (V, R, seed) only, so every K sees the same ones (and K = 1's
    component is the first of K = 8's); the target temperature is set per run."""
    w = synth.make(f"sweep-K{K}-ZT{ZT:g}", R=R, V=V, K=K, T=1.0, steps=steps, seed=seed, vseed=7, cat_T=ZT)
    w.mix = mix_at(w.mix, ZT)
    return w


def verify_steps(w: synth.Workload, temps, device="cuda") -> dict:
    """Run every step of a full-verification mixture workload through libsv at
    each target temperature in `temps` (the same for every request); returns
    {T: [VerifyStep.results() per step]}."""
    import torch

    from .step import VerifyStep, row_pitch, to_device_rows

    R, b, V, K = w.R, w.b, w.V, w.K
    ld = row_pitch(V, w.dtype)
    vs = VerifyStep(R=R, b=b, V=V, dtype=w.dtype, K=K, device=device, diagnostics=True)
    tgt = to_device_rows(w.tgt, ld, device)   # L_r = b: the packed layout is every row in order
    comp = to_device_rows(w.comp, ld, device)
    out = {}
    for T in temps:
        out[T] = []
        for s in range(w.steps):
            vs.set_inputs(T=np.full(R, T, np.float32), x=w.x[s], seed=int(w.seeds[s]), top_p=w.top_p, mix=w.mix)
            vs.set_full_verification()
            vs.run_verify(tgt, ld, comp=comp, comp_ld=ld, fused=True)
            out[T].append(vs.results())
    del tgt, comp
    torch.cuda.synchronize()
    return out


def target_entropy(w: synth.Workload, T: float, rows: int = 64) -> float:
    """Mean entropy (nats) of softmax(l / T) over a sample of target rows."""
    vals = synth.values(w.tgt.reshape(-1, w.V)[:rows]).astype(np.float64)
    if T == 0.0:
        return 0.0
    z = vals / T
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return float(np.mean(-(p * np.log(np.where(p > 0, p, 1.0))).sum(axis=1)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--V", type=int, default=synth.QWEN3_VOCAB)
    ap.add_argument("--R", type=int, default=32)
    ap.add_argument("--steps", type=int, default=8)
    args = ap.parse_args()
    import torch

    torch.cuda.set_device(0)
    rows = []
    for K, zts in ((1, (0.0,)), (8, ZTS)):
        for ZT in zts:
            t0 = time.time()
            w = workload(K, ZT, V=args.V, R=args.R, steps=args.steps)
            res = verify_steps(w, TEMPS)
            for T in TEMPS:
                n_acc = np.stack([r["n_acc"] for r in res[T]])
                row = {"K": K, "ZT": ZT, "T": T, "target_entropy": round(target_entropy(w, T), 4),
                       "mean_accepted": round(float(n_acc.mean()), 4),
                       "mean_emitted": round(float(n_acc.mean()) + 1.0, 4),
                       "positions": int(n_acc.size * w.b)}
                print(json.dumps(row), flush=True)
                rows.append(row)
            print(f"[sweep] K={K} ZT={ZT:g}: {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    print("\n| K | ZT | T | target entropy (nats) | mean accepted | mean emitted |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['K']} | {r['ZT']:g} | {r['T']:g} | {r['target_entropy']:.3f} | {r['mean_accepted']:.3f} | "
              f"{r['mean_emitted']:.3f} |")


if __name__ == "__main__":
    main()
