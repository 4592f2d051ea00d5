"""Seeded synthetic inputs for the verification workloads.

This module is shared by the GPU tests, the benchmark and the oracle tests.
It holds none of the verification arithmetic: it draws logits, survival
scores, mixing logits and the drafter's own samples (the draft tokens), and
packs target rows for a given allocation (the stand-in for the target
forward, which is outside the verification path).

Workload recipes (shapes and regimes of the pages' workloads; the pages'
datasets and models are not used):
  * Qwen3 vocabulary V = 151936, concurrency 8-32, block 16
    (DScale abstract: concurrency 8-32 on Qwen3-4B/8B).
  * target logits: Zipfian base -1.1*ln(rank) over a seeded permutation of
    the vocabulary per row, plus N(0, 1) noise; bf16 (round to nearest even).
  * independent draft: target + N(0, sigma^2); draft token sampled from
    softmax(draft / T) (Gumbel-max), argmax at T = 0.
  * latent mixture (DBLast review, "What carries the argument"): K component
    rows per position = the target row's Zipfian base + N(0, 1.5^2); mixing
    logits N(0, 1); the drafter samples z ~ softmax(mixing logits)
    (Gumbel-max) and decodes branch z greedily (argmax of the stored values),
    or, with a branch temperature T_b > 0, samples every position of branch z
    from softmax(c / T_b) (Gumbel-max).
  * survival estimates a ~ Beta(8, 2) per position for DVL.
All randomness comes from numpy Generators seeded from SeedSequence(seed);
work is split per request with spawned child sequences, so the output does
not depend on the number of threads.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from typing import Optional

import numpy as np

QWEN3_VOCAB = 151936


# ------------------------------------------------------------ bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def values(a: np.ndarray) -> np.ndarray:
    """Exact float32 values of a stored logit array (float32 or bf16 bits)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


# ------------------------------------------------------------ workload
@dataclasses.dataclass
class Workload:
    name: str
    R: int
    b: int
    V: int
    K: int                      # 0: independent draft
    dtype: str                  # "f32" or "bf16"
    tgt: np.ndarray             # [R, b+1, V] target rows for every position (+ bonus row)
    draft: Optional[np.ndarray]  # [R, b, V] dense draft rows (independent mode)
    comp: Optional[np.ndarray]   # [R, K, b, V] component rows (mixture mode)
    mix: Optional[np.ndarray]    # [R, K] mixing logits (float32)
    T: np.ndarray               # [R] float32
    top_p: Optional[np.ndarray]  # [R] float32 or None (off)
    budget: Optional[int]        # DVL budget or None (full verification)
    a: Optional[np.ndarray]      # [S, R, b] survival estimates per step
    x: np.ndarray               # [S, R, b] draft tokens per step
    seeds: np.ndarray           # [S] uint64 verification seeds
    branch_tok: Optional[np.ndarray] = None  # [R, K, b] drafter's greedy branch tokens
    branch_T: float = 0.0       # mixture branches: 0 greedy; > 0 sampled from softmax(c / branch_T)
    block_len: Optional[np.ndarray] = None  # [R] drafted positions per request (None: b for every request)

    @property
    def steps(self) -> int:
        return int(self.x.shape[0])


def _pool_map(fn, items, threads):
    if threads <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def _default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _zipf_base(rng: np.random.Generator, nrows: int, V: int, logtab: np.ndarray) -> np.ndarray:
    ranks = np.tile(np.arange(V, dtype=np.int32), (nrows, 1))
    rng.permuted(ranks, axis=1, out=ranks)
    return logtab[ranks]


def _gumbel_argmax(rng, logits: np.ndarray, T: float) -> np.ndarray:
    """The drafter's own sample from softmax(logits / T) over the last axis."""
    lg = np.asarray(logits, dtype=np.float64)
    if T == 0.0:
        return np.argmax(lg, axis=-1).astype(np.int32)
    g = -np.log(-np.log(rng.random(lg.shape)))
    return np.argmax(lg / T + g, axis=-1).astype(np.int32)


def make(name: str, *, R: int, b: int = 16, V: int = QWEN3_VOCAB, K: int = 0, dtype: str = "bf16",
         target: str = "zipf", draft_sigma: float = 1.0, comp_sigma: float = 1.5,
         T=1.0, top_p: Optional[float] = None, budget: Optional[int] = None, steps: int = 1,
         seed: int = 1000, vseed: int = 1, threads: Optional[int] = None, branch_T: float = 0.0,
         cat_T: float = 1.0) -> Workload:
    """Draw one workload.  ``target`` is "zipf" (Zipfian base + N(0,1)) or
    "normal2" (N(0, 2^2)); ``K`` > 0 selects the latent-mixture drafter, whose
    branches decode greedily (``branch_T`` = 0) or sample from
    softmax(c / branch_T); its category is drawn from softmax(mix / cat_T)
    (``cat_T`` = 0: the argmax category)."""
    threads = threads or _default_threads()
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(R + 1)
    Tr = np.broadcast_to(np.asarray(T, dtype=np.float32), (R,)).copy()
    logtab = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    store = f32_to_bf16_bits if dtype == "bf16" else (lambda v: np.asarray(v, np.float32))

    def per_request(r):
        rng = np.random.default_rng(kids[r])
        if target == "zipf":
            base = _zipf_base(rng, b + 1, V, logtab)
            tgt = base + rng.standard_normal((b + 1, V), dtype=np.float32)
        elif target == "normal2":
            base = None
            tgt = 2.0 * rng.standard_normal((b + 1, V), dtype=np.float32)
        else:
            raise ValueError(target)
        tgt_s = store(tgt)
        tv = values(tgt_s)
        draft_s = comp_s = None
        if K == 0:
            draft_s = store(tv[:b] + np.float32(draft_sigma) * rng.standard_normal((b, V), dtype=np.float32))
        else:
            src = base[:b] if base is not None else tv[:b]
            comp_s = np.empty((K, b, V), dtype=tgt_s.dtype)
            for z in range(K):
                comp_s[z] = store(src + np.float32(comp_sigma) * rng.standard_normal((b, V), dtype=np.float32))
        return tgt_s, draft_s, comp_s

    parts = _pool_map(per_request, list(range(R)), threads)
    tgt = np.stack([p[0] for p in parts])
    draft = np.stack([p[1] for p in parts]) if K == 0 else None
    comp = np.stack([p[2] for p in parts]) if K > 0 else None
    del parts

    rng = np.random.default_rng(kids[R])
    seeds = np.arange(steps, dtype=np.uint64) + np.uint64(vseed)
    a = rng.beta(8.0, 2.0, size=(steps, R, b)).astype(np.float32) if budget is not None else None
    mix = None
    branch_tok = None
    if K == 0:
        dv = values(draft)
        x = np.empty((steps, R, b), np.int32)
        for s in range(steps):
            for r in range(R):
                x[s, r] = _gumbel_argmax(rng, dv[r], float(Tr[r]))
    else:
        mix = rng.standard_normal((R, K)).astype(np.float32)
        # the drafter's greedy decode of every branch (argmax of stored values)
        branch_tok = np.stack(
            _pool_map(lambda r: np.argmax(values(comp[r]), axis=-1).astype(np.int32), list(range(R)), threads)
        )
        x = np.empty((steps, R, b), np.int32)
        for s in range(steps):
            zs = _gumbel_argmax(rng, mix, cat_T)
            if branch_T == 0.0:
                x[s] = branch_tok[np.arange(R), zs]
            else:  # the drafter samples every position of the chosen branch
                for r in range(R):
                    x[s, r] = _gumbel_argmax(rng, values(comp[r, zs[r]]), branch_T)
    tp = None if top_p is None else np.full(R, top_p, np.float32)
    return Workload(name=name, R=R, b=b, V=V, K=K, dtype=dtype, tgt=tgt, draft=draft, comp=comp, mix=mix,
                    T=Tr, top_p=tp, budget=budget, a=a, x=x, seeds=seeds, branch_tok=branch_tok,
                    branch_T=float(branch_T))


# ------------------------------------------------------------ the five workloads
def config(c: int, *, V: Optional[int] = None, R: Optional[int] = None, steps: Optional[int] = None,
           threads: Optional[int] = None, branch_T: float = 0.0, ragged: bool = False) -> Workload:
    """Workload c = 1..5 (sizes may be shrunk for quick parity cases).  For the
    mixture workloads (4, 5) ``branch_T`` > 0 gives the soft-branch drafter.
    ``ragged`` gives every request its own block length b_r, uniform on
    0..b (seeded), of which only the first b_r drafted positions count."""
    if branch_T and c not in (4, 5):
        raise ValueError("branch_T applies to the mixture workloads 4 and 5")
    w = _config(c, V=V, R=R, steps=steps, threads=threads, branch_T=branch_T)
    if ragged:
        rng = np.random.default_rng(np.random.SeedSequence([2000 + c, w.R]))
        w.block_len = rng.integers(0, w.b + 1, size=w.R).astype(np.int32)
        w.name += "-ragged"
    return w


def _config(c: int, *, V, R, steps, threads, branch_T) -> Workload:
    soft = f"-softTb{branch_T:g}" if branch_T else ""
    if c == 1:
        R_ = R or 4
        T = np.ones(R_, np.float32)
        T[-1] = 0.0  # last request greedy
        return make("cfg1-tiny-f32", R=R_, V=V or 1024, dtype="f32", target="normal2", draft_sigma=0.5,
                    T=T, seed=1001, vseed=1, steps=steps or 1, threads=threads)
    if c == 2:
        return make("cfg2-conc8-indep", R=R or 8, V=V or QWEN3_VOCAB, T=1.0, seed=1002, vseed=2,
                    steps=steps or 1, threads=threads)
    if c == 3:
        R_ = R or 32
        return make("cfg3-conc32-dvl-indep", R=R_, V=V or QWEN3_VOCAB, T=1.0, budget=R_ * 16 // 2,
                    seed=1003, vseed=3, steps=steps or 1, threads=threads)
    if c == 4:
        return make("cfg4-conc16-mix8-T1.5-topp" + soft, R=R or 16, V=V or QWEN3_VOCAB, K=8, T=1.5, top_p=0.95,
                    seed=1004, vseed=4, steps=steps or 1, threads=threads, branch_T=branch_T)
    if c == 5:
        R_ = R or 32
        return make("cfg5-conc32-dvl-mix8-topp" + soft, R=R_, V=V or QWEN3_VOCAB, K=8, T=1.0, top_p=0.95,
                    budget=R_ * 16 // 2, seed=1005, vseed=5, steps=200 if steps is None else steps,
                    threads=threads, branch_T=branch_T)
    raise ValueError(c)


def pack_target(w: Workload, L: np.ndarray) -> np.ndarray:
    """Target rows as the target forward would emit them for allocation L:
    request r contributes its first L[r] + 1 rows, requests in order."""
    return np.concatenate([w.tgt[r, : int(L[r]) + 1] for r in range(w.R)], axis=0)


# ------------------------------------------------------------ draft trees
@dataclasses.dataclass
class TreeWorkload:
    name: str
    R: int
    b: int                      # depth limit (draft positions)
    V: int
    dtype: str
    max_kids: int               # most children of any node
    node_off: np.ndarray        # [R+1] int32 exclusive scan of the node counts
    parent: np.ndarray          # [n] int32 local parent index (-1 for each root)
    token: np.ndarray           # [n] int32 draft token of each node (0 for the roots)
    depth: np.ndarray           # [n] int32
    tgt: np.ndarray             # [n, V] target row of every node (stored dtype)
    draft: np.ndarray           # [R, b, V] the drafter's row per depth (stored dtype)
    T: np.ndarray               # [R] float32
    top_p: Optional[np.ndarray]  # [R] float32 or None
    seed: int                   # verification seed


def tree(name: str, *, R: int, b: int = 16, V: int = QWEN3_VOCAB, width: int = 4, nodes: int = 64,
         dtype: str = "bf16", T=1.0, top_p: Optional[float] = None, shape: str = "random",
         draft_sigma: float = 1.0, seed: int = 3000, vseed: int = 11, threads: Optional[int] = None,
         fill: bool = False) -> TreeWorkload:
    """Draft trees per request (the budget-aware trees of tree drafters).

    ``shape`` "random": a node budget N_r uniform on 1..``nodes``; nodes are
    expanded breadth-first (so every parent precedes its children), the root
    with 1..``width`` children and every other node with 0..``width``, within
    depth b and the budget.  "chain": a chain of L_r uniform on 0..b draft
    nodes.  "wide": the root alone with ``width`` children (the multi-candidate
    case at its simplest).
    Target row of a node at depth d: the request's Zipfian base for position d
    plus N(0, 1) noise of the node's own (a target's rows depend on the path).
    Drafter row d: that base plus N(0, ``draft_sigma``^2); the children of a
    depth-d node are independent samples of softmax(draft row d / T_r)
    (Gumbel-max), its argmax at T_r = 0.  ``fill``: every request's tree has
    exactly ``nodes`` nodes (each node below depth b gets 1..``width``
    children until the budget is spent)."""
    threads = threads or _default_threads()
    ss = np.random.SeedSequence([seed, R, b, V, width, nodes])
    kids_ss = ss.spawn(R)
    Tr = np.broadcast_to(np.asarray(T, dtype=np.float32), (R,)).copy()
    logtab = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    store = f32_to_bf16_bits if dtype == "bf16" else (lambda v: np.asarray(v, np.float32))

    def shape_of(rng):
        if shape == "chain":
            L = int(rng.integers(0, b + 1))
            return [-1] + list(range(L)), [0] + list(range(1, L + 1))
        if shape == "wide":
            return [-1] + [0] * width, [0] + [1] * width
        if shape != "random":
            raise ValueError(shape)
        budget = nodes if fill else int(rng.integers(1, nodes + 1))
        par, dep = [-1], [0]
        u = 0
        while u < len(par) and len(par) < budget:
            if dep[u] < b:
                k = int(rng.integers(1 if (u == 0 or fill) else 0, width + 1))
                for _ in range(min(k, budget - len(par))):
                    par.append(u)
                    dep.append(dep[u] + 1)
            u += 1
        return par, dep

    def per_request(r):
        rng = np.random.default_rng(kids_ss[r])
        par, dep = shape_of(rng)
        base = _zipf_base(rng, b + 1, V, logtab)
        d = np.asarray(dep)
        tgt = store(base[d] + rng.standard_normal((len(par), V), dtype=np.float32))
        draft = store(base[:b] + np.float32(draft_sigma) * rng.standard_normal((b, V), dtype=np.float32))
        dv = values(draft)
        tok = np.zeros(len(par), np.int32)
        for j in range(1, len(par)):
            tok[j] = _gumbel_argmax(rng, dv[dep[par[j]]], float(Tr[r]))
        return np.asarray(par, np.int32), d.astype(np.int32), tok, tgt, draft

    parts = _pool_map(per_request, list(range(R)), threads)
    node_off = np.concatenate([[0], np.cumsum([len(p[0]) for p in parts])]).astype(np.int32)
    parent = np.concatenate([p[0] for p in parts])
    kidc = max(int(np.bincount(p[0][1:], minlength=1).max()) if len(p[0]) > 1 else 0 for p in parts)
    tp = None if top_p is None else np.full(R, top_p, np.float32)
    return TreeWorkload(name=name, R=R, b=b, V=V, dtype=dtype, max_kids=max(1, kidc), node_off=node_off,
                        parent=parent, token=np.concatenate([p[2] for p in parts]),
                        depth=np.concatenate([p[1] for p in parts]), tgt=np.concatenate([p[3] for p in parts]),
                        draft=np.stack([p[4] for p in parts]), T=Tr, top_p=tp, seed=int(vseed))
