"""CPU oracle for batched speculative-sampling verification (double precision).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never does, and the two share no code: this wrapper loads
``liboracle.so`` built from ``sv_oracle.c`` with plain gcc (no fast-math).

What each function computes, with the page and section it follows, is written
in ``sv_oracle.h`` / ``sv_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point this package at another build of the oracle (a copy with a
# planted mistake, to show that the pins catch it); it is never built here.
_LIB_OVERRIDE = os.environ.get("SV_ORACLE_LIB")

F32 = 0
BF16 = 1
Q_DENSE = 0
Q_MIXTURE = 1


def compile_command(src: str, out: str) -> list:
    return ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-fPIC", "-shared", "-o", out, src, "-lm"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc -O2 -fopenmp (IEEE double, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(compile_command(_SRC, tmp))
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None and _LIB_OVERRIDE:
        _lib = C.CDLL(_LIB_OVERRIDE)
        _declare(_lib)
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


ROW_STATS_DT = np.dtype(
    [("max", "f4"), ("argmax", "i4"), ("lse", "f8"), ("cut", "f4"), ("kept_lse", "f8"), ("margin", "f8")],
    align=True,
)


class _StepIn(C.Structure):
    _fields_ = [
        ("R", C.c_int32), ("b", C.c_int32), ("V", C.c_int32), ("K", C.c_int32),
        ("dtype", C.c_int32),
        ("tgt", C.c_void_p), ("tgt_ld", C.c_int64), ("tgt_row0", C.c_void_p),
        ("L", C.c_void_p), ("T", C.c_void_p), ("top_p", C.c_void_p), ("x", C.c_void_p),
        ("q_mode", C.c_int32),
        ("draft", C.c_void_p), ("draft_ld", C.c_int64), ("draft_row0", C.c_void_p),
        ("comp", C.c_void_p), ("comp_ld", C.c_int64), ("comp_row0", C.c_void_p),
        ("mix", C.c_void_p), ("branch_T", C.c_double), ("seed", C.c_uint64),
    ]


class _StepOut(C.Structure):
    _fields_ = [
        ("n_acc", C.c_void_p), ("token", C.c_void_p), ("is_bonus", C.c_void_p),
        ("sample_margin", C.c_void_p), ("u_res", C.c_void_p),
        ("u_acc", C.c_void_p), ("p_x", C.c_void_p), ("q_x", C.c_void_p), ("acc_margin", C.c_void_p),
        ("branch_tok", C.c_void_p), ("post_w", C.c_void_p),
    ]


class _TreeIn(C.Structure):
    _fields_ = [
        ("R", C.c_int32), ("b", C.c_int32), ("V", C.c_int32), ("dtype", C.c_int32),
        ("node_off", C.c_void_p), ("parent", C.c_void_p), ("token", C.c_void_p),
        ("tgt", C.c_void_p), ("tgt_ld", C.c_int64), ("tgt_row", C.c_void_p),
        ("T", C.c_void_p), ("top_p", C.c_void_p),
        ("draft", C.c_void_p), ("draft_ld", C.c_int64), ("draft_row0", C.c_void_p),
        ("seed", C.c_uint64),
    ]


class _TreeOut(C.Structure):
    _fields_ = [
        ("n_acc", C.c_void_p), ("path", C.c_void_p), ("stop_node", C.c_void_p), ("token", C.c_void_p),
        ("is_bonus", C.c_void_p), ("sample_margin", C.c_void_p), ("u_res", C.c_void_p),
        ("u_acc", C.c_void_p), ("p_x", C.c_void_p), ("q_x", C.c_void_p), ("acc_margin", C.c_void_p),
    ]


def _declare(L):
    vp, i32, i64, u64, dbl = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_double
    L.orc_philox4x32_10.argtypes = [vp, vp, vp]
    L.orc_philox4x32_10.restype = None
    L.orc_u24.argtypes = [C.c_uint32]
    L.orc_u24.restype = dbl
    L.orc_uniform_words.argtypes = [u64, i32, i32, vp]
    L.orc_uniform_words.restype = None
    L.orc_dvl.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    L.orc_dvl.restype = C.c_int
    L.orc_dvl_ragged.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp, vp]
    L.orc_dvl_ragged.restype = C.c_int
    L.orc_dvl_objective.argtypes = [vp, vp, i32, i32]
    L.orc_dvl_objective.restype = dbl
    L.orc_row_stats.argtypes = [vp, i32, i32, dbl, dbl, vp]
    L.orc_row_stats.restype = None
    L.orc_row_stats_batch.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp, vp]
    L.orc_row_stats_batch.restype = None
    L.orc_argmax_rows.argtypes = [vp, i32, i64, i32, i32, vp]
    L.orc_argmax_rows.restype = None
    L.orc_step.argtypes = [C.POINTER(_StepIn), C.POINTER(_StepOut)]
    L.orc_step.restype = C.c_int
    L.orc_tree_step.argtypes = [C.POINTER(_TreeIn), C.POINTER(_TreeOut)]
    L.orc_tree_step.restype = C.c_int
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = C.c_int
    L.orc_set_num_threads.argtypes = [C.c_int]
    L.orc_set_num_threads.restype = None


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _rows_dtype(rows):
    if rows.dtype == np.float32:
        return F32
    if rows.dtype == np.uint16:
        return BF16
    raise TypeError("logit rows must be float32 or uint16 (bf16 bits)")


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- Philox
def philox4x32_10(ctr, key) -> np.ndarray:
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def u24(w: int) -> float:
    return float(lib().orc_u24(int(w) & 0xFFFFFFFF))


def uniform_words(seed: int, R: int, n_pos: int) -> np.ndarray:
    out = np.zeros((R, n_pos, 4), np.uint32)
    lib().orc_uniform_words(int(seed) & (2**64 - 1), R, n_pos, _ptr(out))
    return out


# ---------------------------------------------------------------- DVL
def dvl(a, budget: int, block_len=None) -> dict:
    """DVL allocation of survival estimates a [R, b] under `budget`; with
    `block_len` [R], request r drafted only its first block_len[r] positions."""
    a = _c(a, np.float32)
    R, b = a.shape
    s = np.zeros((R, b), np.float32)
    Lr = np.zeros(R, np.int32)
    pos_off = np.zeros(R + 1, np.int32)
    tgt_off = np.zeros(R + 1, np.int32)
    bl = None if block_len is None else _c(block_len, np.int32)
    bad = lib().orc_dvl_ragged(_ptr(a), R, b, _ptr(bl), int(budget), _ptr(s), _ptr(Lr), _ptr(pos_off),
                               _ptr(tgt_off))
    if bad == 2:
        raise ValueError("block_len outside [0, b]")
    return {"s": s, "L": Lr, "pos_off": pos_off, "tgt_off": tgt_off, "bad": int(bad)}


def dvl_objective(s, Lr) -> float:
    s = _c(s, np.float32)
    Lr = _c(Lr, np.int32)
    R, b = s.shape
    return float(lib().orc_dvl_objective(_ptr(s), _ptr(Lr), R, b))


# ---------------------------------------------------------------- rows
def row_stats(row, T: float, top_p: float = 1.0) -> np.void:
    row = np.ascontiguousarray(row)
    out = np.zeros(1, ROW_STATS_DT)
    lib().orc_row_stats(_ptr(row), _rows_dtype(row), row.shape[-1], float(T), float(top_p), _ptr(out))
    return out[0]


def row_stats_batch(rows, req, T, top_p=None) -> np.ndarray:
    """Statistics of rows[k] at temperature T[req[k]] and top_p[req[k]]."""
    rows = np.ascontiguousarray(rows)
    n, V = rows.shape
    req = _c(req, np.int32)
    T = _c(T, np.float32)
    tp = None if top_p is None else _c(top_p, np.float32)
    out = np.zeros(n, ROW_STATS_DT)
    lib().orc_row_stats_batch(_ptr(rows), _rows_dtype(rows), V, V, n, _ptr(req), _ptr(T), _ptr(tp), _ptr(out))
    return out


def argmax_rows(rows) -> np.ndarray:
    rows = np.ascontiguousarray(rows)
    shape = rows.shape
    flat = rows.reshape(-1, shape[-1])
    out = np.zeros(flat.shape[0], np.int32)
    lib().orc_argmax_rows(_ptr(flat), _rows_dtype(flat), shape[-1], shape[-1], flat.shape[0], _ptr(out))
    return out.reshape(shape[:-1])


# ---------------------------------------------------------------- step
def step(*, tgt, tgt_row0, L, T, x, seed, top_p=None, draft=None, draft_row0=None,
         comp=None, comp_row0=None, mix=None, branch_T: float = 0.0) -> dict:
    """One verification step over R requests.

    tgt:   [rows, V] target logit rows (float32 or uint16 bf16 bits); request r
           uses rows tgt_row0[r] .. tgt_row0[r] + L[r].
    x:     [R, b] draft tokens.  Dense mode when ``draft`` is given (row of
           position i of r: draft_row0[r] + i); mixture mode when ``comp`` is
           given (row of branch z, position i: comp_row0[r] + z*b + i) with
           mixing logits mix [R, K].
    """
    tgt = np.ascontiguousarray(tgt)
    dt = _rows_dtype(tgt)
    x = _c(x, np.int32)
    R, b = x.shape
    V = tgt.shape[-1]
    Lr = _c(L, np.int32)
    Tr = _c(T, np.float32)
    tp = None if top_p is None else _c(top_p, np.float32)
    t0 = _c(tgt_row0, np.int64)
    si = _StepIn()
    si.R, si.b, si.V, si.dtype = R, b, V, dt
    si.tgt, si.tgt_ld, si.tgt_row0 = _ptr(tgt), V, _ptr(t0)
    si.L, si.T, si.top_p, si.x = _ptr(Lr), _ptr(Tr), _ptr(tp), _ptr(x)
    keep = [tgt, x, Lr, Tr, tp, t0]
    K = 0
    if comp is not None:
        comp = np.ascontiguousarray(comp)
        assert _rows_dtype(comp) == dt
        mix = _c(mix, np.float32)
        K = mix.shape[1]
        c0 = _c(comp_row0, np.int64)
        si.q_mode = Q_MIXTURE
        si.comp, si.comp_ld, si.comp_row0 = _ptr(comp), comp.shape[-1], _ptr(c0)
        si.mix, si.branch_T = _ptr(mix), float(branch_T)
        keep += [comp, mix, c0]
    else:
        draft = np.ascontiguousarray(draft)
        assert _rows_dtype(draft) == dt
        d0 = _c(draft_row0, np.int64)
        si.q_mode = Q_DENSE
        si.draft, si.draft_ld, si.draft_row0 = _ptr(draft), draft.shape[-1], _ptr(d0)
        keep += [draft, d0]
    si.K = K
    si.seed = int(seed) & (2**64 - 1)
    out = {
        "n_acc": np.zeros(R, np.int32), "token": np.zeros(R, np.int32), "is_bonus": np.zeros(R, np.int32),
        "sample_margin": np.zeros(R), "u_res": np.zeros(R),
        "u_acc": np.full((R, b), np.nan), "p_x": np.full((R, b), np.nan),
        "q_x": np.full((R, b), np.nan), "acc_margin": np.full((R, b), np.nan),
    }
    so = _StepOut()
    for k in ("n_acc", "token", "is_bonus", "sample_margin", "u_res", "u_acc", "p_x", "q_x", "acc_margin"):
        setattr(so, k, _ptr(out[k]))
    if K:
        out["branch_tok"] = np.full((R, K, b), -1, np.int32)
        out["post_w"] = np.full((R, b, K), np.nan)
        so.branch_tok, so.post_w = _ptr(out["branch_tok"]), _ptr(out["post_w"])
    rc = lib().orc_step(C.byref(si), C.byref(so))
    if rc != 0:
        raise ValueError(f"orc_step rejected its input (code {rc})")
    del keep
    return out


# ---------------------------------------------------------------- tree verification
def tree_step(*, tgt, tgt_row, node_off, parent, token, T, b, seed, draft, draft_row0, top_p=None) -> dict:
    """Tree verification of R requests (orc_tree_step).

    node_off: [R+1] exclusive scan of the node counts; parent, token, tgt_row:
    one entry per node (request r's nodes at node_off[r] + j, j = 0 the root,
    parent -1); tgt: [rows, V] target rows (row tgt_row[k] for node k); draft:
    [rows, V] with the children of a depth-d node of request r drawn from row
    draft_row0[r] + d.  Per-node outputs are NaN for nodes never tested."""
    tgt = np.ascontiguousarray(tgt)
    dt = _rows_dtype(tgt)
    draft = np.ascontiguousarray(draft)
    assert _rows_dtype(draft) == dt
    node_off = _c(node_off, np.int32)
    R = len(node_off) - 1
    n = int(node_off[-1])
    par, tok = _c(parent, np.int32), _c(token, np.int32)
    trow, d0 = _c(tgt_row, np.int64), _c(draft_row0, np.int64)
    Tr = _c(np.broadcast_to(np.asarray(T, np.float32), (R,)), np.float32)
    tp = None if top_p is None else _c(np.broadcast_to(np.asarray(top_p, np.float32), (R,)), np.float32)
    ti = _TreeIn()
    ti.R, ti.b, ti.V, ti.dtype = R, int(b), tgt.shape[-1], dt
    ti.node_off, ti.parent, ti.token = _ptr(node_off), _ptr(par), _ptr(tok)
    ti.tgt, ti.tgt_ld, ti.tgt_row = _ptr(tgt), tgt.shape[-1], _ptr(trow)
    ti.T, ti.top_p = _ptr(Tr), _ptr(tp)
    ti.draft, ti.draft_ld, ti.draft_row0 = _ptr(draft), draft.shape[-1], _ptr(d0)
    ti.seed = int(seed) & (2**64 - 1)
    out = {"n_acc": np.zeros(R, np.int32), "path": np.full((R, int(b)), -1, np.int32),
           "stop_node": np.zeros(R, np.int32), "token": np.zeros(R, np.int32), "is_bonus": np.zeros(R, np.int32),
           "sample_margin": np.zeros(R), "u_res": np.zeros(R),
           "u_acc": np.full(n, np.nan), "p_x": np.full(n, np.nan), "q_x": np.full(n, np.nan),
           "acc_margin": np.full(n, np.nan)}
    to = _TreeOut()
    for k in out:
        setattr(to, k, _ptr(out[k]))
    keep = [tgt, draft, node_off, par, tok, trow, d0, Tr, tp]
    rc = lib().orc_tree_step(C.byref(ti), C.byref(to))
    del keep
    if rc != 0:
        raise ValueError(f"orc_tree_step rejected its input (code {rc})")
    return out
