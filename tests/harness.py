"""Parity harness: run one verification step through libsv and through the
oracle on the same seeded inputs, and compare them.

Comparison rule: Philox uniforms, DVL scores/lengths/offsets, argmax indices,
row maxima and branch tokens exactly; log-sum-exp, kept mass and p, q at the
draft tokens within 1e-5 relative; accepted lengths, residual and bonus
tokens exactly, except a mismatch whose oracle decision margin is below 1e-6
(after a request's first mismatch its later decisions are not compared); such
mismatches must number fewer than 1e-4 of the verified positions.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

REL = 1e-5
MARGIN = 1e-6

# One line per long parity run (positions compared, excused disagreements),
# printed in pytest's terminal summary by conftest.py.
PARITY_LOG: list = []


def log_parity(name: str, rep: dict):
    line = (f"{name}: {rep['positions']} positions, {rep['mismatches']} excused decision mismatches "
            f"{[tuple(x) for x in rep['low_margin']]}, {rep['cut_diff']} excused top-p cut differences")
    PARITY_LOG.append(line)
    print(f"[parity] {line}", flush=True)


def gpu_step_runner(w: synth.Workload, device="cuda", two_streams: bool = False, fused: bool = False):
    """Upload a workload once and return (VerifyStep, run(s) -> results)."""
    import torch

    from draft_verification_sv_amd.step import VerifyStep, pack_rows_device, row_pitch, to_device_rows

    R, b, V, K = w.R, w.b, w.V, w.K
    ld = row_pitch(V, w.dtype)
    max_pos = min(w.budget, R * b) if w.budget is not None else R * b
    soft = bool(np.any(np.asarray(w.branch_T) > 0))
    if soft:
        fused = True  # soft branches run on the fused calls
    vs = VerifyStep(R=R, b=b, V=V, dtype=w.dtype, K=K, max_pos=max_pos, device=device, diagnostics=True,
                    soft_branches=soft, ragged=w.block_len is not None)
    full = to_device_rows(w.tgt, ld, device)  # [R*(b+1), ld]
    packed = torch.empty_like(full)
    draft = to_device_rows(w.draft, ld, device) if K == 0 else None
    comp = to_device_rows(w.comp, ld, device) if K > 0 else None
    side = torch.cuda.Stream() if two_streams else None

    def run(s: int, L=None) -> dict:
        """Step s; with ``L`` the verified lengths (and their exclusive-scan
        offsets) are written by the caller instead of DVL or full verification."""
        vs.set_inputs(T=w.T, x=w.x[s], seed=int(w.seeds[s]), top_p=w.top_p, mix=w.mix,
                      a=None if w.a is None else w.a[s], budget=w.budget,
                      branch_T=w.branch_T if soft else None, block_len=w.block_len)
        if L is not None:
            L = np.asarray(L, np.int32)
            vs.L.copy_(torch.from_numpy(L))
            vs.pos_off.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(L)]).astype(np.int32)))
            vs.tgt_off.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)))
        elif w.budget is not None:
            vs.run_dvl()
            L = vs.L.cpu().numpy()
        else:
            vs.set_full_verification()
            L = np.full(R, b, np.int32) if w.block_len is None else w.block_len.copy()
        pack_rows_device(full, L, b + 1, packed)
        vs.run_verify(packed, ld, draft=draft, draft_ld=ld, comp=comp, comp_ld=ld, side_stream=side, fused=fused)
        vs.last_rows = (packed, draft if K == 0 else comp)
        return vs.results()

    return vs, run


def gpu_graph_runner(w: synth.Workload, device="cuda"):
    """The whole step captured once as a HIP graph over fixed-address buffers:
    dvl_alloc_pack (with a budget), a device-side packing of the target rows
    by the new offsets (the target forward's stand-in), and the fused
    verification calls.  Returns (VerifyStep, graph, run(s) -> results), where
    run(s) writes step s's inputs to the fixed addresses eagerly and replays."""
    import torch

    from draft_verification_sv_amd.step import (VerifyStep, capture_graph, pack_rows_by_offsets, row_pitch,
                                                to_device_rows)

    R, b, V, K = w.R, w.b, w.V, w.K
    ld = row_pitch(V, w.dtype)
    max_pos = min(w.budget, R * b) if w.budget is not None else R * b
    soft = bool(np.any(np.asarray(w.branch_T) > 0))
    vs = VerifyStep(R=R, b=b, V=V, dtype=w.dtype, K=K, max_pos=max_pos, device=device, diagnostics=True,
                    soft_branches=soft, ragged=w.block_len is not None)
    full = to_device_rows(w.tgt, ld, device)
    packed = torch.empty((vs.max_rows, ld), dtype=full.dtype, device=device)
    slots = torch.arange(vs.max_rows, dtype=torch.int32, device=device)
    draft = to_device_rows(w.draft, ld, device) if K == 0 else None
    comp = to_device_rows(w.comp, ld, device) if K > 0 else None

    def set_step(s: int):
        vs.set_inputs(T=w.T, x=w.x[s], seed=int(w.seeds[s]), top_p=w.top_p, mix=w.mix,
                      a=None if w.a is None else w.a[s], budget=w.budget,
                      branch_T=w.branch_T if soft else None, block_len=w.block_len)
        if w.budget is None:
            vs.set_full_verification()

    def body():
        if w.budget is not None:
            vs.run_dvl()
        pack_rows_by_offsets(full, vs.tgt_off, b + 1, packed, slots)
        vs.run_verify(packed, ld, draft=draft, draft_ld=ld, comp=comp, comp_ld=ld, fused=True)

    set_step(0)
    graph = capture_graph(body)

    def run(s: int) -> dict:
        set_step(s)
        graph.replay()
        return vs.results()

    return vs, graph, run


def oracle_step(w: synth.Workload, s: int, row_cache: dict | None = None, L: np.ndarray | None = None) -> dict:
    """The oracle's step s of workload w.  ``row_cache`` (optional, one dict
    per workload whose logits, temperatures and top-p values stay fixed)
    keeps the statistics of each target row once computed, for long runs in
    which every step re-reads the same rows.  ``L`` (optional) takes these
    verified lengths instead of the oracle's DVL allocation."""
    R, b, V, K = w.R, w.b, w.V, w.K
    if L is not None:
        L = np.asarray(L, np.int32)
        dv = {"L": L, "s": None, "pos_off": np.concatenate([[0], np.cumsum(L)]).astype(np.int32),
              "tgt_off": np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)}
    elif w.budget is not None:
        dv = oracle.dvl(w.a[s], w.budget, block_len=w.block_len)
    else:
        L = np.full(R, b, np.int32) if w.block_len is None else w.block_len.astype(np.int32)
        dv = {"L": L, "s": None, "pos_off": np.concatenate([[0], np.cumsum(L)]).astype(np.int32),
              "tgt_off": np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)}
    L = dv["L"]
    tgt = w.tgt.reshape(R * (b + 1), V)
    common = dict(tgt=tgt, tgt_row0=np.arange(R) * (b + 1), L=L, T=w.T, x=w.x[s], seed=int(w.seeds[s]),
                  top_p=w.top_p)
    if K == 0:
        out = oracle.step(**common, draft=w.draft.reshape(R * b, V), draft_row0=np.arange(R) * b)
    else:
        # the oracle takes one branch temperature; requests are independent, so a
        # per-request T_b is one oracle run per distinct value, merged by request
        bT = np.broadcast_to(np.asarray(w.branch_T, np.float64), (R,))
        runs = {float(t): oracle.step(**common, comp=w.comp.reshape(R * K * b, V), comp_row0=np.arange(R) * K * b,
                                      mix=w.mix, branch_T=float(t)) for t in np.unique(bT)}
        out = {k: np.stack([runs[float(bT[r])][k][r] for r in range(R)]) for k in runs[float(bT[0])]}
    out["dvl"] = dv
    # statistics of every target row read in this step, in packed order
    rows = np.concatenate([r * (b + 1) + np.arange(L[r] + 1) for r in range(R)])
    req = np.repeat(np.arange(R), L + 1)
    if row_cache is None:
        out["rows"] = oracle.row_stats_batch(tgt[rows], req, w.T, w.top_p)
    else:
        miss = np.array([k for k in rows if k not in row_cache], np.int64)
        if len(miss):
            st = oracle.row_stats_batch(tgt[miss], miss // (b + 1), w.T, w.top_p)
            row_cache.update(zip(miss.tolist(), st))
        out["rows"] = np.array([row_cache[k] for k in rows.tolist()], dtype=oracle.ROW_STATS_DT)
    if K == 0:
        drows = np.concatenate([r * b + np.arange(L[r]) for r in range(R)]).astype(np.int64)
        dreq = np.repeat(np.arange(R), L)
        out["drows"] = oracle.row_stats_batch(w.draft.reshape(R * b, V)[drows], dreq, w.T, None)
    return out


def _rel_close(a, b, rel=REL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = (a == b)
    return same_inf | (np.abs(a - b) <= rel * np.maximum(np.abs(b), 1e-300))


def compare_step(w: synth.Workload, g: dict, o: dict, report: dict | None = None, skip=(), offsets: bool = True) -> dict:
    """Compare one step; returns counters and raises AssertionError on a violation.
    ``skip``: requests left out of the comparison (inputs the step flags as
    malformed, whose outputs are unspecified); their packed rows, positions and
    decisions are not compared.  ``offsets=False``: the GPU's offsets were
    written by the caller (not computed), and only the oracle's lengths of the
    compared requests are checked against them."""
    R, b = w.R, w.b
    rep = report if report is not None else {"positions": 0, "mismatches": 0, "low_margin": [], "cut_diff": 0}
    dv = o["dvl"]
    L = dv["L"]
    keep = np.array([r not in set(skip) for r in range(R)])
    if offsets:
        # DVL: bit-exact
        assert np.array_equal(g["L"], L), "DVL lengths differ"
        assert np.array_equal(g["pos_off"], dv["pos_off"]), "pos_off differs"
        assert np.array_equal(g["tgt_off"], dv["tgt_off"]), "tgt_off differs"
        if dv["s"] is not None:
            assert np.array_equal(g["s"].view(np.uint32), dv["s"].reshape(-1).view(np.uint32)), "DVL scores differ"
    return _compare_kept(w, g, o, rep, keep)


def _compare_kept(w, g, o, rep, keep):
    R, b = w.R, w.b
    dv = o["dvl"]
    L = dv["L"]
    # packed rows of the compared requests, in the GPU's and the oracle's packing
    gto = np.asarray(g["tgt_off"])
    gpo = np.asarray(g["pos_off"])
    grows = np.concatenate([np.arange(gto[r], gto[r] + L[r] + 1) for r in range(R) if keep[r]] or [np.zeros(0, int)])
    orows = np.concatenate([np.arange(dv["tgt_off"][r], dv["tgt_off"][r] + L[r] + 1) for r in range(R) if keep[r]]
                           or [np.zeros(0, int)])
    for r in range(R):
        if keep[r]:
            assert int(gpo[r + 1] - gpo[r]) == int(L[r]), f"verified length of request {r} differs"
    rows = o["rows"][orows]
    sel = lambda x: np.asarray(x)[grows]  # noqa: E731
    # target row statistics
    assert np.array_equal(sel(g["row_max"]), rows["max"]), "row max differs"
    assert np.array_equal(sel(g["row_argmax"]), rows["argmax"]), "row argmax differs"
    assert _rel_close(sel(g["row_lse"]), rows["lse"]).all(), "row lse differs"
    cut_eq = sel(g["row_cut"]) == rows["cut"]
    for k in np.nonzero(~cut_eq)[0]:
        assert rows["margin"][k] < MARGIN, f"top-p cut of packed row {grows[k]} differs at margin {rows['margin'][k]}"
        rep["cut_diff"] += 1
    assert _rel_close(sel(g["row_kept"])[cut_eq], rows["kept_lse"][cut_eq]).all(), "kept lse differs"
    if w.K == 0:
        gp = np.concatenate([np.arange(gpo[r], gpo[r] + L[r]) for r in range(R) if keep[r]] or [np.zeros(0, int)])
        op = np.concatenate([np.arange(dv["pos_off"][r], dv["pos_off"][r] + L[r]) for r in range(R) if keep[r]]
                            or [np.zeros(0, int)])
        d = o["drows"][op]
        assert np.array_equal(np.asarray(g["d_max"])[gp], d["max"]), "draft max differs"
        assert np.array_equal(np.asarray(g["d_argmax"])[gp], d["argmax"]), "draft argmax differs"
        assert _rel_close(np.asarray(g["d_lse"])[gp], d["lse"]).all(), "draft lse differs"
    else:
        for r in np.nonzero(keep)[0]:
            Lr = L[r]
            assert np.array_equal(g["branch_tok"][r, :, :Lr], o["branch_tok"][r, :, :Lr]), f"branch tokens differ (r={r})"
            assert np.allclose(g["post_w"][r, :Lr], o["post_w"][r, :Lr], rtol=REL, atol=1e-15), f"posterior differs (r={r})"
            assert _rel_close(g["q_at_draft"][r, :Lr], o["q_x"][r, :Lr]).all(), f"q at draft differs (r={r})"
    # per-position diagnostics and decisions
    for r in np.nonzero(keep)[0]:
        Lr = int(L[r])
        rep["positions"] += Lr
        if Lr:
            assert np.array_equal(g["u_acc"][r, :Lr].astype(np.float64), o["u_acc"][r, :Lr]), "uniforms differ"
            assert _rel_close(g["p_x"][r, :Lr], o["p_x"][r, :Lr]).all(), f"p(x) differs (r={r})"
            assert _rel_close(g["q_x"][r, :Lr], o["q_x"][r, :Lr]).all(), f"q(x) differs (r={r})"
        ng, no = int(g["n_acc"][r]), int(o["n_acc"][r])
        if ng != no:
            k = min(ng, no)
            m = o["acc_margin"][r, k]
            rep["mismatches"] += 1
            rep["low_margin"].append(("accept", r, k, float(m)))
            assert m < MARGIN, f"n_acc differs for r={r}: gpu {ng} oracle {no}, margin {m}"
            continue
        if int(g["is_bonus"][r]) != int(o["is_bonus"][r]):
            raise AssertionError(f"bonus flag differs for r={r}")
        if int(g["token"][r]) != int(o["token"][r]):
            m = o["sample_margin"][r]
            rep["mismatches"] += 1
            rep["low_margin"].append(("sample", r, no, float(m)))
            assert m < MARGIN, f"token differs for r={r}: gpu {g['token'][r]} oracle {o['token'][r]}, margin {m}"
    return rep


def excused(rep: dict) -> int:
    """Disagreements excused by a low oracle margin: decisions (n_acc, token)
    and top-p cuts alike."""
    return rep["mismatches"] + rep["cut_diff"]


def assert_rate(rep: dict):
    """Excused disagreements must number fewer than 1e-4 of the verified
    positions (so none at all below 10,000 positions)."""
    n = excused(rep)
    assert n < 1e-4 * rep["positions"] or n == 0, (
        f"{rep['mismatches']} low-margin decision mismatches and {rep['cut_diff']} top-p cut differences "
        f"over {rep['positions']} positions")
