"""Host logic of the parity harness (CPU only): the comparison accepts a
result that equals the oracle's, rejects one with a changed decision or
statistic, and leaves skipped requests out."""
import numpy as np
import pytest

import synth
from harness import assert_rate, compare_step, oracle_step


def _as_gpu(w, o):
    """The oracle's step laid out as the GPU's results are (packed rows,
    positions by pos_off)."""
    dv = o["dvl"]
    R, b, K = w.R, w.b, w.K
    rows = o["rows"]
    g = {"L": dv["L"].copy(), "pos_off": dv["pos_off"].copy(), "tgt_off": dv["tgt_off"].copy(),
         "s": (dv["s"].reshape(-1).copy() if dv["s"] is not None else None),
         "row_max": rows["max"].copy(), "row_argmax": rows["argmax"].copy(), "row_lse": rows["lse"].copy(),
         "row_cut": rows["cut"].copy(), "row_kept": rows["kept_lse"].copy(),
         "n_acc": o["n_acc"].copy(), "token": o["token"].copy(), "is_bonus": o["is_bonus"].copy(),
         "u_acc": o["u_acc"].astype(np.float32), "p_x": o["p_x"].copy(), "q_x": o["q_x"].copy()}
    if K == 0:
        d = o["drows"]
        g.update(d_max=d["max"].copy(), d_argmax=d["argmax"].copy(), d_lse=d["lse"].copy())
    else:
        g.update(branch_tok=o["branch_tok"].copy(), post_w=o["post_w"].copy(), q_at_draft=o["q_x"].copy())
    return g


@pytest.mark.parametrize("c", [3, 5])
def test_compare_step_accepts_the_oracle_and_catches_changes(c):
    w = synth.config(c, V=257, R=6, steps=1)
    o = oracle_step(w, 0)
    rep = compare_step(w, _as_gpu(w, o), o)
    assert rep["mismatches"] == 0 and rep["positions"] == int(o["dvl"]["L"].sum())
    assert_rate(rep)
    r = int(np.argmax(o["dvl"]["L"]))
    for key, change in (("row_argmax", lambda g: g["row_argmax"].__setitem__(g["tgt_off"][r], -5)),
                        ("p_x", lambda g: g["p_x"].__setitem__((r, 0), g["p_x"][r, 0] * 1.01 + 1e-3)),
                        ("n_acc", lambda g: g["n_acc"].__setitem__(r, (g["n_acc"][r] + 1) % (g["L"][r] + 1)))):
        g = _as_gpu(w, o)
        change(g)
        with pytest.raises(AssertionError):
            compare_step(w, g, o)
        # the same change in a skipped request is not compared
        rep = compare_step(w, g, o, skip={r})
        assert rep["positions"] == int(o["dvl"]["L"].sum()) - int(o["dvl"]["L"][r]), key


def test_compare_step_with_caller_offsets_and_length_override():
    """Offsets written by the caller: a request with a malformed length is
    skipped, and the oracle runs the other requests at the GPU's lengths."""
    w = synth.config(4, V=257, R=4, steps=1)
    L = np.array([2, 5, 1, 3], np.int32)  # request 1 stands for one whose offsets the GPU flags
    Lo = L.copy()
    Lo[1] = 0
    o = oracle_step(w, 0, L=Lo)
    g = _as_gpu(w, o)
    # the GPU's packing follows L (request 1 holds 6 rows)
    g["pos_off"] = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    g["tgt_off"] = np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)
    src = o["dvl"]["tgt_off"]
    for k in ("row_max", "row_argmax", "row_lse", "row_cut", "row_kept"):
        full = np.zeros(int(g["tgt_off"][-1]), g[k].dtype)
        for r in (0, 2, 3):
            full[g["tgt_off"][r]:g["tgt_off"][r] + L[r] + 1] = g[k][src[r]:src[r] + L[r] + 1]
        g[k] = full
    g["L"] = L
    rep = compare_step(w, g, o, skip={1}, offsets=False)
    assert rep["positions"] == int(L[[0, 2, 3]].sum())
    with pytest.raises(AssertionError):
        compare_step(w, g, o, offsets=False)
