"""Device status bits (failure detection): each malformed input sets its bit
in the workspace's status word, the kernels stay in bounds, and the requests
the input does not touch still match the oracle.  Needs an MI355X; run with
``-m gpu``.  The inputs used here are those the kernels are written to clamp
(out-of-range values, malformed lengths within the buffers' capacity)."""
import copy

import numpy as np
import pytest

import synth
from harness import assert_rate, compare_step, gpu_step_runner, oracle_step

pytestmark = pytest.mark.gpu

BAD_TEMPERATURE, BAD_TOP_P, NONFINITE, BAD_SCORE = 0x001, 0x002, 0x004, 0x008
BAD_TOKEN, BAD_OFFSETS, EMPTY_POSTERIOR, BAD_BUDGET, BAD_NACC, BAD_BLOCK = 0x010, 0x020, 0x040, 0x080, 0x100, 0x200


def banner(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _sv():
    import draft_verification_sv_amd as sv

    return sv


def _step(w, fused, L=None):
    vs, run = gpu_step_runner(w, fused=fused)
    g = run(0, L=L)
    return vs, g, _sv().sv_get_status(vs.ws)


def _bf16(v):
    return np.uint16(synth.f32_to_bf16_bits(np.array([v], np.float32))[0])


CHAINS = pytest.mark.parametrize("fused", [False, True], ids=["standalone", "fused"])


@CHAINS
def test_bad_temperature(fused):
    w = synth.config(5, V=1031, R=8, steps=1)
    wg = copy.copy(w)
    wg.T = w.T.copy()
    wg.T[3], wg.T[5] = -1.0, np.nan
    banner(f"status BAD_TEMPERATURE fused={fused}")
    vs, g, st = _step(wg, fused)
    assert st & BAD_TEMPERATURE, st
    assert_rate(compare_step(w, g, oracle_step(w, 0), skip={3, 5}))


@CHAINS
def test_bad_top_p(fused):
    w = synth.config(5, V=1031, R=8, steps=1)
    wg = copy.copy(w)
    wg.top_p = w.top_p.copy()
    wg.top_p[2], wg.top_p[6] = 0.0, np.nan
    banner(f"status BAD_TOP_P fused={fused}")
    vs, g, st = _step(wg, fused)
    assert st & BAD_TOP_P, st
    assert_rate(compare_step(w, g, oracle_step(w, 0), skip={2, 6}))
    # the flagged rows keep only their top value (ties included)
    for r in (2, 6):
        k = int(g["tgt_off"][r])
        assert g["row_cut"][k] == g["row_max"][k]


@CHAINS
def test_nonfinite_in_greedy_target_rows_without_top_p(fused):
    """T = 0 forms no sums, so NaN must be caught apart from them: a positive
    NaN in a full 8-value vector, one in the ragged tail, and +inf."""
    w = synth.config(3, V=1031, R=6, steps=1)
    w.T = w.T.copy()
    w.T[[1, 2, 4]] = 0.0
    wg = copy.copy(w)
    wg.tgt = w.tgt.copy()
    wg.tgt[1, 0, 5] = 0x7FC0                   # NaN in a full vector of request 1's first row
    wg.tgt[2, 0, 1029] = 0x7FC1                # NaN in the tail (V = 1031 = 128 * 8 + 7)
    wg.tgt[4, 0, 300] = 0x7F80                 # +inf
    for r in (1, 2, 4):
        banner(f"status NONFINITE greedy target rows fused={fused} request {r}")
        wr = copy.copy(w)
        wr.tgt = w.tgt.copy()
        wr.tgt[r] = wg.tgt[r]
        vs, g, st = _step(wr, fused)
        assert st & NONFINITE, (r, st)
        assert_rate(compare_step(w, g, oracle_step(w, 0), skip={r}))


@CHAINS
def test_nonfinite_in_component_rows(fused):
    """NaN and +-inf in the mixture's component rows (read for the branch
    argmax only): in a full vector and in the ragged tail of a row."""
    w = synth.config(4, V=1031, R=4, steps=1)
    cases = {0: (2, 3, 17, 0x7FC0), 1: (5, 0, 1030, 0xFFC0), 2: (0, 7, 640, 0xFF80), 3: (7, 15, 1024, 0x7F80)}
    for r, (z, i, v, bits) in cases.items():
        banner(f"status NONFINITE component row fused={fused} request {r} z={z} i={i} v={v}")
        wg = copy.copy(w)
        wg.comp = w.comp.copy()
        wg.comp[r, z, i, v] = bits
        vs, g, st = _step(wg, fused)
        assert st & NONFINITE, (r, st)
        assert_rate(compare_step(w, g, oracle_step(w, 0), skip={r}))


def test_bad_survival_scores():
    """Estimates outside [0, 1] set the bit; the allocation still verifies
    min(B, R b) positions in well-formed offsets, and the step matches the
    oracle at those lengths."""
    w = synth.config(5, V=1031, R=8, steps=1)
    wg = copy.copy(w)
    wg.a = w.a.copy()
    wg.a[0, 2, 3], wg.a[0, 4, 0], wg.a[0, 6, 5] = 1.5, -0.25, np.nan
    banner("status BAD_SCORE")
    vs, g, st = _step(wg, True)
    assert st & BAD_SCORE, st
    L = g["L"]
    assert (L >= 0).all() and (L <= w.b).all() and L.sum() == min(w.budget, w.R * w.b)
    assert np.array_equal(g["pos_off"], np.concatenate([[0], np.cumsum(L)]))
    assert np.array_equal(g["tgt_off"], np.concatenate([[0], np.cumsum(L + 1)]))
    assert_rate(compare_step(w, g, oracle_step(w, 0, L=L), offsets=False))


def test_negative_budget():
    """A negative budget sets the bit and verifies nothing: every request
    emits one token from its first target row, as the oracle does."""
    w = synth.config(5, V=1031, R=8, steps=1)
    vs, run = gpu_step_runner(w, fused=True)  # buffers at the usual capacity
    w.budget = -3                             # the value the device reads
    banner("status BAD_BUDGET")
    g = run(0)
    st = _sv().sv_get_status(vs.ws)
    assert st & BAD_BUDGET, st
    assert (g["L"] == 0).all()
    assert_rate(compare_step(w, g, oracle_step(w, 0)))


def test_bad_block_lengths():
    """Block lengths outside [0, b] set the bit and are clamped: DVL and the
    step then match the oracle at the clamped lengths."""
    w = synth.config(5, V=1031, R=8, steps=1, ragged=True)
    wg = copy.copy(w)
    wg.block_len = w.block_len.copy()
    wg.block_len[1], wg.block_len[3] = w.b + 4, -2
    wc = copy.copy(w)
    wc.block_len = np.clip(wg.block_len, 0, w.b).astype(np.int32)
    banner("status BAD_BLOCK")
    vs, g, st = _step(wg, True)
    assert st & BAD_BLOCK, st
    assert_rate(compare_step(wc, g, oracle_step(wc, 0)))


@CHAINS
@pytest.mark.parametrize("cfg", [5, 3], ids=["mixture", "dense"])
def test_bad_draft_tokens(fused, cfg):
    """Draft tokens outside the vocabulary in two requests (the rows launches
    clamp them for their gathers; the draw reports them): the bit is set, and
    the other requests match the oracle."""
    w = synth.config(cfg, V=1031, R=8, steps=1)
    wg = copy.copy(w)
    wg.x = w.x.copy()
    wg.x[0, 2, 1], wg.x[0, 5, 0] = w.V + 3, -1
    wg.budget = w.R * w.b  # every position verified, so both tokens are read
    wo = copy.copy(w)
    wo.budget = wg.budget
    banner(f"status BAD_TOKEN config {cfg} fused={fused}")
    vs, g, st = _step(wg, fused)
    assert st & BAD_TOKEN, st
    assert_rate(compare_step(wo, g, oracle_step(wo, 0), skip={2, 5}))


@CHAINS
def test_bad_offsets(fused):
    """A verified length above b (offsets written by the caller, within the
    buffers' capacity): the request is flagged and left out; the others match
    the oracle."""
    w = synth.config(4, V=1031, R=4, steps=1)
    L = np.array([3, w.b + 1, 2, 4], np.int32)
    Lo = L.copy()
    Lo[1] = 0
    banner(f"status BAD_OFFSETS fused={fused}")
    vs, g, st = _step(w, fused, L=L)
    assert st & BAD_OFFSETS, st
    assert_rate(compare_step(w, g, oracle_step(w, 0, L=Lo), skip={1}, offsets=False))


@CHAINS
def test_empty_posterior(fused):
    """A draft token that no branch decodes at position 1: q = 0 there and
    the posterior is empty from position 2 on (the bit is set), which the
    oracle defines too (q = 0, so the residual is p); the whole step
    matches."""
    w = synth.config(4, V=1031, R=4, steps=1)
    r = 1
    used = set(w.branch_tok[r, :, 0].tolist())
    w.x = w.x.copy()
    w.x[0, r, 0] = next(v for v in range(w.V) if v not in used)
    banner(f"status EMPTY_POSTERIOR fused={fused}")
    vs, g, st = _step(w, fused)
    assert st & EMPTY_POSTERIOR, st
    assert_rate(compare_step(w, g, oracle_step(w, 0)))
    assert g["q_at_draft"][r, 0] == 0.0 and (g["post_w"][r, 1:] == 0).all()


def test_bad_accepted_length_in_standalone_draw():
    """sv_residual_sample with n_acc outside [0, L_r]: the bit is set, the
    value is clamped, and the other requests' tokens are unchanged."""
    import torch

    sv = _sv()
    w = synth.config(3, V=1031, R=8, steps=1)
    vs, run = gpu_step_runner(w)
    g = run(0)
    assert sv.sv_get_status(vs.ws) == 0
    tok0 = g["token"].copy()
    n = torch.from_numpy(g["n_acc"].copy())
    n[2], n[6] = int(g["L"][2]) + 5, -3
    vs.n_acc.copy_(n)
    from draft_verification_sv_amd.step import row_pitch

    ld = row_pitch(w.V, w.dtype)
    banner("status BAD_NACC")
    tgt, draft = vs.last_rows  # the step's packed target rows and draft rows, still in place
    sv.sv_residual_sample(tgt, vs.dt, ld, w.V, vs.tgt_off, vs.pos_off, w.R, w.b, vs.T, vs.row_argmax, vs.row_cut,
                          vs.row_kept, vs.q_mode, draft, vs.dt, ld, vs.d_argmax, vs.d_lse, 0, None, None, vs.seed,
                          vs.n_acc, vs.token, vs.is_bonus, vs.ws, vs.ws_bytes)
    st = sv.sv_get_status(vs.ws)
    assert st & BAD_NACC, st
    tok = vs.token.cpu().numpy()
    keep = [r for r in range(w.R) if r not in (2, 6)]
    assert np.array_equal(tok[keep], tok0[keep])
    assert ((tok >= 0) & (tok < w.V)).all()
