"""The allocation-free draw (sv_residual_sample_noalloc) against the
workspace entry point it mirrors (sv_residual_sample), through the C ABI, on
two calls in a row -- the second with a smaller problem, so that it runs on
what the first left in the library's fixed scratch -- and against the
oracle.  Needs an MI355X; run with ``-m gpu``."""
import numpy as np
import pytest

import synth
from harness import assert_rate, compare_step, oracle_step

pytestmark = pytest.mark.gpu


def _standalone_step(w, s):
    """One step through the workspace entry points (DVL when w has a budget,
    statistics, proposal, sv_accept, sv_residual_sample); returns the step
    object, the packed target rows and the proposal rows."""
    import torch

    from draft_verification_sv_amd.step import VerifyStep, pack_rows_device, row_pitch, to_device_rows

    R, b, V, K = w.R, w.b, w.V, w.K
    ld = row_pitch(V, w.dtype)
    max_pos = min(w.budget, R * b) if w.budget is not None else R * b
    vs = VerifyStep(R=R, b=b, V=V, dtype=w.dtype, K=K, max_pos=max_pos, diagnostics=True)
    full = to_device_rows(w.tgt, ld)
    packed = torch.empty_like(full)
    draft = to_device_rows(w.draft, ld) if K == 0 else None
    comp = to_device_rows(w.comp, ld) if K > 0 else None
    vs.set_inputs(T=w.T, x=w.x[s], seed=int(w.seeds[s]), top_p=w.top_p, mix=w.mix,
                  a=None if w.a is None else w.a[s], budget=w.budget)
    if w.budget is not None:
        vs.run_dvl()
        L = vs.L.cpu().numpy()
    else:
        vs.set_full_verification()
        L = np.full(R, b, np.int32)
    pack_rows_device(full, L, b + 1, packed)
    vs.run_verify(packed, ld, draft=draft, draft_ld=ld, comp=comp, comp_ld=ld, fused=False)
    return vs, packed, ld, draft


def _noalloc_draw(vs, packed, ld, draft):
    import torch

    import draft_verification_sv_amd as sv

    dense = vs.q_mode == sv.SV_Q_DENSE
    R = vs.R
    token = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    bonus = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sv.sv_residual_sample_noalloc(packed, vs.dt, ld, vs.V, vs.tgt_off, vs.pos_off, R, vs.b, vs.T, vs.row_argmax,
                                  vs.row_cut, vs.row_kept, vs.q_mode, draft if dense else None, vs.dt,
                                  ld if dense else 0, vs.d_argmax if dense else None, vs.d_lse if dense else None,
                                  vs.K, None if dense else vs.branch_tok, None if dense else vs.post_w, vs.seed,
                                  vs.n_acc, token, bonus, status)
    torch.cuda.synchronize()
    return token.cpu().numpy(), bonus.cpu().numpy(), int(status.cpu().numpy()[0])


def test_noalloc_draw_matches_workspace_entry_point():
    import draft_verification_sv_amd as sv

    # first the full-size mixture step (conc 32, V 151936, K 8, DVL 256, top-p),
    # then a smaller dense step with DVL and a ragged vocabulary
    cases = [(synth.config(5, steps=1), 0), (synth.config(3, V=2053, R=8, steps=2), 1)]
    for w, s in cases:
        print(f"\n[gpu-case] sv_residual_sample_noalloc {w.name} V={w.V} R={w.R} step {s}", flush=True)
        vs, packed, ld, draft = _standalone_step(w, s)
        g = vs.results()
        tok, bon, st = _noalloc_draw(vs, packed, ld, draft)
        assert np.array_equal(tok, g["token"]), (tok, g["token"])
        assert np.array_equal(bon, g["is_bonus"])
        assert st == 0 and sv.sv_get_status(vs.ws) == 0
        g["token"], g["is_bonus"] = tok, bon
        rep = compare_step(w, g, oracle_step(w, s))
        assert_rate(rep)


def test_noalloc_draw_rejects_oversized_problems():
    """The size check runs on the host before any launch: a problem whose
    records and sub-chunk sums exceed the fixed scratch returns
    SV_ERR_TOO_LARGE."""
    import torch

    import draft_verification_sv_amd as sv

    R, b, V = 400, 16, 151936
    z = torch.zeros(R * b * 4, dtype=torch.float64, device="cuda")
    with pytest.raises(sv.SvError) as e:
        sv.sv_residual_sample_noalloc(z, sv.SV_BF16, V, V, z, z, R, b, z, z, z, z, sv.SV_Q_DENSE, z, sv.SV_BF16, V, z, z, 0, None, None, z, z, z, z, z)
    assert e.value.code == sv.SV_ERR_TOO_LARGE
