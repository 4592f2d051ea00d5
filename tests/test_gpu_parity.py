"""GPU parity: libsv (through its C ABI) against the CPU oracle on the same
seeded inputs.  Needs an MI355X; run with ``-m gpu``."""
import os

import numpy as np
import pytest

import oracle
import synth
from harness import assert_rate, compare_step, excused, gpu_graph_runner, gpu_step_runner, log_parity, oracle_step

pytestmark = pytest.mark.gpu


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


# ---------------------------------------------------------------- Philox
@pytest.mark.parametrize("seed", [0, 1, 5, 2**32 + 7, 2**64 - 1])
def test_philox_words_bitexact(seed):
    import torch

    sv = _sv()
    R, n = 33, 17
    banner(f"sv_philox_uniforms seed={seed} R={R} n={n}")
    sd = torch.tensor([np.uint64(seed).view(np.int64)], device="cuda")
    out = torch.zeros(R * n * 4, dtype=torch.int32, device="cuda")
    sv.sv_philox_uniforms(sd, R, n, out)
    got = out.cpu().numpy().view(np.uint32).reshape(R, n, 4)
    assert np.array_equal(got, oracle.uniform_words(seed, R, n))


# ---------------------------------------------------------------- DVL
def _dvl_cases():
    rng = np.random.default_rng(7)
    cases = []
    # R*b up to 8192 keeps the scores in LDS, beyond that in global memory
    # (8192 and 8193: the two sides of that switch)
    for R, b in [(1, 1), (3, 5), (32, 16), (7, 64), (64, 16), (65, 16), (300, 16), (512, 16), (8193, 1), (600, 16)]:
        for kind in ("beta", "ties", "signed_zeros"):
            if kind == "beta":
                a = rng.beta(8, 2, size=(R, b)).astype(np.float32)
            elif kind == "ties":
                a = rng.choice([0.0, 0.5, 0.75, 1.0], size=(R, b)).astype(np.float32)
            else:  # -0 orders as 0: ties broken by (r, i)
                a = rng.choice([0.0, -0.0, 0.5, 1.0], size=(R, b)).astype(np.float32)
            for B in sorted({0, 1, R * b // 2, R * b - 1, R * b, R * b + 5}):
                if B >= 0:
                    cases.append((R, b, kind, B, a))
    return cases


@pytest.mark.parametrize("R,b,kind,B,a", _dvl_cases(), ids=lambda v: str(v) if not hasattr(v, "shape") else "a")
def test_dvl_bitexact(R, b, kind, B, a):
    import torch

    sv = _sv()
    banner(f"dvl_alloc_pack R={R} b={b} {kind} B={B}")
    ws, nb = sv.make_workspace(R, b, 0, 8)
    d = dict(device="cuda")
    at = torch.from_numpy(a.reshape(-1)).to(**d)
    bud = torch.tensor([B], dtype=torch.int32, **d)
    s = torch.zeros(R * b, dtype=torch.float32, **d)
    L = torch.zeros(R, dtype=torch.int32, **d)
    po = torch.zeros(R + 1, dtype=torch.int32, **d)
    to = torch.zeros(R + 1, dtype=torch.int32, **d)
    sv.dvl_alloc_pack(at, R, b, None, bud, s, L, po, to, ws, nb)
    o = oracle.dvl(a, B)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), o["s"].reshape(-1).view(np.uint32))
    assert np.array_equal(L.cpu().numpy(), o["L"])
    assert np.array_equal(po.cpu().numpy(), o["pos_off"])
    assert np.array_equal(to.cpu().numpy(), o["tgt_off"])
    assert sv.sv_get_status(ws) == 0


def _dvl_ragged_cases():
    rng = np.random.default_rng(8)
    cases = []
    for R, b in [(1, 1), (3, 5), (32, 16), (7, 64), (64, 16), (600, 16)]:
        for pattern in ("random", "zeros_and_full", "all_zero"):
            if pattern == "random":
                bl = rng.integers(0, b + 1, size=R)
            elif pattern == "zeros_and_full":
                bl = np.where(rng.random(R) < 0.5, 0, b)
            else:
                bl = np.zeros(R)
            bl = bl.astype(np.int32)
            kind = "ties" if R % 2 else "beta"
            a = (rng.choice([0.0, 0.5, 0.75, 1.0], size=(R, b)) if kind == "ties"
                 else rng.beta(8, 2, size=(R, b))).astype(np.float32)
            n = int(bl.sum())
            for B in sorted({0, 1, n // 2, max(n - 1, 0), n, n + 3, R * b}):
                cases.append((R, b, pattern, B, a, bl))
    return cases


@pytest.mark.parametrize("R,b,pattern,B,a,bl", _dvl_ragged_cases(),
                         ids=lambda v: str(v) if not hasattr(v, "shape") else "arr")
def test_dvl_ragged_block_lengths_bitexact(R, b, pattern, B, a, bl):
    """Per-request block length b_r: only the first b_r positions of request r
    are candidates (scores past b_r are 0); bit-exact against the oracle."""
    import torch

    sv = _sv()
    banner(f"dvl_alloc_pack ragged R={R} b={b} {pattern} B={B}")
    ws, nb = sv.make_workspace(R, b, 0, 8)
    d = dict(device="cuda")
    at = torch.from_numpy(a.reshape(-1)).to(**d)
    blt = torch.from_numpy(bl).to(**d)
    bud = torch.tensor([B], dtype=torch.int32, **d)
    s = torch.full((R * b,), 7.0, dtype=torch.float32, **d)
    L = torch.zeros(R, dtype=torch.int32, **d)
    po = torch.zeros(R + 1, dtype=torch.int32, **d)
    to = torch.zeros(R + 1, dtype=torch.int32, **d)
    sv.dvl_alloc_pack(at, R, b, blt, bud, s, L, po, to, ws, nb)
    o = oracle.dvl(a, B, block_len=bl)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), o["s"].reshape(-1).view(np.uint32))
    assert np.array_equal(L.cpu().numpy(), o["L"])
    assert np.array_equal(po.cpu().numpy(), o["pos_off"])
    assert np.array_equal(to.cpu().numpy(), o["tgt_off"])
    assert sv.sv_get_status(ws) == 0


# ---------------------------------------------------------------- row statistics
def _edge_rows(V, rng):
    base = (3.0 * rng.standard_normal(V)).astype(np.float32)
    rows = {"normal": base}
    rows["ties_at_max"] = base.copy()
    rows["ties_at_max"][[3 % V, (V // 2), V - 1]] = base.max() + 1.0
    rows["constant"] = np.full(V, -1.25, np.float32)
    rows["zeros"] = np.zeros(V, np.float32)
    z = base.copy()
    z[::5] = 0.0
    z[1::7] = -0.0
    rows["with_zeros"] = z
    t = base.copy()
    t[::3] = 1e-30
    rows["tiny"] = t
    h = base.copy()
    h[::11] = 3e7
    rows["huge"] = h
    rows["wide"] = (40.0 * rng.standard_normal(V)).astype(np.float32)
    rows["neg_only"] = -np.abs(base) - 0.5
    return rows


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 1031, 4096, 151936])
def test_row_stats_edges(dtype, V):
    import torch

    sv = _sv()
    from draft_verification_sv_amd.step import row_pitch, to_device_rows

    rng = np.random.default_rng(V)
    rows = _edge_rows(V, rng)
    names = list(rows)
    mat = np.stack([rows[k] for k in names])
    stored = synth.f32_to_bf16_bits(mat) if dtype == "bf16" else mat
    settings = [(T, tp) for T in (0.0, 0.5, 1.0, 1.5) for tp in (None, 0.95, 0.5, 1e-3)]
    R = len(settings)
    # request k reads all rows with its own (T, top_p): packed rows = R copies
    allrows = np.concatenate([stored] * R)
    ld = row_pitch(V, dtype)
    dev = to_device_rows(allrows, ld)
    n = len(names)
    off = torch.arange(R + 1, dtype=torch.int32, device="cuda") * n
    T = np.array([s[0] for s in settings], np.float32)
    tp = np.array([1.0 if s[1] is None else s[1] for s in settings], np.float32)
    banner(f"sv_topp_threshold edges dtype={dtype} V={V} rows={R * n}")
    ws, nb = sv.make_workspace(R, 16, 0, V)
    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    outs = [torch.zeros(R * n, dtype=t, device="cuda") for t in (f32, i32, f64, f32, f64)]
    sv.sv_topp_threshold(dev, sv.SV_BF16 if dtype == "bf16" else sv.SV_F32, ld, V, off, 0, R, R * n,
                         torch.from_numpy(T).cuda(), torch.from_numpy(tp).cuda(), *outs, ws, nb)
    mx, am, lse, cut, kept = [t.cpu().numpy() for t in outs]
    req = np.repeat(np.arange(R), n)
    o = oracle.row_stats_batch(allrows, req, T, tp)
    assert np.array_equal(mx, o["max"])
    assert np.array_equal(am, o["argmax"])
    # bf16 rows with top-p off take the streaming pass (fp32 exponentials,
    # double sums): the 1e-5 relative bar of the row statistics; the exact
    # histogram (top-p on) and the fp32 generic path agree to 1e-12
    stream = np.repeat(tp >= 1.0, n) & (dtype == "bf16")
    np.testing.assert_allclose(lse[~stream], o["lse"][~stream], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[stream], o["lse"][stream], rtol=1e-5, atol=1e-12)
    ok = cut == o["cut"]
    assert np.all(ok | (o["margin"] < 1e-6)), list(zip(np.nonzero(~ok)[0], o["margin"][~ok]))
    np.testing.assert_allclose(kept[ok & ~stream], o["kept_lse"][ok & ~stream], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kept[ok & stream], o["kept_lse"][ok & stream], rtol=1e-5, atol=1e-12)
    assert sv.sv_get_status(ws) == 0


@pytest.mark.parametrize("V", [7, 1031, 151936])
def test_dense_rows_edges(V):
    """sv_verify_rows_dense without top-p (rows split into parts, streamed in
    batches with one maximum check per batch): maximum and argmax (lowest index
    among ties, ties inside a batch, across batches and across parts) exactly,
    lse to the 1e-5 bar, for target and draft rows at T = 0, 0.5, 1 and 1.5."""
    import torch

    sv = _sv()
    from draft_verification_sv_amd.step import row_pitch, to_device_rows

    rng = np.random.default_rng(V + 7)
    rows = _edge_rows(V, rng)
    t = rows["normal"].copy()  # the maximum at two positions one batch stride apart, and at the row's end
    for i in (V // 3, V // 3 + 256 * 8, V - 1):
        t[i % V] = t.max() + 2.0
    rows["ties_spread"] = t
    stored = synth.f32_to_bf16_bits(np.stack(list(rows.values())))
    n = len(stored)
    T = np.array([0.0, 0.5, 1.0, 1.5], np.float32)
    R, b = len(T), n - 1
    tgt = np.concatenate([stored] * R)  # request r: all n rows as its L_r + 1 = n target rows
    dft = np.stack([stored[1 + (r + j) % (n - 1)] for r in range(R) for j in range(b)])  # [R * b, V]
    ld = row_pitch(V, "bf16")
    dt, dd = to_device_rows(tgt, ld), to_device_rows(dft, ld)
    d = dict(device="cuda")
    tgt_off = torch.arange(R + 1, dtype=torch.int32, **d) * n
    pos_off = torch.arange(R + 1, dtype=torch.int32, **d) * b
    ws, nb = sv.make_workspace(R, b, 0, V)
    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    ro = [torch.zeros(R * n, dtype=x, **d) for x in (f32, i32, f64, f32, f64)]
    do = [torch.zeros(R * b, dtype=x, **d) for x in (f32, i32, f64)]
    banner(f"sv_verify_rows_dense edges V={V}")
    x = torch.from_numpy(rng.integers(0, V, R * b, dtype=np.int32)).cuda()  # draft tokens (slot records)
    sv.sv_verify_rows_dense(dt, sv.SV_BF16, ld, V, tgt_off, R, R * n, torch.from_numpy(T).cuda(), None, *ro, dd,
                            sv.SV_BF16, ld, b, pos_off, R * b, x, *do, ws, nb)
    torch.cuda.synchronize()
    for got, rows_, per in ((ro, tgt, n), (do, dft, b)):
        o = oracle.row_stats_batch(rows_, np.repeat(np.arange(R), per), T)
        mx, am, lse = [x.cpu().numpy() for x in got[:3]]
        assert np.array_equal(mx, o["max"])
        assert np.array_equal(am, o["argmax"])
        hot = np.repeat(T > 0, per)
        np.testing.assert_allclose(lse[hot], o["lse"][hot], rtol=1e-5, atol=1e-12)
    assert sv.sv_get_status(ws) == 0


DENSE_SHAPES = [  # (V, b, L per request)
    (8192, 4, [1, 4, 0]),            # short rows, one part each
    (8200, 2, [0]),                  # one target row, no draft rows
    (151936, 4, [0, 3]),             # full rows, few
    (65536, 16, "random40"),         # ragged counts, many rows
    (8192, 16, "full64"),            # every position verified
]


@pytest.mark.parametrize("V,b,Ls", DENSE_SHAPES,
                         ids=[f"V{v}-b{b}-{l if isinstance(l, str) else len(l)}" for v, b, l in DENSE_SHAPES])
def test_dense_rows_shapes(V, b, Ls):
    """sv_verify_rows_dense without top-p over several row lengths and
    request mixes: device-side row counts below the capacities, per-request
    temperatures (0 included), the maximum repeated 1024 and 4096 vectors
    apart and at the row end (across batches and parts); maximum and argmax
    exactly, lse to 1e-5; two runs bit-equal; a non-finite value sets the
    status bit."""
    import torch

    sv = _sv()
    from draft_verification_sv_amd.step import row_pitch, to_device_rows

    rng = np.random.default_rng(V * 31 + b)
    if Ls == "random40":
        L = rng.integers(0, b + 1, size=40)
    elif Ls == "full64":
        L = np.full(64, b)
    else:
        L = np.array(Ls)
    R = len(L)
    nt, nd = int((L + 1).sum()), int(L.sum())
    tgt = (3.0 * rng.standard_normal((nt, V))).astype(np.float32)
    dft = (2.0 * rng.standard_normal((R * b, V))).astype(np.float32)
    for k in range(0, nt, 3):  # ties at the maximum, 1024 and 4096 vectors apart and at the row end
        m = tgt[k].max() + 1.0
        for i in (V // 5, V // 5 + 1024 * 8, V // 5 + 4096 * 8, V - 1):
            tgt[k, i % V] = m
    T = np.array([(0.0, 0.5, 1.0, 1.5)[r % 4] for r in range(R)], np.float32)
    tb, db = synth.f32_to_bf16_bits(tgt), synth.f32_to_bf16_bits(dft)
    ld = row_pitch(V, "bf16")
    dt, dd = to_device_rows(tb, ld), to_device_rows(db, ld)
    d = dict(device="cuda")
    tgt_off = torch.from_numpy(np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)).cuda()
    pos_off = torch.from_numpy(np.concatenate([[0], np.cumsum(L)]).astype(np.int32)).cuda()
    x = torch.from_numpy(rng.integers(0, V, R * b, dtype=np.int32)).cuda()  # draft tokens (slot records)
    ws, nb = sv.make_workspace(R, b, 0, V)
    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    cap_t, cap_d = R * (b + 1), R * b
    runs = []
    for rep in range(2):
        ro = [torch.zeros(cap_t, dtype=x, **d) for x in (f32, i32, f64, f32, f64)]
        do = [torch.zeros(cap_d, dtype=x, **d) for x in (f32, i32, f64)]
        banner(f"sv_verify_rows_dense V={V} R={R} rows {nt}+{nd} run {rep}")
        sv.sv_verify_rows_dense(dt, sv.SV_BF16, ld, V, tgt_off, R, cap_t, torch.from_numpy(T).cuda(), None, *ro, dd,
                                sv.SV_BF16, ld, b, pos_off, cap_d, x, *do, ws, nb)
        torch.cuda.synchronize()
        runs.append([x.cpu().numpy() for x in ro[:3] + do[:3]])
    for a, c in zip(runs[0], runs[1]):
        assert a.tobytes() == c.tobytes()
    mx, am, lse, dmx, dam, dlse = runs[0]
    o = oracle.row_stats_batch(tb, np.repeat(np.arange(R), L + 1), T)
    assert np.array_equal(mx[:nt], o["max"]) and np.array_equal(am[:nt], o["argmax"])
    hot = np.repeat(T > 0, L + 1)
    np.testing.assert_allclose(lse[:nt][hot], o["lse"][hot], rtol=1e-5, atol=1e-12)
    drows = np.concatenate([np.arange(r * b, r * b + L[r]) for r in range(R)]).astype(np.int64)
    o = oracle.row_stats_batch(db[drows], np.repeat(np.arange(R), L), T)
    assert np.array_equal(dmx[:nd], o["max"]) and np.array_equal(dam[:nd], o["argmax"])
    hot = np.repeat(T > 0, L)
    np.testing.assert_allclose(dlse[:nd][hot], o["lse"][hot], rtol=1e-5, atol=1e-12)
    assert sv.sv_get_status(ws) == 0
    # a non-finite value in the last target row sets the status bit
    for bad in (-np.inf, np.nan, np.inf):
        t2 = tgt.copy()
        t2[nt - 1, V // 2] = bad
        d2 = to_device_rows(synth.f32_to_bf16_bits(t2), ld)
        ws2, nb2 = sv.make_workspace(R, b, 0, V)
        T2 = torch.ones(R, **d)
        sv.sv_verify_rows_dense(d2, sv.SV_BF16, ld, V, tgt_off, R, cap_t, T2, None, *ro, dd, sv.SV_BF16, ld, b,
                                pos_off, cap_d, x, *do, ws2, nb2)
        assert sv.sv_get_status(ws2) & 0x004, bad


def test_row_stats_nonfinite_sets_status():
    import torch

    sv = _sv()
    from draft_verification_sv_amd.step import to_device_rows

    V = 1024
    row = np.linspace(-3, 3, V).astype(np.float32)
    row[17] = np.inf
    row[99] = np.nan
    dev = to_device_rows(synth.f32_to_bf16_bits(row[None]), V)
    ws, nb = sv.make_workspace(1, 16, 0, V)
    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    outs = [torch.zeros(1, dtype=t, device="cuda") for t in (f32, i32, f64, f32, f64)]
    off = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    banner("sv_topp_threshold non-finite row")
    sv.sv_topp_threshold(dev, sv.SV_BF16, V, V, off, 0, 1, 1, torch.ones(1, device="cuda"),
                         torch.full((1,), 0.9, device="cuda"), *outs, ws, nb)
    assert sv.sv_get_status(ws) & 0x004
    # the streaming pass (top-p off), with +inf / NaN and with -inf alone
    ninf = np.linspace(-3, 3, V).astype(np.float32)
    ninf[500] = -np.inf
    for r in (row, ninf):
        d2 = to_device_rows(synth.f32_to_bf16_bits(r[None]), V)
        ws2, nb2 = sv.make_workspace(1, 16, 0, V)
        sv.sv_topp_threshold(d2, sv.SV_BF16, V, V, off, 0, 1, 1, torch.ones(1, device="cuda"), None, *outs, ws2, nb2)
        assert sv.sv_get_status(ws2) & 0x004


def test_host_argument_errors():
    import torch

    sv = _sv()
    ws, nb = sv.make_workspace(2, 16, 0, 64)
    z = torch.zeros(64, device="cuda")
    with pytest.raises(sv.SvError):  # misaligned row pitch
        sv.sv_softmax_stats(z, sv.SV_BF16, 63, 60, z, 0, 2, 4, z, z, z, z, ws, nb)
    with pytest.raises(sv.SvError):  # unknown dtype
        sv.sv_softmax_stats(z, 7, 64, 60, z, 0, 2, 4, z, z, z, z, ws, nb)
    with pytest.raises(sv.SvError):  # workspace too small
        sv.sv_mixture_q(z, sv.SV_BF16, 64, 64, 8, 16, z, z, 2, 32, z, z, z, z, ws, 256)


# ---------------------------------------------------------------- whole steps
SMALL = [
    (1, dict(steps=20)),                           # tiny fp32, T=1 x3 and greedy (the full workload)
    (2, dict(V=2053, R=4)),                        # independent draft, ragged V
    (3, dict(V=2053, R=8, steps=3)),               # DVL + independent draft
    (4, dict(V=4099, R=4)),                        # mixture, T=1.5, top-p
    (5, dict(V=4099, R=8, steps=4)),               # DVL + mixture + top-p
    (5, dict(V=64, R=64, steps=3)),                # many requests, tiny vocabulary
]


@pytest.mark.parametrize("c,kw", SMALL, ids=[f"cfg{c}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for c, kw in SMALL])
def test_config_small(c, kw):
    w = synth.config(c, **kw)
    vs, run = gpu_step_runner(w)
    rep = None
    for s in range(w.steps):
        banner(f"{w.name} V={w.V} R={w.R} step={s}")
        g = run(s)
        rep = compare_step(w, g, oracle_step(w, s), rep)
    if c == 1:  # cfg1 at its own size
        log_parity(f"{w.name} full size, standalone, {w.steps} steps", rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


FULL = [(2, 4), (3, 4), (4, 5)]  # (config, steps)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("c,steps", FULL, ids=[f"cfg{c}-{s}steps" for c, s in FULL])
@pytest.mark.parametrize("fused", [False, True], ids=["standalone", "fused"])
def test_config_full_size(c, steps, fused):
    """Full-size cfg2, cfg3 and cfg4 over several steps, on the standalone
    chain and on the fused calls, every step against the oracle."""
    w = synth.config(c, steps=steps)
    vs, run = gpu_step_runner(w, fused=fused)
    rep, cache = None, {}
    for s in range(steps):
        banner(f"{w.name} full size {'fused' if fused else 'standalone'} step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s, cache), rep)
    log_parity(f"{w.name} full size, {'fused' if fused else 'standalone'}, {steps} steps", rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


@pytest.mark.timeout(900)
def test_config5_full_size_200_steps():
    """The headline workload (conc 32, V 151936, K 8 greedy-branch mixture, DVL
    256, top-p 0.95) over its 200 steps on the calls the benchmark times
    (dvl_alloc_pack, sv_verify_rows, sv_accept_sample): every step against the
    oracle.  The standalone chain runs the same steps, checked against the
    oracle on a sample of them and for DVL, branch tokens and invariants on
    the rest."""
    steps = int(os.environ.get("SV_CFG5_STEPS", "200"))
    w = synth.config(5, steps=steps)
    R, b, K, V = w.R, w.b, w.K, w.V
    cache = {}
    _, run_fused = gpu_step_runner(w, fused=True)
    rep = None
    for s in range(steps):
        if s % 20 == 0:
            banner(f"{w.name} fused step {s}/{steps}")
        rep = compare_step(w, run_fused(s), oracle_step(w, s, cache), rep)
    log_parity(f"{w.name} fused (the benchmark's calls), all {steps} steps", rep)
    assert_rate(rep)
    assert excused(rep) <= 5
    vs, run = gpu_step_runner(w)
    g_all = oracle.argmax_rows(w.comp.reshape(-1, V)).reshape(R, K, b)
    sample = set(np.linspace(0, steps - 1, min(steps, 12)).astype(int).tolist())
    rep = None
    for s in range(steps):
        if s % 20 == 0:
            banner(f"{w.name} standalone step {s}/{steps}")
        g = run(s)
        if s in sample:
            rep = compare_step(w, g, oracle_step(w, s, cache), rep)
            continue
        dv = oracle.dvl(w.a[s], w.budget)
        assert np.array_equal(g["L"], dv["L"]) and np.array_equal(g["tgt_off"], dv["tgt_off"])
        for r in range(R):
            Lr = dv["L"][r]
            assert np.array_equal(g["branch_tok"][r, :, :Lr], g_all[r, :, :Lr])
        assert np.all((g["n_acc"] >= 0) & (g["n_acc"] <= g["L"]))
        assert np.array_equal(g["is_bonus"], (g["n_acc"] == g["L"]).astype(np.int32))
        assert np.all((g["token"] >= 0) & (g["token"] < V))
    log_parity(f"{w.name} standalone, {len(sample)} sampled steps of {steps}", rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


def test_edge_steps_all_accept_all_reject_empty():
    """Greedy drafts that match the target argmax (all accepted, bonus), draft
    tokens outside the nucleus (first position rejected), and requests that
    DVL gives no slots (L_r = 0: one token from p_1)."""
    w = synth.config(5, V=1031, R=8, steps=1)
    R, b, K = w.R, w.b, w.K
    tv = synth.values(w.tgt)
    # requests 0-1: greedy target with drafts equal to the target argmax
    w.T[:2] = 0.0
    w.x[0, :2] = np.argmax(tv[:2, :b], axis=-1)
    # make those drafts the greedy branches of every component
    comp = synth.values(w.comp).copy()
    for r in range(2):
        for i in range(b):
            comp[r, :, i, w.x[0, r, i]] = comp[r, :, i].max() + 1.0
    w.comp = synth.f32_to_bf16_bits(comp)
    # request 2: tiny nucleus, draft outside it
    w.top_p[2] = 1e-6
    # requests 5-7: scores near zero so DVL starves them
    w.a[0, 5:] = 1e-3
    w.budget = 40
    vs, run = gpu_step_runner(w)
    banner("edge steps: all-accept / all-reject / empty")
    g = run(0)
    o = oracle_step(w, 0)
    rep = compare_step(w, g, o)
    assert_rate(rep)
    assert g["n_acc"][0] == g["L"][0] and g["is_bonus"][0] == 1
    assert (g["L"][5:] == 0).all()


@pytest.mark.parametrize("c", [3, 5])
def test_two_stream_step_matches_oracle(c):
    """Target-row statistics on a second stream, concurrent with the proposal."""
    w = synth.config(c, V=4099, R=16, steps=3)
    vs, run = gpu_step_runner(w, two_streams=True)
    rep = None
    for s in range(w.steps):
        banner(f"two streams {w.name} step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s), rep)
    assert_rate(rep)


FUSED = [(1, dict()), (2, dict(V=2053, R=4)), (3, dict(V=2053, R=8, steps=3)),
         (4, dict(V=4099, R=4)), (5, dict(V=4099, R=8, steps=4)), (5, dict(V=1031, R=48, steps=2)),
         (5, dict(steps=6)),
         # tiny rows: more row slices than 8-value vectors (empty slices), a
         # row shorter than one vector, and a vector plus a ragged tail
         (3, dict(V=13, R=2, steps=2)), (3, dict(V=7, R=2, steps=2)), (2, dict(V=8, R=1))]


@pytest.mark.parametrize("c,kw", FUSED, ids=[f"cfg{c}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for c, kw in FUSED])
def test_fused_rows_mixture_matches_oracle(c, kw):
    """The fused path: sv_verify_rows (mixture) and sv_accept_sample."""
    w = synth.config(c, **kw)
    vs, run = gpu_step_runner(w, fused=True)
    rep = None
    for s in range(w.steps):
        banner(f"fused {w.name} V={w.V} R={w.R} step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s), rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


@pytest.mark.parametrize("fused", [False, True])
def test_mixture_without_top_p_matches_oracle(fused):
    """The mixture proposal with no top-p: the draw's sums take every value
    (no cut) and still apply the branch-token corrections of the residual."""
    w = synth.config(5, V=4099, R=8, steps=3)
    w.top_p = None
    vs, run = gpu_step_runner(w, fused=fused)
    rep = None
    for s in range(w.steps):
        banner(f"mixture without top-p fused={fused} step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s), rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


def _random_workloads(seed, n):
    """Seeded draws over config, vocabulary, request count, soft or greedy
    branches, per-request block lengths, top-p on or off and the fused or
    separate calls."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        c = int(rng.choice([1, 2, 3, 4, 5]))
        V = int(rng.choice([7, 13, 64, 257, 1031, 2053, 4099, 9001, 32768]))
        R = int(rng.integers(1, 24)) if V <= 10000 else int(rng.integers(2, 12))
        soft = c in (4, 5) and rng.random() < 0.4
        bt = float(rng.choice([0.3, 1.0, 2.0])) if soft else 0.0
        ragged = bool(rng.random() < 0.3)
        fused = bool(rng.random() < 0.6) or soft
        topp_off = c in (4, 5) and rng.random() < 0.3
        out.append((c, V, R, bt, ragged, fused, topp_off))
    return out


@pytest.mark.parametrize("seed", [101, 202, 303])
def test_random_workloads_match_oracle(seed):
    """Twenty seeded random small workloads per seed (two steps each) against
    the oracle, under the usual bar."""
    for c, V, R, bt, ragged, fused, topp_off in _random_workloads(seed, 20):
        w = synth.config(c, V=V, R=R, steps=2, branch_T=bt, ragged=ragged)
        if topp_off:
            w.top_p = None
        banner(f"random cfg{c} V={V} R={R} T_b={bt} ragged={ragged} fused={fused} top-p off={topp_off}")
        vs, run = gpu_step_runner(w, fused=fused)
        rep = None
        for s in range(w.steps):
            rep = compare_step(w, run(s), oracle_step(w, s), rep)
        assert_rate(rep)
        assert _sv().sv_get_status(vs.ws) == 0


def test_determinism_repeat_runs():
    w = synth.config(4, V=8191, R=4)
    vs, run = gpu_step_runner(w)
    banner("determinism")
    a = run(0)
    b = run(0)
    for k in a:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k


# ---------------------------------------------------------------- whole step in a HIP graph
GRAPH = [(3, dict(V=2053, R=8, steps=4)), (5, dict(V=4099, R=8, steps=4)), (4, dict(V=4099, R=4, steps=2)),
         (2, dict(V=2053, R=4, steps=2)), (5, dict(steps=4)), (5, dict(V=4099, R=8, steps=3, branch_T=1.0))]


def _same_bits(a: dict, b: dict):
    """Bitwise equality over the entries a step defines (positions i < L_r,
    packed rows below tgt_off[R], draft rows below pos_off[R]); the rest keep
    whatever earlier steps left there."""
    L = a["L"]
    assert np.array_equal(L, b["L"]), "L"
    n_rows, n_pos = int(a["tgt_off"][-1]), int(a["pos_off"][-1])
    pos_mask = np.arange(a["u_acc"].shape[1])[None, :] < L[:, None]
    for k in a:
        x, y = np.asarray(a[k]), np.asarray(b[k])
        if k.startswith("row_"):
            x, y = x[:n_rows], y[:n_rows]
        elif k.startswith("d_"):
            x, y = x[:n_pos], y[:n_pos]
        elif k in ("p_x", "q_x", "u_acc", "q_at_draft"):
            x, y = x[pos_mask], y[pos_mask]
        elif k == "post_w":
            x, y = x[pos_mask], y[pos_mask]
        elif k == "branch_tok":
            x, y = x.transpose(0, 2, 1)[pos_mask], y.transpose(0, 2, 1)[pos_mask]
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k


@pytest.mark.parametrize("c,kw", GRAPH, ids=[f"cfg{c}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for c, kw in GRAPH])
def test_graph_replay_matches_eager_and_oracle(c, kw):
    """One captured graph (DVL, device-side packing by the new offsets, the
    verification calls) replayed for several steps whose inputs are written to
    the same addresses: every replay equals the eager run bit for bit and
    passes the oracle comparison, with unrelated eager work and
    synchronisations between replays."""
    import torch

    w = synth.config(c, **kw)
    banner(f"graph capture {w.name} V={w.V} R={w.R}")
    _, _, run_graph = gpu_graph_runner(w)
    _, run_eager = gpu_step_runner(w, fused=True)
    order = [s % w.steps for s in (1, 0, 2, 3, 1)]
    rep = None
    lengths = set()
    for s in order:
        banner(f"graph replay {w.name} step {s}")
        g = run_graph(s)
        noise = torch.randn(1 << 20, device="cuda")
        float((noise * noise).sum())
        torch.cuda.synchronize()
        _same_bits(g, run_eager(s))
        rep = compare_step(w, g, oracle_step(w, s), rep)
        lengths.add(tuple(g["L"].tolist()))
    assert_rate(rep)
    if w.budget is not None and w.steps > 1:
        assert len(lengths) > 1, "the steps should change the DVL boundaries"


@pytest.mark.parametrize("c,kw", [(5, dict(V=4099, R=8, steps=3)), (3, dict(V=2053, R=16, steps=2)), (5, dict(steps=2))],
                         ids=["cfg5-small", "cfg3-small", "cfg5-full"])
def test_graph_replay_budget_changes(c, kw):
    """The verification budget sits at a fixed device address: one graph
    captured at budget B (its capacity) replays at other budgets, down to 0
    (every request then emits one token from its first target row), without
    recapture; each replay matches the eager run and the oracle."""
    w = synth.config(c, **kw)
    B = w.budget
    banner(f"graph budgets {w.name} V={w.V} R={w.R} capacity {B}")
    _, _, run_graph = gpu_graph_runner(w)
    _, run_eager = gpu_step_runner(w, fused=True)
    rep = None
    for k, budget in enumerate([B // 2, 0, B, 1, B - 3, w.R]):
        s = k % w.steps
        w.budget = budget
        banner(f"graph replay {w.name} step {s} budget {budget}")
        g = run_graph(s)
        _same_bits(g, run_eager(s))
        assert int(g["pos_off"][-1]) == min(budget, w.R * w.b)
        rep = compare_step(w, g, oracle_step(w, s), rep)
    assert_rate(rep)


# ---------------------------------------------------------------- soft branches
SOFT = [(4, dict(V=4099, R=4, branch_T=1.0)), (5, dict(V=4099, R=8, steps=3, branch_T=0.7)),
        (5, dict(V=1031, R=16, steps=2, branch_T=2.0)), (4, dict(V=64, R=8, steps=2, branch_T=0.3)),
        (4, dict(branch_T=1.0)), (5, dict(steps=3, branch_T=1.0))]


@pytest.mark.parametrize("c,kw", SOFT, ids=[f"cfg{c}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for c, kw in SOFT])
def test_soft_branches_match_oracle(c, kw):
    """Soft-branch mixture (each branch softmax(c / T_b), drafts sampled from
    it): branch argmax, posterior, q at the drafts, decisions and the dense
    K-row residual against the oracle."""
    w = synth.config(c, **kw)
    vs, run = gpu_step_runner(w)
    rep = None
    for s in range(w.steps):
        banner(f"soft {w.name} V={w.V} R={w.R} step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s), rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


@pytest.mark.parametrize("K,top_p", [(3, 0.95), (12, 0.95), (2, None)])
def test_soft_branches_other_component_counts(K, top_p):
    """Soft branches with K below the eight branch rows the nucleus-list sums
    hold (rows past K unused), above them (the per-group sums in passes of
    eight branches), and without top-p (every value in the nucleus)."""
    w = synth.make(f"soft-K{K}", R=8, V=4099, K=K, T=1.0, top_p=top_p, budget=64, seed=1200 + K, vseed=7,
                   steps=2, branch_T=1.0)
    vs, run = gpu_step_runner(w)
    rep = None
    for s in range(w.steps):
        banner(f"soft K={K} top_p={top_p} step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s), rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


def test_soft_branches_per_request_temperatures():
    """T_b per request, some 0 (point-mass branches, drafts from greedy
    branches) and some soft, in one step."""
    w = synth.config(5, V=4099, R=8, steps=3, branch_T=1.0)
    tb = np.array([1.0, 0.0, 0.5, 0.0, 2.0, 1.5, 0.0, 0.25], np.float32)
    w.branch_T = tb
    for s in range(w.steps):
        for r in np.nonzero(tb == 0)[0]:
            w.x[s, r] = w.branch_tok[r, (s + r) % w.K]
    vs, run = gpu_step_runner(w)
    rep = None
    for s in range(w.steps):
        banner(f"soft per-request T_b step {s}")
        rep = compare_step(w, run(s), oracle_step(w, s), rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


# ---------------------------------------------------------------- per-request block length
RAGGED = [(3, dict(V=2053, R=8, steps=3)), (5, dict(V=4099, R=8, steps=3)), (4, dict(V=4099, R=6)),
          (2, dict(V=2053, R=6)), (1, dict()), (5, dict(steps=2)), (5, dict(V=4099, R=8, steps=2, branch_T=1.0))]


@pytest.mark.parametrize("c,kw", RAGGED, ids=[f"cfg{c}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for c, kw in RAGGED])
def test_ragged_block_lengths_match_oracle(c, kw):
    """Every request drafted its own number b_r of positions (some 0): DVL
    chooses among drafted positions only, or all b_r are verified without a
    budget; the whole step against the oracle."""
    w = synth.config(c, ragged=True, **kw)
    vs, run = gpu_step_runner(w, fused=True)
    rep = None
    for s in range(w.steps):
        banner(f"ragged {w.name} V={w.V} R={w.R} b_r={w.block_len.tolist()} step {s}")
        g = run(s)
        assert (g["L"] <= w.block_len).all()
        rep = compare_step(w, g, oracle_step(w, s), rep)
    assert_rate(rep)
    assert _sv().sv_get_status(vs.ws) == 0


def test_graph_replay_block_lengths_change():
    """Block lengths, like the budget, sit at fixed addresses: one captured
    graph replays with new b_r per step."""
    w = synth.config(5, V=4099, R=8, steps=3, ragged=True)
    _, _, run_graph = gpu_graph_runner(w)
    _, run_eager = gpu_step_runner(w, fused=True)
    rng = np.random.default_rng(17)
    rep = None
    for k in range(5):
        s = k % w.steps
        w.block_len = rng.integers(0, w.b + 1, size=w.R).astype(np.int32)
        if k == 1:
            w.block_len[:] = 0
        banner(f"graph replay ragged step {s} b_r={w.block_len.tolist()}")
        g = run_graph(s)
        _same_bits(g, run_eager(s))
        rep = compare_step(w, g, oracle_step(w, s), rep)
    assert_rate(rep)


# ---------------------------------------------------------------- temperature / category-temperature sweep
def test_sweep_points_match_oracle():
    """The sweep's steps (K = 1 and K = 8 greedy branches, category temperature
    ZT applied to the mixing logits, ZT = 0 giving -inf logits off the argmax
    category, target temperatures 0 to 2) against the oracle."""
    from draft_verification_sv_amd import sweep

    temps = (0.0, 1.0, 2.0)
    rep = None
    for K, ZT in ((1, 0.0), (8, 0.0), (8, 0.6), (8, 1.4)):
        w = sweep.workload(K, ZT, V=1031, R=8, steps=2)
        banner(f"sweep K={K} ZT={ZT}")
        res = sweep.verify_steps(w, temps)
        for T in temps:
            w.T = np.full(w.R, T, np.float32)
            for s in range(w.steps):
                rep = compare_step(w, res[T][s], oracle_step(w, s), rep)
    assert_rate(rep)


# ---------------------------------------------------------------- the library's double exponential
def test_table_exp_error_against_host_exp():
    """exp_tab (Tang's table method) over the probabilities' argument range
    [-746, 0] and a little above 0: within 3 ulp of the host's exp for normal
    results, 2 units of the smallest subnormal below them; exp(0) = 1,
    exp(-inf) = 0, NaN stays NaN, arguments below -746 give 0."""
    import torch

    sv = _sv()
    rng = np.random.default_rng(23)
    xs = np.concatenate([
        -np.linspace(0.0, 746.0, 400001), rng.uniform(-40.0, 0.0, 200000), -rng.uniform(0, 1e-6, 1000),
        -(2.0 ** -np.arange(1, 1075, dtype=np.float64)), rng.uniform(0.0, 1e-3, 1000),
        np.array([0.0, -0.0, -708.39, -708.4, -744.4, -745.13, -745.14, -745.2, -746.0, -746.5, -1e5, -np.inf]),
    ])
    banner(f"exp_tab on {xs.size} arguments")
    xt = torch.from_numpy(xs).cuda()
    out = torch.empty_like(xt)
    sv.sv_selftest_exp(xt, out, xs.size)
    got = out.cpu().numpy()
    ref = np.exp(xs)
    normal = ref >= np.finfo(np.float64).tiny
    ulps = np.abs(got[normal] - ref[normal]) / np.spacing(ref[normal])
    assert ulps.max() <= 3.0, f"max {ulps.max()} ulp at x = {xs[normal][np.argmax(ulps)]}"
    sub = ~normal
    assert np.all(np.abs(got[sub] - ref[sub]) <= 2 * 2.0 ** -1074)
    assert got[xs == 0.0].tolist() == [1.0] * int((xs == 0.0).sum())
    assert got[np.isneginf(xs)].tolist() == [0.0]
    assert np.all(got[xs < -746.0] == 0.0)
    nan = torch.tensor([np.nan], dtype=torch.float64).cuda()
    o1 = torch.empty_like(nan)
    sv.sv_selftest_exp(nan, o1, 1)
    assert np.isnan(o1.cpu().numpy()[0])
    print(f"\n[exp_tab] max error {ulps.max():.2f} ulp, mean {ulps.mean():.3f} ulp", flush=True)
