"""Pins of the CPU oracle to what the pages and the mathematics fix.

CPU only.  Each test checks the oracle against something other than itself:
published known-answer vectors, library routines on special cases, closed
forms, brute-force enumeration on tiny inputs, and distributional invariants
of speculative sampling (DBLast review, "Assumptions": rejection correction
keeps the target distribution for any proposal q).
"""
import itertools
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def np_target(l, T, top_p=1.0):
    """Target distribution from library routines: scipy softmax, numpy stable
    argsort and cumsum for the nucleus (reference graph [18] of the DBLast
    review).  Returns (p, cut)."""
    l = np.asarray(l, dtype=np.float64)
    if T == 0:
        p = np.zeros_like(l)
        p[np.argmax(l)] = 1.0
        return p, l.max()
    p = special.softmax(l / T)
    if top_p >= 1.0:
        return p, -np.inf
    order = np.argsort(-l, kind="stable")
    c = np.cumsum(p[order])
    k = min(int(np.searchsorted(c, top_p, side="left")), len(l) - 1)
    cut = l[order[k]]
    q = np.where(l >= cut, p, 0.0)
    return q / q.sum(), cut


def sample_idx(rng, probs, n):
    c = np.cumsum(probs)
    c /= c[-1]
    return np.minimum(np.searchsorted(c, rng.random(n), side="right"), len(probs) - 1).astype(np.int32)


def chi2_check(counts, probs, alpha=1e-4):
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.sum()
    nz = probs > 0
    assert counts[~nz].sum() == 0, "tokens outside the target support were emitted"
    expct = n * probs[nz]
    chi2 = float(((counts[nz] - expct) ** 2 / expct).sum())
    crit = float(stats.chi2.isf(alpha, int(nz.sum()) - 1))
    assert chi2 < crit, f"chi2 {chi2:.2f} >= critical {crit:.2f}"
    return chi2


def bincount(tok, V):
    return np.bincount(tok, minlength=V)[:V]


# ---------------------------------------------------------------- Philox
def _kat():
    rows = []
    with open(os.path.join(GOLD, "philox_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                v = [int(t, 16) for t in line.split()]
                rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(ctr, key, expect):
    assert list(oracle.philox4x32_10(ctr, key)) == expect


def test_uniform_grid_endpoints():
    assert oracle.u24(0) == 0.0
    assert oracle.u24(0xFF) == 0.0
    assert oracle.u24(0x100) == 2.0 ** -24
    assert oracle.u24(0xFFFFFFFF) == 1.0 - 2.0 ** -24


def test_uniform_counter_layout():
    seed = 0x0123456789ABCDEF
    w = oracle.uniform_words(seed, 3, 5)
    for r in range(3):
        for i in range(5):
            ref = oracle.philox4x32_10([i, r, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
            assert list(w[r, i]) == list(ref)


# ---------------------------------------------------------------- row statistics
@pytest.mark.parametrize("V", [1, 7, 1000, 1031])
@pytest.mark.parametrize("T", [0.5, 1.0, 1.5])
@pytest.mark.parametrize("top_p", [1.0, 0.95, 0.5, 0.05])
@pytest.mark.parametrize("bf16", [False, True])
def test_row_stats_vs_library(V, T, top_p, bf16):
    rng = np.random.default_rng(V * 7 + int(T * 10) + int(top_p * 100))
    l32 = (3.0 * rng.standard_normal(V)).astype(np.float32)
    row = synth.f32_to_bf16_bits(l32) if bf16 else l32
    lv = synth.values(row).astype(np.float64)
    st = oracle.row_stats(row, T, top_p)
    assert st["max"] == lv.max()
    assert st["argmax"] == int(np.argmax(lv))
    assert st["lse"] == pytest.approx(special.logsumexp(lv / T), rel=1e-13, abs=1e-13)
    p, cut = np_target(lv, T, top_p)
    if top_p >= 1:
        assert st["cut"] == -np.inf
        assert st["kept_lse"] == st["lse"]
    else:
        assert st["cut"] == cut
        assert st["kept_lse"] == pytest.approx(special.logsumexp(lv[lv >= cut] / T), rel=1e-13, abs=1e-13)
        full = special.softmax(lv / T)
        assert full[lv >= cut].sum() >= top_p - 1e-12   # kept mass reaches top_p
        assert full[lv > cut].sum() < top_p + 1e-12     # strictly-above-cut mass does not


def test_row_stats_constant_row_closed_form():
    V, c, T = 1000, -2.5, 0.7
    row = np.full(V, c, np.float32)
    for tp in (1.0, 0.3, 1e-6):
        st = oracle.row_stats(row, T, tp)
        assert st["argmax"] == 0 and st["max"] == c
        assert st["lse"] == pytest.approx(c / T + np.log(V), rel=1e-14)
        assert st["kept_lse"] == pytest.approx(c / T + np.log(V), rel=1e-14)  # ties all kept
        if tp < 1:
            assert st["cut"] == c


def test_row_stats_two_level_closed_form():
    # n1 tokens at value a, n2 tokens at value c < a: mass of the top level is
    # n1 e^{a/T} / (n1 e^{a/T} + n2 e^{c/T}); the cut is a iff top_p <= that mass.
    n1, n2, a, c, T = 3, 997, 2.0, -1.0, 1.0
    row = np.full(n1 + n2, c, np.float32)
    row[[5, 400, 999]] = a
    top_mass = n1 * np.exp(a / T) / (n1 * np.exp(a / T) + n2 * np.exp(c / T))
    st = oracle.row_stats(row, T, top_mass * 0.999)
    assert st["cut"] == a and st["argmax"] == 5
    assert st["kept_lse"] == pytest.approx(np.log(n1) + a / T, rel=1e-14)
    st = oracle.row_stats(row, T, min(top_mass * 1.001, 0.99))
    assert st["cut"] == c


def test_row_stats_greedy():
    row = np.array([1.0, 3.0, -2.0, 3.0], np.float32)
    st = oracle.row_stats(row, 0.0, 0.9)
    assert st["argmax"] == 1 and st["max"] == 3.0 and st["lse"] == 0.0 and st["cut"] == 3.0


def test_argmax_rows_lowest_index():
    rows = np.array([[0, 5, 5, 1], [7, 7, 7, 7], [-1, -3, -1, -2]], np.float32)
    assert list(oracle.argmax_rows(rows)) == [1, 0, 0]
    assert list(oracle.argmax_rows(synth.f32_to_bf16_bits(rows))) == [1, 0, 0]


# ---------------------------------------------------------------- greedy verification
def test_greedy_is_longest_argmax_prefix():
    """T = 0: accepted length = longest prefix of draft tokens equal to the
    target argmax (ties: lowest index); the extra token is the argmax of the
    next target row, as residual and as bonus (DBLast review, Referee report:
    the high-determinism regime)."""
    rng = np.random.default_rng(5)
    R, b, V = 40, 6, 7
    tgt = rng.integers(-3, 3, size=(R, b + 1, V)).astype(np.float32)  # many ties
    am = np.argmax(tgt, axis=-1)
    k = rng.integers(0, b + 1, size=R)
    x = am[:, :b].copy()
    for r in range(R):
        if k[r] < b:
            x[r, k[r]] = (am[r, k[r]] + 1 + rng.integers(0, V - 1)) % V
    # greedy draft rows whose argmax is the draft token
    draft = np.zeros((R, b, V), np.float32)
    draft[np.arange(R)[:, None], np.arange(b)[None, :], x] = 1.0
    out = oracle.step(tgt=tgt.reshape(-1, V), tgt_row0=np.arange(R) * (b + 1), L=np.full(R, b),
                      T=np.zeros(R), x=x, seed=9, draft=draft.reshape(-1, V), draft_row0=np.arange(R) * b)
    for r in range(R):
        n = 0
        while n < b and x[r, n] == am[r, n]:
            n += 1
        assert out["n_acc"][r] == n
        assert out["token"][r] == am[r, n]
        assert out["is_bonus"][r] == (n == b)


# ---------------------------------------------------------------- distribution preservation
N_TRIALS = 1_000_000


def _dense_run(rng, V, b, T, top_p, seed):
    tl = (1.5 * rng.standard_normal((b + 1, V))).astype(np.float32)
    dl = (tl[:b] + rng.standard_normal((b, V))).astype(np.float32)
    q = [special.softmax(dl[i].astype(np.float64) / T) for i in range(b)]
    x = np.stack([sample_idx(rng, q[i], N_TRIALS) for i in range(b)], axis=1)
    n = N_TRIALS
    out = oracle.step(tgt=tl, tgt_row0=np.zeros(n, np.int64), L=np.full(n, b), T=np.full(n, T),
                      top_p=None if top_p >= 1 else np.full(n, top_p), x=x, seed=seed,
                      draft=dl, draft_row0=np.zeros(n, np.int64))
    return tl, dl, q, x, out


@pytest.mark.parametrize("T,top_p", [(1.0, 1.0), (0.7, 0.8)])
def test_chi2_dense_first_and_second_token(T, top_p):
    rng = np.random.default_rng(11 if top_p >= 1 else 12)
    V, b = 8, 2
    tl, dl, q, x, out = _dense_run(rng, V, b, T, top_p, seed=77)
    n_acc, tok = out["n_acc"], out["token"]
    first = np.where(n_acc >= 1, x[:, 0], tok)
    chi2_check(bincount(first, V), np_target(tl[0], T, top_p)[0])
    sel = n_acc >= 1
    second = np.where(n_acc[sel] >= 2, x[sel, 1], tok[sel])
    chi2_check(bincount(second, V), np_target(tl[1], T, top_p)[0])


def test_chi2_residual_given_rejection():
    rng = np.random.default_rng(13)
    V, b, T = 8, 1, 1.0
    tl, dl, q, x, out = _dense_run(rng, V, b, T, 1.0, seed=78)
    rej = out["n_acc"] == 0
    p = np_target(tl[0], T)[0]
    res = np.maximum(p - q[0], 0.0)
    chi2_check(bincount(out["token"][rej], V), res / res.sum())
    assert not out["is_bonus"][rej].any()


def test_expected_accepted_length_closed_form():
    """E[n_acc] = sum_l prod_{i<=l} alpha_i and P(n_acc >= l) = prod_{i<=l}
    alpha_i, alpha_i = sum_v min(p_i, q_i), for an independent draft."""
    rng = np.random.default_rng(14)
    V, b, T = 8, 4, 1.0
    tl, dl, q, x, out = _dense_run(rng, V, b, T, 1.0, seed=79)
    alpha = np.array([np.minimum(np_target(tl[i], T)[0], q[i]).sum() for i in range(b)])
    surv = np.cumprod(alpha)
    n_acc = out["n_acc"].astype(np.float64)
    se = n_acc.std() / np.sqrt(len(n_acc))
    assert abs(n_acc.mean() - surv.sum()) < 5 * se
    for l in range(1, b + 1):
        frac = (n_acc >= l).mean()
        se_l = np.sqrt(surv[l - 1] * (1 - surv[l - 1]) / len(n_acc))
        assert abs(frac - surv[l - 1]) < 5 * se_l + 1e-12


def _mixture_run(rng, V, b, K, T, top_p, branch_T, seed):
    tl = (1.5 * rng.standard_normal((b + 1, V))).astype(np.float32)
    comp = (tl[None, :b] + 1.2 * rng.standard_normal((K, b, V))).astype(np.float32)
    mix = rng.standard_normal(K).astype(np.float32)
    n = N_TRIALS
    z = sample_idx(rng, special.softmax(mix.astype(np.float64)), n)
    if branch_T == 0:
        g = np.argmax(comp, axis=-1)  # [K, b]
        x = g[z].astype(np.int32)
    else:
        x = np.empty((n, b), np.int32)
        for zz in range(K):
            sel = np.nonzero(z == zz)[0]
            for i in range(b):
                x[sel, i] = sample_idx(rng, special.softmax(comp[zz, i].astype(np.float64) / branch_T), len(sel))
    out = oracle.step(tgt=tl, tgt_row0=np.zeros(n, np.int64), L=np.full(n, b), T=np.full(n, T),
                      top_p=None if top_p >= 1 else np.full(n, top_p), x=x, seed=seed,
                      comp=comp.reshape(K * b, V), comp_row0=np.zeros(n, np.int64),
                      mix=np.tile(mix, (n, 1)), branch_T=branch_T)
    return tl, comp, mix, x, out


@pytest.mark.parametrize("branch_T,T,top_p", [(0.0, 1.0, 1.0), (0.0, 1.5, 0.95), (1.0, 1.0, 1.0)])
def test_chi2_mixture_first_and_second_token(branch_T, T, top_p):
    """Greedy-branch and soft-branch latent mixtures (DBLast review, "What
    carries the argument"; Referee report, minor 1 and 5): with the posterior
    along the accepted prefix, the emitted tokens follow the target."""
    rng = np.random.default_rng(21 + int(branch_T))
    V, b, K = 8, 2, 2
    tl, comp, mix, x, out = _mixture_run(rng, V, b, K, T, top_p, branch_T, seed=80)
    n_acc, tok = out["n_acc"], out["token"]
    first = np.where(n_acc >= 1, x[:, 0], tok)
    chi2_check(bincount(first, V), np_target(tl[0], T, top_p)[0])
    sel = n_acc >= 1
    second = np.where(n_acc[sel] >= 2, x[sel, 1], tok[sel])
    chi2_check(bincount(second, V), np_target(tl[1], T, top_p)[0])


# ---------------------------------------------------------------- mixture posterior
@pytest.mark.parametrize("branch_T", [0.0, 0.8])
def test_mixture_posterior_brute_force(branch_T):
    """K = 2, b = 3, V = 4: q(x_i | x_<i) and P(z | x_<i) from summing the full
    joint pi_z prod_i q_i(x_i | z) over every completion of the block."""
    rng = np.random.default_rng(31)
    K, b, V = 2, 3, 4
    comp = rng.standard_normal((K, b, V)).astype(np.float32)
    mix = rng.standard_normal(K).astype(np.float32)
    pi = special.softmax(mix.astype(np.float64))
    if branch_T == 0:
        qz = np.zeros((K, b, V))
        g = np.argmax(comp, axis=-1)
        for z in range(K):
            for i in range(b):
                qz[z, i, g[z, i]] = 1.0
    else:
        qz = special.softmax(comp.astype(np.float64) / branch_T, axis=-1)
    seqs = np.array(list(itertools.product(range(V), repeat=b)), np.int32)
    joint = np.zeros((K, len(seqs)))
    for z in range(K):
        joint[z] = pi[z] * np.prod(qz[z, np.arange(b)[None, :], seqs], axis=1)
    R = len(seqs)
    tl = rng.standard_normal((b + 1, V)).astype(np.float32)
    out = oracle.step(tgt=tl, tgt_row0=np.zeros(R, np.int64), L=np.full(R, b), T=np.ones(R), x=seqs,
                      seed=3, comp=comp.reshape(K * b, V), comp_row0=np.zeros(R, np.int64),
                      mix=np.tile(mix, (R, 1)), branch_T=branch_T)
    for r, xs in enumerate(seqs):
        for i in range(b):
            pre = np.all(seqs[:, :i] == xs[:i], axis=1)        # completions sharing x_<i
            upto = pre & (seqs[:, i] == xs[i])                  # ... and x_i
            P_pre = joint[:, pre].sum()
            if P_pre == 0:
                assert out["q_x"][r, i] == 0.0
                assert np.all(out["post_w"][r, i] == 0.0)
                continue
            assert out["q_x"][r, i] == pytest.approx(joint[:, upto].sum() / P_pre, abs=1e-12)
            post = joint[:, pre].sum(axis=1) / P_pre
            np.testing.assert_allclose(out["post_w"][r, i], post, atol=1e-12)


def test_mixture_single_component_is_independent_draft():
    """K = 1 reduces the mixture to the independent draft (DBLast review,
    "What would settle it": the K = 1 DFlash baseline)."""
    rng = np.random.default_rng(32)
    R, b, V, T = 50, 4, 16, 1.0
    tl = rng.standard_normal((R * (b + 1), V)).astype(np.float32)
    comp = rng.standard_normal((R * b, V)).astype(np.float32)
    x = rng.integers(0, V, size=(R, b)).astype(np.int32)
    common = dict(tgt=tl, tgt_row0=np.arange(R) * (b + 1), L=np.full(R, b), T=np.full(R, T), x=x, seed=4)
    mixo = oracle.step(**common, comp=comp, comp_row0=np.arange(R) * b, mix=np.zeros((R, 1)), branch_T=T)
    dens = oracle.step(**common, draft=comp, draft_row0=np.arange(R) * b)
    np.testing.assert_allclose(mixo["q_x"], dens["q_x"], rtol=1e-12)
    for k in ("n_acc", "token", "is_bonus"):
        assert np.array_equal(mixo[k], dens[k])


# ---------------------------------------------------------------- DVL
def _brute_dvl(s, B):
    R, b = s.shape
    pref = np.concatenate([np.zeros((R, 1)), np.cumsum(s.astype(np.float64), axis=1)], axis=1)
    best, arg, count = -1.0, None, 0
    for L in itertools.product(range(b + 1), repeat=R):
        if sum(L) > B:
            continue
        obj = sum(pref[r, L[r]] for r in range(R))
        if obj > best + 1e-15:
            best, arg, count = obj, L, 1
        elif abs(obj - best) <= 1e-15:
            count += 1
    return best, np.array(arg), count


def test_dvl_brute_force_optimum():
    """DScale abstract: DVL spends a budget of verification slots on the
    best-scored prefixes; with survival scores s_i = prod_{j<=i} a_j the
    allocation maximises the expected number of accepted positions; checked
    against exhaustive search."""
    rng = np.random.default_rng(41)
    for trial in range(120):
        R, b = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        if trial % 3 == 0:
            a = rng.choice([0.0, 0.25, 0.5, 1.0], size=(R, b)).astype(np.float32)  # exact ties
        else:
            a = rng.beta(8, 2, size=(R, b)).astype(np.float32)
        for B in range(0, R * b + 2):
            o = oracle.dvl(a, B)
            assert o["bad"] == 0
            np.testing.assert_array_equal(o["s"], np.cumprod(a, axis=1, dtype=np.float32))
            best, arg, count = _brute_dvl(o["s"], B)
            assert o["L"].sum() == min(B, R * b)
            assert oracle.dvl_objective(o["s"], o["L"]) == pytest.approx(best, abs=1e-12)
            if count == 1:
                np.testing.assert_array_equal(o["L"], arg)
            np.testing.assert_array_equal(o["pos_off"], np.concatenate([[0], np.cumsum(o["L"])]))
            np.testing.assert_array_equal(o["tgt_off"], np.concatenate([[0], np.cumsum(o["L"] + 1)]))


def _brute_dvl_ragged(s, bl, B):
    R, b = s.shape
    pref = np.concatenate([np.zeros((R, 1)), np.cumsum(s.astype(np.float64), axis=1)], axis=1)
    best, arg, count = -1.0, None, 0
    for L in itertools.product(*[range(int(x) + 1) for x in bl]):
        if sum(L) > B:
            continue
        obj = sum(pref[r, L[r]] for r in range(R))
        if obj > best + 1e-15:
            best, arg, count = obj, L, 1
        elif abs(obj - best) <= 1e-15:
            count += 1
    return best, np.array(arg), count


def test_dvl_ragged_block_lengths_brute_force():
    """Per-request block length (wispaper Q&A on block-diffusion decode
    failures, section "Why is a fixed block size a failure mode in production?":
    BlockPilot's block size varies per request): request r drafted b_r
    positions; the allocation over its prefixes of length <= b_r is checked
    against exhaustive search."""
    rng = np.random.default_rng(43)
    for trial in range(150):
        R, b = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        bl = rng.integers(0, b + 1, size=R).astype(np.int32)
        if trial % 3 == 0:
            a = rng.choice([0.0, 0.25, 0.5, 1.0], size=(R, b)).astype(np.float32)
        else:
            a = rng.beta(8, 2, size=(R, b)).astype(np.float32)
        n = int(bl.sum())
        for B in range(0, n + 2):
            o = oracle.dvl(a, B, block_len=bl)
            assert o["bad"] == 0
            for r in range(R):
                np.testing.assert_array_equal(o["s"][r, :bl[r]], np.cumprod(a[r, :bl[r]], dtype=np.float32))
                assert (o["s"][r, bl[r]:] == 0).all()
            assert (o["L"] <= bl).all() and o["L"].sum() == min(B, n)
            best, arg, count = _brute_dvl_ragged(o["s"], bl, B)
            assert oracle.dvl_objective(o["s"], o["L"]) == pytest.approx(best, abs=1e-12)
            if count == 1:
                np.testing.assert_array_equal(o["L"], arg)
            np.testing.assert_array_equal(o["pos_off"], np.concatenate([[0], np.cumsum(o["L"])]))
            np.testing.assert_array_equal(o["tgt_off"], np.concatenate([[0], np.cumsum(o["L"] + 1)]))


def test_dvl_ragged_special_cases():
    a = np.full((4, 16), 0.9, np.float32)
    full = np.full(4, 16, np.int32)
    for B in (0, 7, 33, 64):
        u, g = oracle.dvl(a, B), oracle.dvl(a, B, block_len=full)
        for k in ("s", "L", "pos_off", "tgt_off"):
            np.testing.assert_array_equal(u[k], g[k])
    bl = np.array([16, 0, 5, 9], np.int32)
    assert list(oracle.dvl(a, 1000, block_len=bl)["L"]) == [16, 0, 5, 9]   # budget above sum b_r
    assert list(oracle.dvl(a, 12, block_len=bl)["L"]) == [4, 0, 4, 4]     # equal scores: even split
    assert list(oracle.dvl(a, 19, block_len=bl)["L"]) == [7, 0, 5, 7]     # request 2 is exhausted
    with pytest.raises(ValueError):
        oracle.dvl(a, 10, block_len=np.array([17, 0, 0, 0], np.int32))


def test_dvl_special_cases():
    a = np.full((4, 16), 0.9, np.float32)
    assert list(oracle.dvl(a, 64)["L"]) == [16] * 4          # full capacity
    assert list(oracle.dvl(a, 1000)["L"]) == [16] * 4
    assert list(oracle.dvl(a, 0)["L"]) == [0] * 4
    assert list(oracle.dvl(a, 32)["L"]) == [8] * 4           # equal scores: even split
    assert list(oracle.dvl(a, 34)["L"]) == [9, 9, 8, 8]      # remaining ties by request order
    bad = a.copy()
    bad[1, 3] = 1.5
    assert oracle.dvl(bad, 10)["bad"] == 1


# ---------------------------------------------------------------- decision margins
# The margins decide which GPU/oracle disagreements may be excused, so each is
# pinned on inputs whose probabilities are known in closed form.  Rows are
# built from logits 0 and ln k, so that softmax gives simple fractions; fp32
# rounding of ln k moves them by ~1e-8, far inside the 1e-9 + 1e-6 tolerances
# below and far below the O(0.1) change any plausible mistake makes.
#   accept: |u - min(1, p/q)|                    (q = 0: as if p/q were +inf, or 0 when p = 0 too)
#   draw:   distance of u*W to the ends of the chosen token's CDF interval, / W
#   top-p:  min(|C_{>cut} - top_p|, |C_{>=cut} - top_p|)
# (DBLast review, "Assumptions & free parameters": rejection correction keeps
# the target distribution, so a decision that sits within a tiny margin of its
# threshold is the only place two exact implementations may part.)
MTOL = 1e-6


def _ln(k):
    return np.float32(np.log(k))


def _margin_workload(R=256):
    """b = 1, V = 4: target row 1 uniform (p = 1/4 each), bonus row with
    logits (0, 0, ln 2, 0) (p = 1/5, 1/5, 2/5, 1/5); the draft row (0, 0, 0,
    ln 3) gives q = 1/6, 1/6, 1/6, 1/2.  Even requests draft token 3 (rho =
    1/2), odd ones token 0 (rho = 3/2)."""
    tgt = np.array([[0, 0, 0, 0], [0, 0, _ln(2), 0]], np.float32)
    draft = np.array([[0, 0, 0, _ln(3)]], np.float32)
    x = np.where(np.arange(R) % 2 == 0, 3, 0).astype(np.int32)[:, None]
    return tgt, draft, x


def test_accept_margin_closed_form():
    R = 256
    tgt, draft, x = _margin_workload(R)
    out = oracle.step(tgt=tgt, tgt_row0=np.zeros(R, np.int64), L=np.ones(R, np.int32), T=np.ones(R, np.float32),
                      x=x, seed=20240611, draft=draft, draft_row0=np.zeros(R, np.int64))
    u = out["u_acc"][:, 0]
    even = np.arange(R) % 2 == 0
    np.testing.assert_allclose(out["p_x"][:, 0], 0.25, atol=1e-9)
    np.testing.assert_allclose(out["q_x"][:, 0], np.where(even, 0.5, 1 / 6), atol=1e-8)
    # rho = 1/2 (token 3) and rho = 3/2 (token 0, capped at 1 by min(1, .))
    want = np.where(even, np.abs(u - 0.5), 1.0 - u)
    np.testing.assert_allclose(out["acc_margin"][:, 0], want, atol=MTOL)
    # the decision sits on the side of the threshold the margin measures from
    assert np.array_equal(out["n_acc"] == 1, np.where(even, u < 0.5, True))
    assert (out["acc_margin"][:, 0] > 0).all()


def test_accept_margin_zero_q_and_point_masses():
    """T = 0: p and q are one-hot at the target and draft argmax, so the
    ratio is 1 (both hit), +inf (q = 0 < p), 0 (p = 0 < q) or undefined (both
    0, rejected): margins 1 - u, 1 - u, u, u."""
    R = 64
    tgt = np.array([[0, 5, 0, 0], [1, 0, 0, 0]], np.float32)   # target argmax 1
    draft = np.array([[0, 5, 0, 0], [0, 0, 5, 0]], np.float32)  # draft argmax 1 in row 0, 2 in row 1
    kind = np.arange(R) % 4
    # kind 0: x = 1 from row 0 (p = q = 1); 1: x = 1 from row 1 (p = 1, q = 0);
    #      2: x = 2 from row 1 (p = 0, q = 1); 3: x = 3 from row 0 (p = q = 0)
    x = np.array([1, 1, 2, 3], np.int32)[kind][:, None]
    drow = np.array([0, 1, 1, 0])[kind]
    out = oracle.step(tgt=tgt, tgt_row0=np.zeros(R, np.int64), L=np.ones(R, np.int32), T=np.zeros(R, np.float32),
                      x=x, seed=77, draft=draft, draft_row0=drow.astype(np.int64))
    u = out["u_acc"][:, 0]
    want = np.where(kind <= 1, 1.0 - u, u)
    np.testing.assert_allclose(out["acc_margin"][:, 0], want, atol=1e-15)
    assert np.array_equal(out["n_acc"], (kind <= 1).astype(np.int32))


def test_draw_margin_closed_form():
    """Residual at position 1 (rejected token 3): weights max(0, p - q) =
    (1/12, 1/12, 1/12, 0), W = 1/4, so with t = 3u the token is floor(t) and
    the margin min(frac(t), 1 - frac(t)) / 3.  Bonus from (1/5, 1/5, 2/5, 1/5)
    (W = 1): cumulative (1/5, 2/5, 4/5, 1)."""
    R = 512
    tgt, draft, x = _margin_workload(R)
    x[:] = 3
    out = oracle.step(tgt=tgt, tgt_row0=np.zeros(R, np.int64), L=np.ones(R, np.int32), T=np.ones(R, np.float32),
                      x=x, seed=4242, draft=draft, draft_row0=np.zeros(R, np.int64))
    u = out["u_res"]
    rej = out["n_acc"] == 0
    assert 100 < rej.sum() < R - 100
    t = 3.0 * u[rej]
    np.testing.assert_array_equal(out["token"][rej], np.floor(t).astype(np.int32))
    fr = t - np.floor(t)
    np.testing.assert_allclose(out["sample_margin"][rej], np.minimum(fr, 1.0 - fr) / 3.0, atol=MTOL)
    cum = np.array([0.0, 0.2, 0.4, 0.8, 1.0])
    ub = u[~rej]
    tok = np.searchsorted(cum, ub, side="right") - 1
    np.testing.assert_array_equal(out["token"][~rej], tok)
    np.testing.assert_allclose(out["sample_margin"][~rej], np.minimum(ub - cum[tok], cum[tok + 1] - ub), atol=MTOL)


def test_topp_margin_two_level_closed_form():
    """n1 tokens at a above n2 at c: the top level holds mass M1.  A top_p
    below M1 cuts at a (C_> = 0, C_>= = M1); above it, at c (C_> = M1,
    C_>= = 1)."""
    n1, n2, a, c, T = 3, 997, 2.0, -1.0, 1.0
    row = np.full(n1 + n2, c, np.float32)
    row[[5, 400, 999]] = a
    M1 = n1 * np.exp(a / T) / (n1 * np.exp(a / T) + n2 * np.exp(c / T))
    tp = 0.8 * M1                         # nearer to M1 than to 0
    st = oracle.row_stats(row, T, tp)
    assert st["cut"] == a
    assert st["margin"] == pytest.approx(0.2 * M1, abs=1e-12)
    tp = M1 + 0.3 * (1 - M1)              # nearer to M1 than to 1
    st = oracle.row_stats(row, T, tp)
    assert st["cut"] == c
    assert st["margin"] == pytest.approx(0.3 * (1 - M1), abs=1e-12)
    tp = M1 + 0.9 * (1 - M1)              # nearer to 1
    st = oracle.row_stats(row, T, tp)
    assert st["margin"] == pytest.approx(0.1 * (1 - M1), abs=1e-12)
    assert oracle.row_stats(row, T, 1.0)["margin"] == np.inf
    assert oracle.row_stats(row, 0.0, 0.5)["margin"] == np.inf
