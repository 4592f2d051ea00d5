"""Pins of the oracle's tree verification (CPU only).

The rule is multi-round speculative sampling over the candidates of a node
(Miao et al., SpecInfer): each child is tested against the current target,
and every rejection replaces that target by norm(max(0, target - q)).  Pinned
by: the chain it reduces to (orc_step, pinned separately), closed-form
residuals on rows whose probabilities are simple fractions, greedy trees, and
the distribution of the emitted tokens (DBLast review, "Assumptions & free
parameters": rejection correction keeps the target distribution).
"""
import numpy as np
import pytest
from scipy import special

import oracle
from test_oracle_pins import bincount, chi2_check, np_target, sample_idx


def _chain_trees(x, L):
    """Request r's chain: node j >= 1 holds x[r, j - 1], parent j - 1."""
    R = len(L)
    node_off = np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)
    parent = np.concatenate([np.arange(-1, L[r]) for r in range(R)]).astype(np.int32)
    token = np.concatenate([np.concatenate([[0], x[r, :L[r]]]) for r in range(R)]).astype(np.int32)
    return node_off, parent, token


@pytest.mark.parametrize("T,top_p", [(1.0, None), (0.7, 0.8), (0.0, None), (1.5, 0.95)])
def test_chain_tree_equals_the_block_step(T, top_p):
    """A chain (node j's parent j - 1) is the block verification of orc_step,
    with the same uniforms: equal decisions, tokens, probabilities and
    margins."""
    rng = np.random.default_rng(int(T * 10) + (0 if top_p is None else 1))
    R, b, V = 64, 6, 37
    tl = (2.0 * rng.standard_normal((R, b + 1, V))).astype(np.float32)
    dl = (tl[:, :b] + rng.standard_normal((R, b, V))).astype(np.float32)
    x = np.empty((R, b), np.int32)
    for r in range(R):
        for i in range(b):
            x[r, i] = np.argmax(dl[r, i]) if T == 0 else sample_idx(rng, special.softmax(dl[r, i] / T), 1)[0]
        if r % 5 == 0:  # some drafts equal the target argmax, so that long prefixes get accepted
            x[r] = np.argmax(tl[r, :b], axis=-1)
    L = rng.integers(0, b + 1, size=R).astype(np.int32)
    tp = None if top_p is None else np.full(R, top_p, np.float32)
    Tr = np.full(R, T, np.float32)
    st = oracle.step(tgt=tl.reshape(-1, V), tgt_row0=np.arange(R) * (b + 1), L=L, T=Tr, x=x, seed=31,
                     top_p=tp, draft=dl.reshape(-1, V), draft_row0=np.arange(R) * b)
    node_off, parent, token = _chain_trees(x, L)
    tgt_row = np.concatenate([r * (b + 1) + np.arange(L[r] + 1) for r in range(R)])
    tr = oracle.tree_step(tgt=tl.reshape(-1, V), tgt_row=tgt_row, node_off=node_off, parent=parent, token=token,
                          T=Tr, b=b, seed=31, draft=dl.reshape(-1, V), draft_row0=np.arange(R) * b, top_p=tp)
    for k in ("n_acc", "token", "is_bonus", "sample_margin", "u_res"):
        np.testing.assert_array_equal(tr[k], st[k], err_msg=k)
    for r in range(R):
        n = int(st["n_acc"][r])
        assert list(tr["path"][r, :n]) == list(range(1, n + 1))
        tested = min(n + 1, int(L[r]))  # positions 1..n accepted, n + 1 rejected (if it exists)
        sl = slice(node_off[r] + 1, node_off[r] + 1 + tested)
        for k in ("u_acc", "p_x", "q_x", "acc_margin"):
            np.testing.assert_array_equal(tr[k][sl], st[k][r, :tested], err_msg=k)


def _uniform_node_rows():
    """Target rows: node 0 uniform over V = 4 (p = 1/4 each); every other
    node (0, 0, ln 2, 0) -> (1/5, 1/5, 2/5, 1/5).  Draft row (0, 0, 0, ln 3)
    -> q = (1/6, 1/6, 1/6, 1/2)."""
    tgt = np.array([[0, 0, 0, 0], [0, 0, np.log(2), 0]], np.float32)
    draft = np.array([[0, 0, 0, np.log(3)], [0, 0, 0, 0]], np.float32)
    return tgt, draft


def test_second_candidate_against_the_residual_closed_form():
    """Root with children (3, 0): child 1 has rho = (1/4) / (1/2) = 1/2; after
    its rejection the target is norm(max(0, p - q)) = (1/3, 1/3, 1/3, 0), so
    child 2 (token 0) has p = 1/3 against q = 1/6 and is always accepted.
    With children (3, 3) the second test has p = 0 and fails, and the token is
    drawn from norm(max(0, (1/3, 1/3, 1/3, 0) - q)) = (1/3, 1/3, 1/3, 0):
    floor(3 u)."""
    tgt, draft = _uniform_node_rows()
    R = 400
    for second in (0, 3):
        node_off = np.arange(R + 1, dtype=np.int32) * 3
        parent = np.tile(np.array([-1, 0, 0], np.int32), R)
        token = np.tile(np.array([0, 3, second], np.int32), R)
        tgt_row = np.tile(np.array([0, 1, 1]), R)
        o = oracle.tree_step(tgt=tgt, tgt_row=tgt_row, node_off=node_off, parent=parent, token=token,
                             T=np.ones(R), b=2, seed=9 + second, draft=draft, draft_row0=np.zeros(R, np.int64))
        u1 = o["u_acc"][1::3]
        first = u1 < 0.5
        assert 100 < first.sum() < R - 100
        np.testing.assert_allclose(o["p_x"][1::3], 0.25, atol=1e-9)
        np.testing.assert_allclose(o["q_x"][1::3], 0.5, atol=1e-8)
        np.testing.assert_allclose(o["acc_margin"][1::3], np.abs(u1 - 0.5), atol=1e-6)
        assert np.isnan(o["u_acc"][2::3][first]).all()          # child 2 is never tested after child 1's acceptance
        p2 = o["p_x"][2::3][~first]
        np.testing.assert_allclose(p2, 1 / 3 if second == 0 else 0.0, atol=1e-9)
        if second == 0:
            assert (o["n_acc"] == 1).all()
            assert np.array_equal(o["path"][:, 0], np.where(first, 1, 2))
            assert o["is_bonus"].all()                            # a leaf: bonus from (1/5, 1/5, 2/5, 1/5)
            cum = np.array([0.0, 0.2, 0.4, 0.8, 1.0])
            tok = np.searchsorted(cum, o["u_res"], side="right") - 1
            assert np.array_equal(o["token"], tok)
        else:
            rej = ~first
            assert (o["n_acc"][rej] == 0).all() and not o["is_bonus"][rej].any()
            t = 3.0 * o["u_res"][rej]
            assert np.array_equal(o["token"][rej], np.floor(t).astype(np.int32))
            fr = t - np.floor(t)
            np.testing.assert_allclose(o["sample_margin"][rej], np.minimum(fr, 1 - fr) / 3, atol=1e-6)


def test_greedy_tree_follows_the_target_argmax():
    """T = 0: the first child (in index order) whose token is the target's
    argmax is accepted; with none, the extra token is that argmax -- at every
    node of the path."""
    rng = np.random.default_rng(4)
    V, b = 6, 4
    trees, rows = [], []
    for r in range(60):
        N = int(rng.integers(1, 12))
        par = [-1] + [int(rng.integers(0, j)) for j in range(1, N)]
        depth = [0]
        for j in range(1, N):
            depth.append(depth[par[j]] + 1)
        keep = [j for j in range(N) if depth[j] <= b]
        remap = {j: k for k, j in enumerate(keep)}  # a depth cap keeps a prefix-closed subtree
        par = [-1] + [remap[par[j]] for j in keep[1:]]
        N = len(keep)
        tok = [0] + [int(rng.integers(0, V)) for _ in range(1, N)]
        trees.append((par, tok))
        rows.append(rng.integers(-2, 3, size=(N, V)).astype(np.float32))  # ties: the lowest index is the argmax
    node_off = np.concatenate([[0], np.cumsum([len(t[0]) for t in trees])]).astype(np.int32)
    parent = np.concatenate([t[0] for t in trees]).astype(np.int32)
    token = np.concatenate([t[1] for t in trees]).astype(np.int32)
    tgt = np.concatenate(rows)
    draft = rng.standard_normal((b, V)).astype(np.float32)
    R = len(trees)
    o = oracle.tree_step(tgt=tgt, tgt_row=np.arange(len(tgt)), node_off=node_off, parent=parent, token=token,
                         T=np.zeros(R), b=b, seed=3, draft=draft, draft_row0=np.zeros(R, np.int64))
    for r, (par, tok) in enumerate(trees):
        am = np.argmax(rows[r], axis=-1)
        u, path = 0, []
        while True:
            kids = [j for j in range(len(par)) if par[j] == u]
            hit = [j for j in kids if tok[j] == am[u]]
            if not hit:
                break
            u = hit[0]
            path.append(u)
        assert o["n_acc"][r] == len(path) and list(o["path"][r, :len(path)]) == path
        assert o["token"][r] == am[u] and o["stop_node"][r] == u
        assert o["is_bonus"][r] == (len([j for j in range(len(par)) if par[j] == u]) == 0)


N_TRIALS = 1_000_000


def test_chi2_tree_tokens_follow_the_target():
    """V = 8; the root has three candidates drawn independently from q_1, each
    with two candidates drawn from q_2.  A node's target row depends on its
    path's tokens (the root: P0; a depth-1 node with token t: P1[t]; a depth-2
    node: P2[t1, t2]), as a target model's would.  The first emitted token
    follows P0; given a first accepted token t, the second follows P1[t]."""
    rng = np.random.default_rng(77)
    V, b, T, n = 8, 2, 1.0, N_TRIALS
    P0 = (1.5 * rng.standard_normal(V)).astype(np.float32)
    P1 = (1.5 * rng.standard_normal((V, V))).astype(np.float32)
    P2 = (1.5 * rng.standard_normal((V * V, V))).astype(np.float32)
    tgt = np.concatenate([P0[None], P1, P2])  # row 0; 1 + t; 1 + V + 8 t1 + t2
    draft = np.stack([P0 + 1.2 * rng.standard_normal(V), P1.mean(0) + rng.standard_normal(V)]).astype(np.float32)
    q1, q2 = special.softmax(draft[0] / T), special.softmax(draft[1] / T)
    c1 = np.stack([sample_idx(rng, q1, n) for _ in range(3)], axis=1)          # [n, 3]
    c2 = np.stack([sample_idx(rng, q2, n) for _ in range(6)], axis=1)          # [n, 6]: two per depth-1 node
    # nodes: 0 root; 1..3 depth 1; 4..9 depth 2 (children of 1, 1, 2, 2, 3, 3)
    par1 = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3], np.int32)
    token = np.zeros((n, 10), np.int32)
    token[:, 1:4] = c1
    token[:, 4:10] = c2
    trow = np.zeros((n, 10), np.int64)
    trow[:, 1:4] = 1 + c1
    d1 = c1[:, [0, 0, 1, 1, 2, 2]]
    trow[:, 4:10] = 1 + V + V * d1 + c2
    o = oracle.tree_step(tgt=tgt, tgt_row=trow.reshape(-1), node_off=np.arange(n + 1, dtype=np.int32) * 10,
                         parent=np.tile(par1, n), token=token.reshape(-1), T=np.full(n, T), b=b, seed=88,
                         draft=draft, draft_row0=np.zeros(n, np.int64))
    n_acc, tok = o["n_acc"], o["token"]
    first = np.where(n_acc >= 1, token[np.arange(n), o["path"][:, 0].clip(0)], tok)
    chi2_check(bincount(first, V), np_target(P0, T)[0])
    sel = n_acc >= 1
    p1 = o["path"][sel, 0]
    t1 = token[np.nonzero(sel)[0], p1]
    second = np.where(n_acc[sel] >= 2, token[np.nonzero(sel)[0], o["path"][sel, 1].clip(0)], tok[sel])
    for t in np.argsort(-np.bincount(t1, minlength=V))[:3]:  # the three most frequent first tokens
        m = t1 == t
        assert m.sum() > 20000
        chi2_check(bincount(second[m], V), np_target(P1[t], T)[0])


def test_tree_rejects_malformed_input():
    tgt, draft = _uniform_node_rows()
    common = dict(tgt=tgt, tgt_row=[0, 1, 1], T=[1.0], b=2, seed=1, draft=draft, draft_row0=[0])
    with pytest.raises(ValueError):  # a parent that does not precede its child
        oracle.tree_step(node_off=[0, 3], parent=[-1, 2, 0], token=[0, 1, 1], **common)
    with pytest.raises(ValueError):  # a token outside [0, V)
        oracle.tree_step(node_off=[0, 3], parent=[-1, 0, 0], token=[0, 1, 9], **common)
    with pytest.raises(ValueError):  # deeper than the block
        oracle.tree_step(node_off=[0, 3], parent=[-1, 0, 1], token=[0, 1, 1], **{**common, "b": 1})


def _exact_outcomes(par, tok, P, Q):
    """Brute force: the probability of every (accepted path, token) outcome of
    one tree with fixed tokens, by following each branch of the rule with its
    exact probability (P[j]: target distribution at node j; Q[d]: drafter's
    distribution at depth d)."""
    kids = [[] for _ in par]
    depth = [0] * len(par)
    for j in range(1, len(par)):
        kids[par[j]].append(j)
        depth[j] = depth[par[j]] + 1
    out = {}

    def visit(u, path, w):
        if not kids[u]:
            for v in range(len(P[u])):
                out[(path, v)] = out.get((path, v), 0.0) + w * P[u][v]
            return
        t = np.array(P[u], np.float64)
        q = np.array(Q[depth[u]], np.float64)
        for j in kids[u]:
            x = tok[j]
            a = min(1.0, t[x] / q[x]) if q[x] > 0 else float(t[x] > 0)
            if a > 0:
                visit(j, path + (j,), w * a)
            w *= 1.0 - a
            res = np.maximum(t - q, 0.0)
            t = res / res.sum() if res.sum() > 0 else np.array(P[u], np.float64)
        for v in range(len(t)):
            out[(path, v)] = out.get((path, v), 0.0) + w * t[v]

    visit(0, (), 1.0)
    return out


def test_brute_force_outcomes_of_a_fixed_tree():
    """V = 3, fixed tokens: a root with three candidates (two alike), one of
    which has two candidates of its own.  The frequencies of (path, token) over
    400,000 requests (independent uniforms) match the exact outcome
    probabilities by chi-square."""
    rng = np.random.default_rng(21)
    V, b, n = 3, 2, 400_000
    par = [-1, 0, 0, 0, 2, 2]
    tok = [0, 1, 1, 2, 0, 2]
    tl = (1.2 * rng.standard_normal((len(par), V))).astype(np.float32)
    dl = (1.2 * rng.standard_normal((b, V))).astype(np.float32)
    P = [special.softmax(tl[j].astype(np.float64)) for j in range(len(par))]
    Q = [special.softmax(dl[d].astype(np.float64)) for d in range(b)]
    exact = _exact_outcomes(par, tok, P, Q)
    assert abs(sum(exact.values()) - 1.0) < 1e-12
    N = len(par)
    o = oracle.tree_step(tgt=tl, tgt_row=np.tile(np.arange(N), n), node_off=np.arange(n + 1, dtype=np.int32) * N,
                         parent=np.tile(par, n), token=np.tile(tok, n), T=np.ones(n), b=b, seed=5, draft=dl,
                         draft_row0=np.zeros(n, np.int64))
    keys = sorted(exact)
    index = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for r in range(n):
        path = tuple(int(v) for v in o["path"][r, :o["n_acc"][r]])
        counts[index[(path, int(o["token"][r]))]] += 1  # an outcome of zero probability raises KeyError
    chi2_check(counts, np.array([exact[k] for k in keys]))
