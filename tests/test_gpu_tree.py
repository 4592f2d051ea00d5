"""Tree verification on the GPU (sv_tree_verify, through the C ABI) against the
oracle's orc_tree_step on the same seeded trees and rows.

Comparison, per request, along the oracle's order of tests (from the root,
each visited node's children in index order up to the accepted one): the
Philox uniform of every tested node exactly, p and q of its token within
1e-5 relative (1e-9 absolute for residual probabilities that cancel to ~0);
the decisions, accepted path, stopping node, bonus flag and token exactly,
except where the first disagreeing decision (or the draw) has an oracle margin
below 1e-6 -- after such a disagreement the request's later tests are not
compared.  Needs an MI355X; run with ``-m gpu``.
"""
import numpy as np
import pytest

import oracle
import synth
from harness import MARGIN, REL, assert_rate, log_parity

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


def gpu_tree(w: synth.TreeWorkload, *, node_off=None, parent=None, token=None, max_kids=None, max_nodes=None,
             tree_ws_fill=0, calls=1):
    """Row statistics (sv_topp_threshold over the node rows, sv_softmax_stats
    over the drafter's rows) and sv_tree_verify, all on the GPU."""
    import torch

    sv = _sv()
    from draft_verification_sv_amd.step import row_pitch, to_device_rows

    node_off = w.node_off if node_off is None else np.asarray(node_off, np.int32)
    parent = w.parent if parent is None else np.asarray(parent, np.int32)
    token = w.token if token is None else np.asarray(token, np.int32)
    R, b, V = w.R, w.b, w.V
    n = int(node_off[-1])
    max_nodes = max(n, R) if max_nodes is None else max_nodes
    max_kids = w.max_kids if max_kids is None else max_kids
    d = dict(device="cuda")
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    ld = row_pitch(V, w.dtype)
    tg = to_device_rows(w.tgt[:n], ld)
    dr = to_device_rows(w.draft.reshape(R * b, V), ld)
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    T = torch.from_numpy(w.T).to(**d)
    tp = None if w.top_p is None else torch.from_numpy(w.top_p).to(**d)
    no = torch.from_numpy(node_off).to(**d)
    po = torch.arange(R + 1, dtype=i32, **d) * b
    ws, nb = sv.make_workspace(R, b, 0, V)
    st = [torch.zeros(max_nodes, dtype=t, **d) for t in (f32, i32, f64, f32, f64)]
    ds = [torch.zeros(R * b, dtype=t, **d) for t in (f32, i32, f64)]
    tb = sv.sv_tree_workspace_bytes(max_nodes, max_kids, V)
    tws = torch.full((tb,), tree_ws_fill, dtype=torch.uint8, **d)
    par = torch.from_numpy(parent).to(**d)
    tok = torch.from_numpy(token).to(**d)
    seed = torch.tensor([np.uint64(w.seed).view(np.int64)], **d)
    out = dict(n_acc=torch.full((R,), -7, dtype=i32, **d), path=torch.full((R * b,), -1, dtype=i32, **d),
               stop_node=torch.full((R,), -7, dtype=i32, **d), token=torch.full((R,), -7, dtype=i32, **d),
               is_bonus=torch.full((R,), -7, dtype=i32, **d), p_x=torch.full((max_nodes,), np.nan, dtype=f64, **d),
               q_x=torch.full((max_nodes,), np.nan, dtype=f64, **d),
               u_acc=torch.full((max_nodes,), np.nan, dtype=f32, **d))
    sv.sv_topp_threshold(tg, dt, ld, V, no, 0, R, max_nodes, T, tp, *st, ws, nb)
    sv.sv_softmax_stats(dr, dt, ld, V, po, b, R, R * b, T, *ds, ws, nb)
    for _ in range(calls):
        sv.sv_tree_verify(tg, dt, ld, V, no, par, tok, R, b, max_nodes, max_kids, T, st[1], st[3], st[4], dr, dt, ld,
                          ds[1], ds[2], seed, out["n_acc"], out["path"], out["stop_node"], out["token"],
                          out["is_bonus"], out["p_x"], out["q_x"], out["u_acc"], ws, nb, tws, tb)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    g["path"] = g["path"].reshape(R, b)
    g["status"] = sv.sv_get_status(ws)
    return g


def oracle_tree(w: synth.TreeWorkload, *, node_off=None, parent=None, token=None):
    node_off = w.node_off if node_off is None else np.asarray(node_off, np.int32)
    parent = w.parent if parent is None else parent
    token = w.token if token is None else token
    n = int(node_off[-1])
    return oracle.tree_step(tgt=w.tgt[:n], tgt_row=np.arange(n), node_off=node_off, parent=parent, token=token,
                            T=w.T, b=w.b, seed=w.seed, draft=w.draft.reshape(w.R * w.b, w.V),
                            draft_row0=np.arange(w.R) * w.b, top_p=w.top_p)


def _test_order(par, path):
    """The oracle's tests of one request: (node, accepted) in order."""
    kids = [[] for _ in par]
    for j in range(1, len(par)):
        kids[par[j]].append(j)
    seq, u = [], 0
    for nxt in list(path) + [None]:
        for c in kids[u]:
            seq.append((c, c == nxt))
            if c == nxt:
                break
        if nxt is None:
            break
        assert nxt in kids[u], "oracle path leaves the tree"
        u = nxt
    return seq


def compare_tree(g, o, node_off, parent, skip=(), report=None):
    rep = report if report is not None else {"positions": 0, "mismatches": 0, "low_margin": [], "cut_diff": 0}
    R = len(node_off) - 1
    for r in range(R):
        if r in skip:
            continue
        n0, n1 = int(node_off[r]), int(node_off[r + 1])
        opath = [int(v) for v in o["path"][r, :o["n_acc"][r]]]
        gpath = [int(v) for v in g["path"][r, :max(0, g["n_acc"][r])]]
        seq = _test_order(parent[n0:n1], opath)
        rep["positions"] += len(seq)
        diverged = False
        for c, acc in seq:
            k = n0 + c
            assert np.float64(g["u_acc"][k]) == o["u_acc"][k], f"uniform of node {c} differs (r={r})"
            for key in ("p_x", "q_x"):
                a, e = g[key][k], o[key][k]
                assert abs(a - e) <= REL * abs(e) + 1e-9, f"{key} of node {c} differs (r={r}): gpu {a} oracle {e}"
            if (c in gpath) != acc:
                m = o["acc_margin"][k]
                rep["mismatches"] += 1
                rep["low_margin"].append(("accept", r, c, float(m)))
                assert m < MARGIN, f"decision at node {c} differs (r={r}), margin {m}"
                diverged = True
                break
        if diverged:
            continue
        assert gpath == opath, f"path differs (r={r}): gpu {gpath} oracle {opath}"
        assert int(g["stop_node"][r]) == int(o["stop_node"][r]), f"stopping node differs (r={r})"
        assert int(g["is_bonus"][r]) == int(o["is_bonus"][r]), f"bonus flag differs (r={r})"
        tested_g = ~np.isnan(g["u_acc"][n0:n1])
        tested_o = ~np.isnan(o["u_acc"][n0:n1])
        assert np.array_equal(tested_g, tested_o), f"tested nodes differ (r={r})"
        if int(g["token"][r]) != int(o["token"][r]):
            m = o["sample_margin"][r]
            rep["mismatches"] += 1
            rep["low_margin"].append(("sample", r, int(o["token"][r]), float(m)))
            assert m < MARGIN, f"token differs (r={r}): gpu {g['token'][r]} oracle {o['token'][r]}, margin {m}"
    return rep


SMALL = [  # (shape, dtype, V, T, top_p, width, nodes)
    ("random", "bf16", 1031, 1.0, None, 3, 30),
    ("random", "f32", 1031, [1.0, 0.0, 0.6, 1.4] * 6, 0.9, 3, 30),
    ("random", "bf16", 4099, 0.7, 0.95, 4, 60),
    ("wide", "bf16", 257, 1.0, None, 16, 0),
    ("wide", "f32", 9000, 1.0, 0.8, 6, 0),
    ("chain", "bf16", 1031, [1.0, 0.0] * 12, None, 1, 0),
    ("random", "bf16", 1031, 0.0, None, 4, 40),
]


@pytest.mark.parametrize("shape,dtype,V,T,top_p,width,nodes", SMALL,
                         ids=[f"{s[0]}-{s[1]}-V{s[2]}-{i}" for i, s in enumerate(SMALL)])
def test_tree_matches_oracle(shape, dtype, V, T, top_p, width, nodes):
    w = synth.tree(f"tree-{shape}", R=24, b=5, V=V, width=width, nodes=max(nodes, 1), dtype=dtype, T=T, top_p=top_p,
                   shape=shape, seed=3100 + V + width)
    banner(f"sv_tree_verify {shape} {dtype} V={V} nodes={int(w.node_off[-1])} max_kids={w.max_kids}")
    g = gpu_tree(w)
    assert g["status"] == 0, _sv().STATUS_BITS
    o = oracle_tree(w)
    rep = compare_tree(g, o, w.node_off, w.parent)
    assert rep["positions"] > 0
    assert_rate(rep)


def test_tree_full_size_matches_oracle():
    """Qwen3 vocabulary, 32 requests, depth 16, up to 64 nodes per request,
    T = 1 and top-p 0.95 (the target side of the mixture workloads)."""
    w = synth.tree("tree-conc32-w4-n64", R=32, b=16, V=synth.QWEN3_VOCAB, width=4, nodes=64, T=1.0, top_p=0.95,
                   seed=3200)
    banner(f"sv_tree_verify full size nodes={int(w.node_off[-1])}")
    g = gpu_tree(w)
    assert g["status"] == 0
    o = oracle_tree(w)
    rep = compare_tree(g, o, w.node_off, w.parent)
    log_parity(w.name, rep)
    assert_rate(rep)


def test_tree_bench_workload_over_steps():
    """The tree benchmark's own workload (bench.py --tree: its shape and data
    seed) verified with five successive seeds, every step against the
    oracle."""
    import bench

    sh = bench.TREE_SHAPE
    w = synth.tree("tree-bench", R=sh["R"], b=sh["b"], V=synth.QWEN3_VOCAB, width=sh["width"], nodes=sh["nodes"],
                   T=sh["T"], top_p=sh["top_p"], seed=bench.TREE_DATA_SEED)
    rep = None
    for k in range(5):
        w.seed = bench.TREE_DATA_SEED_VERIFY + k
        banner(f"sv_tree_verify bench workload nodes={int(w.node_off[-1])} seed={w.seed}")
        g = gpu_tree(w)
        assert g["status"] == 0
        rep = compare_tree(g, oracle_tree(w), w.node_off, w.parent, report=rep)
    log_parity(f"{w.name} (the benchmark's trees), 5 seeds", rep)
    assert_rate(rep)


def test_tree_greedy_full_size_matches_oracle():
    w = synth.tree("tree-conc32-greedy", R=32, b=16, V=synth.QWEN3_VOCAB, width=3, nodes=48, T=0.0, seed=3300)
    banner(f"sv_tree_verify greedy full size nodes={int(w.node_off[-1])}")
    g = gpu_tree(w)
    assert g["status"] == 0
    o = oracle_tree(w)
    rep = compare_tree(g, o, w.node_off, w.parent)
    assert rep["mismatches"] == 0


def test_tree_maximum_sizes_match_oracle():
    """Requests at the node cap (1024 nodes each), up to 16 children per node,
    bf16 and top-p: the walk's and the checks' LDS arrays filled to their
    ends."""
    w = synth.tree("tree-max", R=2, b=32, V=1031, width=16, nodes=1024, T=1.0, top_p=0.9, seed=3600, fill=True)
    assert list(np.diff(w.node_off)) == [1024, 1024] and w.max_kids <= 16
    banner(f"sv_tree_verify maximum sizes nodes per request {list(np.diff(w.node_off))} max_kids={w.max_kids}")
    g = gpu_tree(w)
    assert g["status"] == 0
    o = oracle_tree(w)
    assert_rate(compare_tree(g, o, w.node_off, w.parent))


def test_tree_deepest_accepted_paths():
    """Chains as deep as the block allows (b = 64) whose every token is its
    parent's target argmax, at T = 0: every test accepts, so the walk runs the
    whole chain, fills the path array to its end and draws the bonus token at
    depth 64 (the chains of other lengths stop earlier, at their leaves)."""
    w = synth.tree("tree-deep", R=8, b=64, V=1031, T=0.0, shape="chain", seed=3800)
    vals = synth.values(w.tgt)
    for r in range(w.R):
        n0, n1 = int(w.node_off[r]), int(w.node_off[r + 1])
        for j in range(n0 + 1, n1):
            w.token[j] = int(np.argmax(vals[j - 1]))  # the parent of node j is node j - 1
    lengths = np.diff(w.node_off) - 1
    banner(f"sv_tree_verify deepest accepted paths, chain lengths {list(lengths)}")
    g = gpu_tree(w)
    assert g["status"] == 0
    o = oracle_tree(w)
    assert np.array_equal(o["n_acc"], lengths) and np.array_equal(g["n_acc"], lengths)
    assert_rate(compare_tree(g, o, w.node_off, w.parent))


def test_tree_reused_workspace_and_repeat_calls():
    """Two calls on one tree workspace left over from a different tree (and one
    filled with garbage bytes): results as from a fresh one."""
    w = synth.tree("tree-reuse", R=16, b=6, V=2053, width=4, nodes=40, T=1.0, seed=3400)
    o = oracle_tree(w)
    banner("sv_tree_verify on a garbage-filled tree workspace, two calls")
    g = gpu_tree(w, tree_ws_fill=0xA5, calls=2)
    assert g["status"] == 0
    assert_rate(compare_tree(g, o, w.node_off, w.parent))


def test_tree_malformed_requests_are_flagged():
    """Malformed trees (root parent not -1, a parent after its child, a node
    deeper than b, more children than max_kids, an empty node range) set
    BAD_TREE and get n_acc = 0 and no token; the other requests are verified
    as usual."""
    sv = _sv()
    w = synth.tree("tree-bad", R=8, b=3, V=1031, width=3, nodes=12, T=1.0, seed=3500)
    node_off = w.node_off.copy()
    parent = w.parent.copy()
    n_of = np.diff(node_off)
    big = [r for r in range(w.R) if n_of[r] >= 4]
    assert len(big) >= 3, n_of
    bad = {}
    r = big[0]
    parent[node_off[r]] = 0  # the root's parent is not -1
    bad[r] = "root"
    r = big[1]
    parent[node_off[r] + 2] = 3  # a parent after its child
    bad[r] = "order"
    r = big[2]  # a chain deeper than b = 3: node j's parent j - 1 for every node
    parent[node_off[r]:node_off[r + 1]] = np.arange(-1, n_of[r] - 1)
    if n_of[r] <= 4:
        bad[r] = None  # depth 3 at most: still a valid tree
    else:
        bad[r] = "depth"
    banner(f"sv_tree_verify malformed {bad}")
    g = gpu_tree(w, parent=parent)
    assert g["status"] & 0x400, sv.STATUS_BITS
    flagged = {r for r, k in bad.items() if k is not None}
    for r in flagged:
        assert g["n_acc"][r] == 0
    good_parent = w.parent.copy()
    for r in flagged:
        good_parent[node_off[r]:node_off[r + 1]] = parent[node_off[r]:node_off[r + 1]]
    o_w = synth.tree("tree-bad", R=8, b=3, V=1031, width=3, nodes=12, T=1.0, seed=3500)
    o = oracle_tree(o_w)  # the unmodified trees; only the requests left as they were are compared
    assert_rate(compare_tree(g, o, node_off, w.parent, skip=flagged | {r for r, k in bad.items() if k is None}))
    # more children than max_kids
    banner("sv_tree_verify with max_kids below the widest node")
    g = gpu_tree(w, max_kids=max(1, w.max_kids - 1))
    assert g["status"] & 0x400
    # an empty node range for request 1 (its nodes go to request 0's range end)
    no2 = node_off.copy()
    no2[1] = no2[2]
    banner("sv_tree_verify with an empty node range")
    g = gpu_tree(w, node_off=no2)
    assert g["status"] & 0x400
    assert g["n_acc"][1] == 0


def test_tree_host_argument_errors():
    import torch

    sv = _sv()
    with pytest.raises(sv.SvError):
        sv.sv_tree_workspace_bytes(10, 17, 100)
    with pytest.raises(sv.SvError):
        sv.sv_tree_workspace_bytes(0, 4, 100)
    z = torch.zeros(64, dtype=torch.int32, device="cuda")
    ws, nb = sv.make_workspace(2, 4, 0, 60)
    with pytest.raises(sv.SvError):  # tree workspace too small
        sv.sv_tree_verify(z, sv.SV_F32, 64, 60, z, z, z, 2, 4, 8, 2, z, z, z, z, z, sv.SV_F32, 64, z, z, z, z, z,
                          z, z, z, None, None, None, ws, nb, z, 4)
    with pytest.raises(sv.SvError):  # max_nodes below R
        sv.sv_tree_verify(z, sv.SV_F32, 64, 60, z, z, z, 2, 4, 1, 2, z, z, z, z, z, sv.SV_F32, 64, z, z, z, z, z,
                          z, z, z, None, None, None, ws, nb, z, 1 << 20)
    with pytest.raises(sv.SvError):  # more than 1024 requests
        sv.sv_tree_verify(z, sv.SV_F32, 64, 60, z, z, z, 1025, 4, 2000, 2, z, z, z, z, z, sv.SV_F32, 64, z, z, z, z,
                          z, z, z, z, None, None, None, ws, nb, z, 1 << 20)
