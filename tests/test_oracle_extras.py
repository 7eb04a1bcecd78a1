"""Pins for the oracle's margin acceptance, KV commit and stochastic verification.

Margin acceptance: the page's worked example (tests/golden), reduction to
greedy acceptance at a zero margin when rows have no ties, path enumeration
with Python's own arithmetic, and monotonicity in the threshold.

KV commit: element-by-element positions against the definition, a path whose
sources overlap later destinations, and the invariance that makes the commit
correct: after it, plain decode attention of the last accepted node over the
new prefix equals that node's tree attention before it.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import tree_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------- margin rule

def test_margin_page_example():
    g = json.load(open(os.path.join(GOLDEN, "margin_example.json")))
    X = np.log(np.array(g["target_probs"], dtype=np.float64))
    for c in g["cases"]:
        L, nodes, bonus = O.accept_margin(X, g["parent"], g["token"], g["depth"], 2, 1,
                                          O.margin_from_ratio(c["theta"]))
        assert L == c["accept_len"], c
        assert nodes.tolist() == c["accept_nodes"], c
        assert bonus == c["bonus"], c


def _tree(rng, n):
    par = [-1] + [int(rng.integers(0, v)) for v in range(1, n)]
    dep = [0] * n
    for v in range(1, n):
        dep[v] = dep[par[v]] + 1
    return par, dep


@pytest.mark.parametrize("seed", range(20))
def test_margin_zero_is_greedy_without_ties(seed):
    rng = np.random.default_rng(seed)
    n, V = int(rng.integers(1, 40)), 50
    par, dep = _tree(rng, n)
    X = rng.standard_normal((n, V)).astype(np.float32)  # continuous: no ties
    a = X.argmax(axis=1)
    tok = [0] + [int(a[par[v]]) if rng.random() < 0.6 else int(rng.integers(0, V))
                 for v in range(1, n)]
    got = O.accept_margin(X, par, tok, dep, n, max(dep) + 1, 0.0)
    ref = O.accept(X, par, tok, dep, n, max(dep) + 1)
    assert got[0] == ref[0] and got[2] == ref[2]
    assert np.array_equal(got[1], ref[1])


def _brute_margin(X, par, tok, dep, n, margin):
    rows = [[float(x) for x in X[r]] for r in range(n)]
    top = [max(r) for r in rows]
    best, best_d = 0, 0
    for v in range(n):
        path, u = [], v
        while u > 0:
            path.append(u)
            u = par[u]
        if all(rows[par[u]][tok[u]] - top[par[u]] >= margin for u in path):
            if len(path) > best_d:
                best, best_d = v, len(path)
    path, u = [], best
    while u > 0:
        path.append(u)
        u = par[u]
    bonus = max(range(len(rows[best])), key=lambda t: (rows[best][t], -t))
    return best_d, path[::-1], bonus


@pytest.mark.parametrize("seed", range(30))
def test_margin_matches_path_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    n, V = int(rng.integers(1, 30)), 12
    par, dep = _tree(rng, n)
    X = np.round(rng.standard_normal((n, V)) * 2, 1).astype(np.float32)  # coarse: ties happen
    tok = [0] + [int(rng.integers(0, V)) for _ in range(1, n)]
    margin = -float(rng.uniform(0.0, 3.0))
    L, nodes, bonus = O.accept_margin(X, par, tok, dep, n, max(dep) + 1, margin)
    bL, bpath, bb = _brute_margin(X, par, tok, dep, n, margin)
    assert L == bL and bonus == bb
    assert nodes[:L].tolist() == bpath and (nodes[L:] == -1).all()


@pytest.mark.parametrize("seed", range(10))
def test_margin_monotone_in_threshold(seed):
    rng = np.random.default_rng(200 + seed)
    n, V = 40, 16
    par, dep = _tree(rng, n)
    X = rng.standard_normal((n, V)).astype(np.float32)
    tok = [0] + [int(rng.integers(0, V)) for _ in range(1, n)]
    lens = [O.accept_margin(X, par, tok, dep, n, max(dep) + 1, O.margin_from_ratio(t))[0]
            for t in (1.0, 0.8, 0.5, 0.2, 0.05)]
    assert lens == sorted(lens)


# ----------------------------------------------------------------- KV commit

def _pool(rng, pages, hkv, d):
    return rng.standard_normal((pages, hkv, 16, d))


@pytest.mark.parametrize("P,nodes", [(5, [1, 2, 3]), (16, [2, 3, 5]), (31, [4]), (0, []),
                                     (20, [1, 5, 6, 9, 12])])
def test_commit_positions(P, nodes):
    rng = np.random.default_rng(P)
    hkv, d, npages = 2, 8, 8
    k, v = _pool(rng, npages, hkv, d), _pool(rng, npages, hkv, d)
    table = rng.permutation(npages)
    L = len(nodes)
    k2, v2, P2 = O.commit_kv(k, v, table, P, L, nodes)
    assert P2 == P + 1 + L

    def row(pool, t):
        return pool[table[t // 16], :, t % 16, :]
    for t in range(npages * 16):
        if P + 1 <= t <= P + L:
            src = P + nodes[t - P - 1]
            assert np.array_equal(row(k2, t), row(k, src)) and np.array_equal(row(v2, t), row(v, src))
        else:
            assert np.array_equal(row(k2, t), row(k, t)) and np.array_equal(row(v2, t), row(v, t))


@pytest.mark.parametrize("seed", range(6))
def test_commit_then_decode_equals_tree_attention(seed):
    rng = np.random.default_rng(300 + seed)
    hq, hkv, d = 4, 2, 16
    n = 12
    par, dep = _tree(rng, n)
    P = int(rng.integers(0, 40))
    npages = (P + n + 15) // 16 + 1
    k, v = _pool(rng, npages, hkv, d), _pool(rng, npages, hkv, d)
    table = rng.permutation(npages)
    q = rng.standard_normal((n, hq, d))
    end = int(rng.integers(1, n))
    path = O.ancestors(par, end)[1:]  # accepted nodes, root excluded
    o_tree, l_tree = O.tree_attention_seq(q, k, v, table, P, par, n, 0.25, nodes=[end])
    k2, v2, P2 = O.commit_kv(k, v, table, P, len(path), path)
    o_dec, l_dec = O.decode_attention(q[end], k2, v2, table, P2, 0.25)
    assert np.abs(o_dec - o_tree[end]).max() <= 1e-12
    assert np.abs(l_dec - l_tree[end]).max() <= 1e-12


# ------------------------------------------------------- stochastic verify

def test_stochastic_hand_example():
    """The i.i.d. proposal mode on one drafted token (q given explicitly)."""
    g = json.load(open(os.path.join(GOLDEN, "stochastic_example.json")))
    X = np.log(np.array(g["target_probs"]))
    Dl = np.log(np.array(g["draft_probs"]))
    for c in g["cases"]:
        ua = np.array([0.0, c["u_accept"]])
        L, nodes, bonus = O.accept_stochastic(X, Dl, g["parent"], g["token"], g["depth"], 2, 1,
                                              1.0, ua, c["u_sample"], draft_mode="sampled")
        assert (L, nodes.tolist(), bonus) == (c["accept_len"], c["accept_nodes"], c["bonus"]), c


def test_stochastic_topw_hand_example():
    """Top-W siblings (point-mass proposals): the hand-worked four-node tree."""
    g = json.load(open(os.path.join(GOLDEN, "stochastic_topw_example.json")))
    X = np.log(np.array(g["target_probs"]))
    for c in g["cases"]:
        L, nodes, bonus = O.accept_stochastic(X, None, g["parent"], g["token"], g["depth"], 4,
                                              g["n_depth"], 1.0, np.array(c["u_accept"]),
                                              c["u_sample"])
        assert (L, nodes.tolist(), bonus) == (c["accept_len"], c["accept_nodes"], c["bonus"]), c


def test_sample_index_is_inverse_cdf():
    p = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert [O.sample_index(p, u) for u in (0.0, 0.2, 0.26, 0.74, 0.76, 0.999)] == [1, 1, 3, 3, 4, 4]


@pytest.mark.parametrize("T", [0.25, 0.7, 1.0, 1.75])
def test_softmax_t_against_scipy(T):
    """softmax(x / T) against scipy's own routine, rows with -inf entries too."""
    from scipy.special import softmax
    rng = np.random.default_rng(int(T * 100))
    for _ in range(5):
        x = rng.standard_normal(37) * 4.0
        x[rng.integers(0, 37, 3)] = -np.inf
        got = O.softmax_t(x, T)
        ref = softmax(x / T)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)
        assert abs(got.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("theta,T", [(0.8, 0.5), (0.8, 1.0), (0.3, 1.75), (0.95, 0.25)])
def test_margin_from_ratio_at_temperature(theta, T):
    """A row whose second logit sits exactly at the margin below the first has
    probability ratio theta under softmax(x / T) (scipy), whatever T is."""
    from scipy.special import softmax
    m = O.margin_from_ratio(theta, T)
    p = softmax(np.array([0.0, m, -3.0]) / T)
    assert abs(p[1] / p[0] - theta) < 1e-12
    if (theta, T) == (0.8, 0.5):
        assert abs(m - (-0.11157177565710485)) < 1e-15  # 0.5 * ln 0.8 by hand


def _first_tokens(tgt, par, toks, dep, n, N, T, rng, trials, mode, dft=None):
    """Runs the walk `trials` times; returns (first emitted token, second emitted
    token or -1, node accepted first or 0) per trial."""
    out = np.empty((trials, 3), dtype=np.int64)
    for i in range(trials):
        ua = rng.random(n)
        us = rng.random()
        L, nodes, bonus = O.accept_stochastic(tgt, dft, par, toks, dep, n, N, T, ua, us,
                                              draft_mode=mode)
        emitted = [toks[v] for v in nodes[:L]] + [bonus]
        out[i] = (emitted[0], emitted[1] if len(emitted) > 1 else -1, nodes[0] if L else 0)
    return out


def _chi2(counts, p):
    expected = p * counts.sum()
    keep = expected > 0
    assert counts[~keep].sum() == 0, (counts, p)
    return float(((counts[keep] - expected[keep]) ** 2 / expected[keep]).sum())


def test_stochastic_topw_counterexample_is_lossless():
    """q = [.5, .3, .2], p = [.2, .2, .6], siblings = the top-2 draft tokens
    [0, 1]: the emitted token must follow p (the i.i.d. rule gives [.4, 0, .6])."""
    rng = np.random.default_rng(7)
    tgt = np.log(np.array([[0.2, 0.2, 0.6]] * 3))
    dft = np.log(np.array([[0.5, 0.3, 0.2]]))
    par, toks, dep = [-1, 0, 0], [0, 0, 1], [0, 1, 1]
    got = _first_tokens(tgt, par, toks, dep, 3, 1, 1.0, rng, 20000, "topw")
    counts = np.bincount(got[:, 0], minlength=3)
    assert _chi2(counts, np.array([0.2, 0.2, 0.6])) < 13.8  # 2 dof, P = 0.001
    # the i.i.d. rule on the same deterministic siblings never emits token 1
    got = _first_tokens(tgt, par, toks, dep, 3, 1, 1.0, rng, 4000, "sampled", dft)
    counts = np.bincount(got[:, 0], minlength=3)
    assert counts[1] == 0 and abs(counts[0] / 4000 - 0.4) < 0.04


@pytest.mark.parametrize("W,T", [(2, 1.0), (3, 0.7), (2, 1.75)])
def test_stochastic_topw_tree_is_lossless_chi_square(W, T):
    """A complete depth-2 tree whose siblings are the top-W tokens of each
    depth's draft row (as the build step makes them).  The first emitted token
    must follow softmax(root row / T); given that depth-1 node v was accepted,
    the second emitted token must follow softmax(row v / T)."""
    rng = np.random.default_rng(300 + 10 * W + int(T * 10))
    V, N = 6, 2
    draft = rng.standard_normal((N, V)) * 1.5
    top = [list(np.lexsort((np.arange(V), -draft[d]))[:W]) for d in range(N)]
    par, toks, dep = [-1], [0], [0]
    for k in range(W):
        par.append(0), toks.append(int(top[0][k])), dep.append(1)
    for v in range(1, W + 1):
        for k in range(W):
            par.append(v), toks.append(int(top[1][k])), dep.append(2)
    n = len(par)
    tgt = rng.standard_normal((n, V)) * 1.5
    trials = 30000
    got = _first_tokens(tgt, par, toks, dep, n, N, T, rng, trials, "topw")
    # 5 degrees of freedom: P(chi2 > 25.7) ~ 1e-4
    assert _chi2(np.bincount(got[:, 0], minlength=V), O.softmax_t(tgt[0], T)) < 25.7
    checked = 0
    for v in range(1, W + 1):
        sel = got[:, 2] == v
        if sel.sum() < 1500:
            continue
        checked += 1
        c2 = _chi2(np.bincount(got[sel, 1], minlength=V), O.softmax_t(tgt[v], T))
        assert c2 < 25.7, (v, c2)
    assert checked >= 1


@pytest.mark.parametrize("k,T", [(1, 1.0), (3, 1.0), (4, 0.7)])
def test_stochastic_sampled_is_lossless_chi_square(k, T):
    """The i.i.d. proposal mode: with k candidates drawn i.i.d. from the draft
    distribution q, the first token the step emits (the accepted child's, else
    the bonus) must follow the target distribution p exactly."""
    rng = np.random.default_rng(1000 + 10 * k)
    V = 6
    tgt = rng.standard_normal((k + 1, V)) * 1.5
    dft = rng.standard_normal((1, V)) * 1.5
    p = O.softmax_t(tgt[0], T)
    q = O.softmax_t(dft[0], T)
    trials = 20000
    counts = np.zeros(V)
    par = [-1] + [0] * k
    dep = [0] + [1] * k
    for _ in range(trials):
        toks = [0] + [int(t) for t in rng.choice(V, size=k, p=q)]
        ua = rng.random(k + 1)
        L, nodes, bonus = O.accept_stochastic(tgt, dft, par, toks, dep, k + 1, 1, T, ua,
                                              rng.random(), draft_mode="sampled")
        counts[toks[nodes[0]] if L else bonus] += 1
    expected = p * trials
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    # 5 degrees of freedom: P(chi2 > 22.1) = 0.0005
    assert chi2 < 22.1, (chi2, counts, expected)


def test_stochastic_sampled_draft_equal_to_target_accepts():
    """q == p: every drafted token passes (u * q(x) < p(x) for u < 1)."""
    rng = np.random.default_rng(5)
    V, n = 20, 12
    par, dep = _tree(rng, n)
    X = rng.standard_normal((n, V))
    Dl = np.tile(X[0], (max(dep) + 1, 1))
    # the target row of every node equals the draft row of its children's depth
    X = np.tile(X[0], (n, 1))
    tok = [0] + [int(rng.integers(0, V)) for _ in range(1, n)]
    L, nodes, _ = O.accept_stochastic(X, Dl, par, tok, dep, n, max(dep) + 1, 1.0,
                                      rng.random(n) * 0.999, 0.5, draft_mode="sampled")
    # the first child of every accepted node is accepted: the path follows first children
    u, expect = 0, []
    while True:
        kids = [v for v in range(1, n) if par[v] == u]
        if not kids:
            break
        u = kids[0]
        expect.append(u)
    assert nodes[:L].tolist() == expect


def test_stochastic_topw_certain_token_is_accepted():
    """A target row that puts all its mass on one token: the sibling holding
    it is accepted whatever its uniform (u < 1 = p(x)); earlier siblings with
    zero mass are rejected without changing p."""
    V = 5
    X = np.full((4, V), -np.inf)
    X[:, 3] = 0.0
    par, tok, dep = [-1, 0, 0, 0], [0, 1, 3, 4], [0, 1, 1, 1]
    for u in (0.0, 0.5, 0.999):
        L, nodes, bonus = O.accept_stochastic(X, None, par, tok, dep, 4, 1, 1.0,
                                              np.array([0.0, u, u, u]), 0.5)
        assert (L, nodes.tolist(), bonus) == (1, [2], 3)


def test_stochastic_topw_duplicate_siblings():
    """A caller tree with the same token on two siblings: the second try sees
    p(x) = 0 after the first rejection and is rejected without changing p."""
    X = np.log(np.array([[0.5, 0.3, 0.2]] * 4))
    par, tok, dep = [-1, 0, 0, 0], [0, 1, 1, 0], [0, 1, 1, 1]
    # 1st sibling (token 1) rejected: p = [5/7, 0, 2/7]; 2nd (token 1 again)
    # rejected; 3rd (token 0): accepted iff u < 5/7
    L, nodes, _ = O.accept_stochastic(X, None, par, tok, dep, 4, 1, 1.0,
                                      np.array([0.0, 0.5, 0.0, 0.7]), 0.5)
    assert (L, nodes.tolist()) == (1, [3])
    L, nodes, bonus = O.accept_stochastic(X, None, par, tok, dep, 4, 1, 1.0,
                                          np.array([0.0, 0.5, 0.0, 0.72]), 0.5)
    assert (L, bonus) == (0, 2)  # p = [0, 0, 1]


# ------------------------------------------------------- build-mode variants

def _variant_tree(t):
    n = t["n_nodes"]
    return [[int(t["parent"][v]), int(t["token"][v]), int(t["depth"][v])] for v in range(1, n)]


def test_variant_hand_examples():
    g = json.load(open(os.path.join(GOLDEN, "build_variant_example.json")))
    for c in g["cases"]:
        L = np.log(np.array(c["rows"]))
        t = O.build_tree_variant(L, 2, c["budget"], 9, c["expand"], c["weight"])
        assert _variant_tree(t) == c["tree"], c
    e = g["entropy"]
    for row, h in zip(e["rows"], e["nats"]):
        assert abs(O.draft_row_entropy(np.log(np.array(row))) - h) < 1e-12


def test_entropy_closed_forms_and_library():
    from scipy.stats import entropy as sp_entropy
    rng = np.random.default_rng(3)
    V = 50
    assert abs(O.draft_row_entropy(np.zeros(V)) - np.log(V)) < 1e-12            # uniform
    one = np.full(V, -np.inf)
    one[7] = 2.0
    assert O.draft_row_entropy(one) == 0.0                                         # one finite entry
    k = np.full(V, -np.inf)
    k[[1, 5, 9, 30]] = -3.5
    assert abs(O.draft_row_entropy(k) - np.log(4)) < 1e-12                         # k equal entries
    for _ in range(20):
        x = rng.standard_normal(V) * 3
        p = np.exp(x - x.max())
        assert abs(O.draft_row_entropy(x) - sp_entropy(p / p.sum())) < 1e-12      # library routine
    # shift invariance
    x = rng.standard_normal(V)
    assert abs(O.draft_row_entropy(x + 100.0) - O.draft_row_entropy(x)) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_variant_candidate_weight0_equals_build_tree(seed):
    """The variant at weight 0 in candidate mode is the default build (pinned by
    brute force elsewhere), ties included (coarse logits)."""
    rng = np.random.default_rng(40 + seed)
    for _ in range(30):
        N, W = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        V = int(rng.integers(W, 12))
        B = int(rng.integers(0, 30))
        L = np.round(rng.standard_normal((N, V)) * 2, 1).astype(np.float32)
        a, b = O.build_tree(L, W, B, 7), O.build_tree_variant(L, W, B, 7)
        assert a["n_nodes"] == b["n_nodes"]
        for key in ("parent", "token", "depth", "score"):
            assert np.array_equal(a[key], b[key])


def _complete_tree(L, W):
    """Every rank path of the complete W-ary tree of depth N: list of
    (rank path tuple, score list along the path, depth)."""
    N = L.shape[0]
    stats = [O.draft_row_stats(L[d], W) for d in range(N)]
    out = []

    def rec(path, raw, scores):
        for k in range(W):
            d = len(path) + 1
            r = raw + float(stats[d - 1][2][k])
            s = r - sum(stats[j][0] for j in range(d))
            p2 = path + (k,)
            out.append((p2, scores + [s], d))
            if d < N:
                rec(p2, r, scores + [s])
    rec((), 0.0, [])
    return out


def _rank_paths(t, W, L):
    """Rank path of every placed node (token -> rank in its depth's top-W)."""
    N = L.shape[0]
    cand = [list(O.draft_row_stats(L[d], W)[1]) for d in range(N)]
    paths = {0: ()}
    for v in range(1, t["n_nodes"]):
        d = int(t["depth"][v])
        paths[v] = paths[int(t["parent"][v])] + (cand[d - 1].index(int(t["token"][v])),)
    return paths


@pytest.mark.parametrize("weight", [0.0, 0.3, 0.7, 1.0])
def test_variant_candidate_bottleneck_property(weight):
    """Best-first on a tree with any priority places the nodes whose bottleneck
    (smallest priority on the root-to-node path) is largest: every placed node's
    bottleneck is >= every unplaced node's.  Brute force over the complete tree
    (continuous logits, no ties)."""
    rng = np.random.default_rng(int(weight * 10) + 60)
    for _ in range(25):
        N, W = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        V = int(rng.integers(W + 1, 10))
        L = rng.standard_normal((N, V)) * 2
        ent = [O.draft_row_entropy(L[d]) for d in range(N)]
        allp = _complete_tree(L, W)
        B = int(rng.integers(0, len(allp) + 2))
        t = O.build_tree_variant(L, W, B, 0, "candidate", weight)
        placed = set(_rank_paths(t, W, L).values()) - {()}
        assert len(placed) == min(B, len(allp))
        bott = {p: min(O.variant_key(s, ent[i], weight) for i, s in enumerate(sc))
                for p, sc, d in allp}
        for p in placed:   # prefix-closed
            assert p[:-1] == () or p[:-1] in placed
        if placed and len(placed) < len(allp):
            assert min(bott[p] for p in placed) >= max(bott[p] for p in bott if p not in placed)


@pytest.mark.parametrize("weight", [0.0, 0.5, 1.0])
def test_variant_node_block_structure(weight):
    """Node-block: the children of every expanded node are consecutive node
    indices in rank order; the expanded nodes (those with children) other than
    the root are the best-first choice among expandable nodes (bottleneck
    property over the complete tree's depth < N nodes); B is filled unless the
    complete tree is smaller."""
    rng = np.random.default_rng(int(weight * 10) + 80)
    for _ in range(25):
        N, W = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        V = int(rng.integers(W + 1, 10))
        L = rng.standard_normal((N, V)) * 2
        ent = [O.draft_row_entropy(L[d]) for d in range(N)]
        allp = _complete_tree(L, W)
        B = int(rng.integers(0, len(allp) + 2))
        t = O.build_tree_variant(L, W, B, 0, "node_block", weight)
        n = t["n_nodes"]
        assert n - 1 == min(B, len(allp))
        par = [int(x) for x in t["parent"][:n]]
        paths = _rank_paths(t, W, L)
        kids = {}
        for v in range(1, n):
            kids.setdefault(par[v], []).append(v)
        for u, ks in kids.items():
            assert ks == list(range(ks[0], ks[0] + len(ks)))          # consecutive
            assert [paths[v][-1] for v in ks] == list(range(len(ks)))  # rank order
            if ks[-1] != n - 1:                                       # only the last block is cut
                assert len(ks) == W
        expanded = {paths[u] for u in kids if u != 0}
        bott = {p: min(O.variant_key(s, ent[i], weight) for i, s in enumerate(sc))
                for p, sc, d in allp if d < N}
        if expanded and len(expanded) < len(bott):
            assert min(bott[p] for p in expanded) >= max(bott[p] for p in bott
                                                         if p not in expanded)
