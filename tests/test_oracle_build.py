"""Pins for the oracle's tree construction (per-depth top-W + best-first).

Every check here compares the oracle with something other than itself: a
library routine (scipy's logsumexp), an independent enumeration (sorting the
whole complete tree), closed-form special cases (W = 1 chain, budget covering
the complete tree), hand-derived fixtures, and structural invariants.
"""
import functools
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import tree_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------- row stats

@pytest.mark.parametrize("seed", range(6))
def test_row_stats_against_library_and_sorted(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(5, 60))
    x = (rng.standard_normal(V) * 3).astype(np.float32)
    if seed % 2:  # plant duplicated values so the id tie-break matters
        x[rng.integers(0, V, 4)] = x[0]
    W = int(rng.integers(1, V + 1))
    lse, tok, val = O.draft_row_stats(x, W)
    assert abs(lse - logsumexp(x.astype(np.float64))) <= 1e-12 * max(1.0, abs(lse))
    ref = sorted(range(V), key=lambda v: (-float(x[v]), v))[:W]
    assert list(tok) == ref
    assert list(val) == [float(x[v]) for v in ref]


def test_row_stats_neg_inf_and_rejections():
    x = np.array([1.0, -np.inf, 0.5, -np.inf], dtype=np.float32)
    lse, tok, val = O.draft_row_stats(x, 4)
    assert list(tok) == [0, 2, 1, 3]
    assert abs(lse - math.log(math.exp(1.0) + math.exp(0.5))) < 1e-15
    for bad in ([np.nan, 1.0], [np.inf, 1.0], [-np.inf, -np.inf]):
        with pytest.raises(O.OracleInputError):
            O.draft_row_stats(np.array(bad), 1)
    with pytest.raises(O.OracleInputError):
        O.draft_row_stats(np.zeros(3), 4)


# --------------------------------------------------------------- brute force

def _brute_tree(L, W, B):
    """All nodes of the complete W-ary depth-N tree, globally sorted.

    Independent of the oracle's queue: log-probs come from scipy's
    logsumexp, the candidates from Python's sort, and the node order from one
    global sort with a comparator that orders by score, then (recursively) by
    the parents' order, then by rank.  Since a child never outranks its
    parent, the first B of this order are the best-first pops.
    """
    N, V = L.shape
    cands, lps = [], []
    for d in range(N):
        row = L[d].astype(np.float64)
        c = sorted(range(V), key=lambda v: (-row[v], v))[:W]
        cands.append(c)
        lps.append([row[v] - logsumexp(row) for v in c])
    paths = [()]
    for d in range(1, N + 1):
        paths += [p for p in itertools.product(range(W), repeat=d)]

    def score(p):
        return sum(lps[i][k] for i, k in enumerate(p))

    sc = {p: score(p) for p in paths}

    def cmp(a, b):
        if a == b:
            return 0
        if a == ():
            return -1
        if b == ():
            return 1
        if sc[a] != sc[b]:
            return -1 if sc[a] > sc[b] else 1
        c = cmp(a[:-1], b[:-1])
        if c:
            return c
        return -1 if a[-1] < b[-1] else 1

    order = sorted(paths, key=functools.cmp_to_key(cmp))[:B + 1]
    pos = {p: i for i, p in enumerate(order)}
    parent = [-1] + [pos[p[:-1]] for p in order[1:]]
    token = [None] + [cands[len(p) - 1][p[-1]] for p in order[1:]]
    depth = [len(p) for p in order]
    return parent, token, depth


@pytest.mark.parametrize("N,W,V", [(1, 1, 3), (1, 3, 5), (2, 2, 4), (2, 3, 7), (3, 2, 6),
                                   (3, 3, 12), (2, 1, 5), (3, 3, 3)])
def test_build_matches_global_sort_for_every_budget(N, W, V):
    rng = np.random.default_rng(100 * N + 10 * W + V)
    for trial in range(3):
        L = (rng.standard_normal((N, V)) * 3).astype(np.float32)
        total = sum(W ** d for d in range(1, N + 1))
        for B in range(0, total + 2):
            t = O.build_tree(L, W, B, root_token=5)
            parent, token, depth = _brute_tree(L, W, min(B, total))
            n = t["n_nodes"]
            assert n == len(parent) == min(B, total) + 1
            assert list(t["parent"][:n]) == parent
            assert list(t["token"][1:n]) == token[1:]
            assert list(t["depth"][:n]) == depth
            assert t["raw_exact"]


def test_width_one_gives_argmax_chain():
    rng = np.random.default_rng(7)
    L = (rng.standard_normal((6, 40)) * 3).astype(np.float32)
    t = O.build_tree(L, 1, 10, root_token=0)
    n = t["n_nodes"]
    assert n == 7  # a chain stops at depth N = 6
    assert list(t["parent"][:n]) == [-1, 0, 1, 2, 3, 4, 5]
    assert list(t["token"][1:n]) == [int(np.argmax(L[d])) for d in range(6)]
    assert list(t["depth"][:n]) == list(range(7))


def test_budget_covering_complete_tree():
    rng = np.random.default_rng(8)
    N, W = 3, 3
    L = (rng.standard_normal((N, 20)) * 3).astype(np.float32)
    t = O.build_tree(L, W, 1000, root_token=0)
    n = t["n_nodes"]
    assert n == 1 + 3 + 9 + 27
    par, dep, tok = t["parent"][:n], t["depth"][:n], t["token"][:n]
    for v in range(n):
        kids = [c for c in range(n) if par[c] == v]
        assert len(kids) == (W if dep[v] < N else 0)
        top = sorted(range(20), key=lambda x: (-float(L[dep[v]][x]), x))[:W] if dep[v] < N else []
        assert sorted(tok[c] for c in kids) == sorted(top)


def _invariants(t, N):
    n = t["n_nodes"]
    par, dep, tok, sc = t["parent"], t["depth"], t["token"], t["score"]
    assert par[0] == -1 and dep[0] == 0
    for j in range(1, n):
        assert 0 <= par[j] < j
        assert dep[j] == dep[par[j]] + 1 <= N
        assert sc[j] <= sc[par[j]]
    assert all(sc[j] >= sc[j + 1] for j in range(1, n - 1))  # pop order
    for v in range(n):
        kids = [tok[c] for c in range(1, n) if par[c] == v]
        assert len(kids) == len(set(kids))
    assert np.all(par[n:] == -1) and np.all(tok[n:] == -1)


@pytest.mark.parametrize("seed", range(5))
def test_random_invariants(seed):
    rng = np.random.default_rng(seed)
    N, W, V, B = 5, 4, 50, 40
    L = (rng.standard_normal((N, V)) * float(rng.uniform(0.5, 6))).astype(np.float32)
    t = O.build_tree(L, W, B, root_token=1)
    assert t["n_nodes"] == B + 1
    _invariants(t, N)


def test_hand_derived_tie_fixtures():
    data = json.load(open(os.path.join(GOLDEN, "build_ties.json")))
    for case in data["cases"]:
        L = np.array([[float(v) for v in row] for row in case["logits"]], dtype=np.float32)
        for B, exp in case["expect"].items():
            t = O.build_tree(L, case["width_w"], int(B), case["root_token"])
            n = t["n_nodes"]
            assert list(t["parent"][:n]) == exp["parent"], case["name"]
            assert list(t["token"][:n]) == exp["token"], case["name"]
            assert list(t["depth"][:n]) == exp["depth"], case["name"]


def test_dropped_term_would_be_caught():
    """A planted mistake (lse of depth 2 dropped from the score) changes the
    tree on an input where cross-depth comparisons matter, so the global-sort
    pin above is sensitive to it."""
    rng = np.random.default_rng(3)
    L = (rng.standard_normal((3, 9)) * 3).astype(np.float32)
    good = O.build_tree(L, 3, 12, 0)
    orig = O.draft_row_stats

    calls = []

    def broken(row, width):
        lse, tok, val = orig(row, width)
        calls.append(1)
        return (0.0 if len(calls) == 2 else lse), tok, val
    O.draft_row_stats = broken
    try:
        bad = O.build_tree(L, 3, 12, 0)
    finally:
        O.draft_row_stats = orig
    parent, token, depth = _brute_tree(L, 3, 12)
    assert list(good["parent"][:13]) == parent
    assert list(bad["parent"][:13]) != parent


def test_oracle_rejects_bad_budget():
    with pytest.raises(O.OracleInputError):
        O.build_tree(np.zeros((2, 4), np.float32), 2, -1, 0)
