"""Pins for the oracle's greedy tree acceptance, plus the decision-margin
report of the tree build on every seeded workload.

Acceptance is checked against an enumeration of every root-to-node path with
Python's own max (an argmax that knows nothing of numpy), planted paths whose
accepted length is known by construction, and the no-match special case.
"""
import numpy as np
import pytest
import torch

from oracle import tree_oracle as O
from tree_causal_attention_amd import workloads as WL


def _py_argmax(row):
    return max(range(len(row)), key=lambda v: (float(row[v]), -v))


def _brute_accept(X, par, tok, n):
    a = [_py_argmax(X[r]) for r in range(n)]
    best, best_depth = 0, 0
    for v in range(n):
        path, u = [], v
        while u > 0:
            path.append(u)
            u = par[u]
        if all(tok[u] == a[par[u]] for u in path) and len(path) > best_depth:
            best, best_depth = v, len(path)
    path, u = [], best
    while u > 0:
        path.append(u)
        u = par[u]
    return best_depth, path[::-1], a[best]


@pytest.mark.parametrize("seed", range(40))
def test_accept_matches_path_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 30))
    V = int(rng.integers(2, 4))            # tiny vocab: matches are common
    par = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
    depth = [0] * n
    for j in range(1, n):
        depth[j] = depth[par[j]] + 1
    tok = [int(rng.integers(0, V)) for _ in range(n)]
    X = rng.integers(0, 3, (n, V)).astype(np.float32)    # many argmax ties
    N = max(depth) + 2
    L, nodes, bonus = O.accept(X, par, tok, depth, n, N)
    bd, bpath, bb = _brute_accept(X, par, tok, n)
    assert (L, bonus) == (bd, bb)
    assert list(nodes[:L]) == bpath and all(nodes[L:] == -1)


def test_argmax_ties_go_to_lowest_id():
    X = np.array([[1.0, 3.0, 3.0, 0.0]], dtype=np.float32)
    assert O.accept(X, [-1], [0], [0], 1, 2)[2] == 1


def test_no_depth_one_match():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 20)).astype(np.float32)
    a0 = int(np.argmax(X[0]))
    tok = [0] + [(a0 + 1 + j) % 20 for j in range(4)]
    L, nodes, bonus = O.accept(X, [-1, 0, 0, 1, 2], tok, [0, 1, 1, 2, 2], 5, 3)
    assert L == 0 and all(nodes == -1) and bonus == a0


def test_planted_paths_on_tiny_workload():
    w = WL.WORKLOADS["tiny_f32"]
    x = WL.make_inputs(w)
    t = O.build_tree(x.draft[0].numpy(), w.width_w, w.budget_b, int(x.root_token[0]))
    n = t["n_nodes"]
    gen = torch.Generator().manual_seed(5)
    for _ in range(5):
        node = int(torch.randint(1, n, (1,), generator=gen))
        tgt = x.target[0].clone()
        WL.plant_path(tgt, t["parent"], t["token"], node)
        L, nodes, bonus = O.accept(tgt.numpy(), t["parent"], t["token"], t["depth"], n, w.depth_n)
        path = O.ancestors(t["parent"], node)[1:]
        assert L >= len(path) and list(nodes[:len(path)]) == path


def test_oracle_rejects_nan_target():
    with pytest.raises(O.OracleInputError):
        O.accept(np.array([[np.nan, 1.0]]), [-1], [0], [0], 1, 1)


# ------------------------------------------- decision margins of the workloads

def _margins(name, instance, seqs):
    w = WL.WORKLOADS[name]
    x = WL.make_inputs(w, instance, with_target=False, batch=seqs)
    out = []
    for s in range(seqs):
        t = O.build_tree(x.draft[s].numpy(), w.width_w, w.budget_b, int(x.root_token[s]))
        out.append(t)
    return w, out


@pytest.mark.parametrize("name,instance,seqs", [("tiny_f32", 0, 1), ("qwen3_8b_b16", 0, 1),
                                                ("qwen3_8b_b256", 0, 1)])
def test_seeded_builds_are_far_from_ties(name, instance, seqs):
    """The GPU and the oracle compute the per-depth log-sum-exp with different
    summation orders (last-bit differences), so their trees can only differ
    where two candidates of different depths are within ~1e-13 of each other.
    The seeded workloads keep every decision well away from that."""
    w, trees = _margins(name, instance, seqs)
    for t in trees:
        assert t["n_nodes"] == w.budget_b + 1
        assert t["raw_exact"]
        assert t["cross_depth_ties"] == 0
        assert t["margin"] > 1e-9


@pytest.mark.slow
@pytest.mark.parametrize("name,instance,seqs", [("qwen3_8b_b256", i, 1) for i in range(1, 8)]
                         + [("serving_b32", 0, 32), ("qwen3_30b_a3b_b8", 0, 8)])
def test_seeded_builds_are_far_from_ties_all(name, instance, seqs):
    w, trees = _margins(name, instance, seqs)
    for t in trees:
        assert t["n_nodes"] == w.budget_b + 1
        assert t["raw_exact"] and t["cross_depth_ties"] == 0 and t["margin"] > 1e-9
