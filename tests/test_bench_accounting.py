"""The benchmark's algorithmic work (the roofline's numerator) against brute force.

``bench.algorithmic_work`` counts each node's visible keys as its prefix plus
depth + 1 tree nodes.  Here the visible keys are counted by walking every
node's ancestor chain, on random trees and on the oracle's trees of the seeded
Qwen3-8B workloads, and the K/V and Q/O bytes are summed directly.
"""
import random
from types import SimpleNamespace

import numpy as np
import pytest

import bench
from oracle import tree_oracle as O
from tree_causal_attention_amd import workloads as WL


def _brute(w, prefixes, parents, ns):
    e = 2 if w.dtype == "bf16" else 4
    kv = qo = pairs = 0
    for P, par, n in zip(prefixes, parents, ns):
        kv += (P + n) * w.hkv * w.head_dim * 2 * e
        qo += n * w.hq * w.head_dim * 2 * e
        for i in range(n):
            u, chain = i, 0
            while u >= 0:  # i and each of its ancestors is one visible tail key
                chain += 1
                u = par[u]
            pairs += P + chain
    return kv, qo, 4 * w.head_dim * w.hq * pairs


def _depths(par, n):
    d = [0] * n
    for i in range(1, n):
        d[i] = d[par[i]] + 1
    return d


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_algorithmic_work_random_trees(seed):
    rng = random.Random(seed)
    w = SimpleNamespace(dtype=rng.choice(["bf16", "f32"]), hq=rng.choice([4, 8, 32]),
                        hkv=rng.choice([1, 2, 4]), head_dim=rng.choice([64, 128]))
    b = rng.randint(1, 5)
    prefixes = [rng.randint(0, 5000) for _ in range(b)]
    ns = [rng.randint(1, 300) for _ in range(b)]
    parents = [[-1] + [rng.randrange(j) for j in range(1, n)] for n in ns]
    depth = [_depths(p, n) for p, n in zip(parents, ns)]
    got = bench.algorithmic_work(w, np.array(prefixes), np.array(ns), depth)
    assert got == _brute(w, prefixes, parents, ns)


@pytest.mark.parametrize("name", ["qwen3_8b_b16", "qwen3_8b_b256"])
def test_algorithmic_work_workload_trees(name):
    w = WL.WORKLOADS[name]
    x = WL.make_inputs(w, with_target=False)
    trees = [O.build_tree(x.draft[s].numpy(), w.width_w, w.budget_b, int(x.root_token[s]),
                          check_exact=False) for s in range(w.batch)]
    prefixes = x.prefix_len.tolist()
    ns = [t["n_nodes"] for t in trees]
    parents = [[int(v) for v in t["parent"][:n]] for t, n in zip(trees, ns)]
    depth = [t["depth"] for t in trees]
    got = bench.algorithmic_work(w, np.array(prefixes), np.array(ns), depth)
    assert got == _brute(w, prefixes, parents, ns)
