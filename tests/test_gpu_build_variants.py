"""GPU parity of the build-mode variants (jt_build_tree_variant) against the
CPU oracle: node-block expansion and entropy / mixed priorities.  Integer
outputs are bit-exact wherever the oracle's search is not within rounding of a
different decision (the per-depth lse and entropy are reductions in another
order); the weight-0 candidate search must equal jt_build_tree bit for bit."""
import json
import os
import zlib

import numpy as np
import pytest
import torch

from oracle import tree_oracle as O
from tree_causal_attention_amd import binding as B
from tree_causal_attention_amd import workloads as WL

from gpu_util import dev, to_np

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_GAP = 1e-10  # decisions closer than this may differ by the reductions' order


def _say(msg):
    print(msg, flush=True)


def _gpu_variant(L, W, Bn, roots, expand, a):
    d = dev()
    err = torch.zeros(1, dtype=torch.int32, device=d)
    r = torch.as_tensor(np.asarray(roots), dtype=torch.int32).to(d)
    out = B.jt_build_tree_variant(L.to(d).contiguous(), W, Bn, r, expand, a, err=err)
    torch.cuda.synchronize()
    return {k: (to_np(v) if v is not None else None) for k, v in out.items()}, int(err.item())


def _check_seq(g, s, t):
    n = t["n_nodes"]
    assert int(g["n_nodes"][s]) == n, f"seq {s}"
    for k in ("parent", "token", "depth"):
        assert np.array_equal(g[k][s], t[k]), (s, k)
    np.testing.assert_allclose(g["score"][s][:n], t["score"][:n], rtol=0, atol=1e-9)


def test_variant_hand_examples_on_gpu():
    gd = json.load(open(os.path.join(GOLDEN, "build_variant_example.json")))
    for c in gd["cases"]:
        L = torch.from_numpy(np.log(np.array(c["rows"])).astype(np.float32))[None]
        g, err = _gpu_variant(L, 2, c["budget"], [9], c["expand"], c["weight"])
        assert err == 0
        n = int(g["n_nodes"][0])
        tree = [[int(g["parent"][0][v]), int(g["token"][0][v]), int(g["depth"][0][v])]
                for v in range(1, n)]
        assert tree == c["tree"], c


@pytest.mark.parametrize("expand,a", [("candidate", 0.0), ("candidate", 0.3), ("candidate", 1.0),
                                      ("node_block", 0.0), ("node_block", 0.6),
                                      ("node_block", 1.0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_variant_small_random(expand, a, dtype):
    rng = np.random.default_rng(zlib.crc32(f"{expand}/{a}/{dtype}".encode()))
    compared = 0
    for case in range(6):
        N, W = int(rng.integers(1, 7)), int(rng.integers(1, 5))
        V = int(rng.integers(max(W, 2), 41))
        Bn = int(rng.integers(0, 80))
        b = 4
        coarse = case % 2 == 0  # rounded logits: many exact ties
        X = rng.standard_normal((b, N, V)) * 2
        if coarse:
            X = np.round(X, 1)
        L = torch.from_numpy(X.astype(np.float32))
        if dtype == "bf16":
            L = L.to(torch.bfloat16)
        roots = rng.integers(0, V, b)
        g, err = _gpu_variant(L, W, Bn, roots, expand, a)
        assert err == 0
        Lf = L.float().numpy()
        for s in range(b):
            t = O.build_tree_variant(Lf[s], W, Bn, int(roots[s]), expand, a)
            if t["margin"] < _GAP or t["cross_ties"]:
                continue
            compared += 1
            _check_seq(g, s, t)
    assert compared >= 18


def test_variant_weight0_candidate_equals_default_build():
    """The sequential search at weight 0 reproduces the parallel default build
    bit for bit (scores included) on the B=256 workload and on small cases."""
    for name in ("qwen3_8b_b256", "qwen3_8b_b16", "tiny_f32"):
        w = WL.WORKLOADS[name]
        x = WL.make_inputs(w, 0, with_target=False)
        d = dev()
        L = x.draft.to(d)
        r = x.root_token.to(d)
        ref = B.jt_build_tree(L, w.width_w, w.budget_b, r)
        g, err = _gpu_variant(x.draft, w.width_w, w.budget_b, x.root_token, "candidate", 0.0)
        assert err == 0
        for k in ("parent", "token", "depth", "n_nodes", "score"):
            assert np.array_equal(to_np(ref[k]), g[k]), (name, k)


@pytest.mark.parametrize("expand,a", [("candidate", 0.5), ("candidate", 1.0),
                                      ("node_block", 0.0), ("node_block", 0.5)])
def test_variant_workload_b256(expand, a):
    """B = 256, W = 8, N = 16 over the 151936-token vocabulary."""
    name = "qwen3_8b_b256"
    w = WL.WORKLOADS[name]
    xs = [WL.make_inputs(w, inst, with_target=False) for inst in (0, 1)]
    L = torch.cat([x.draft for x in xs])
    roots = torch.cat([x.root_token for x in xs])
    _say(f"variant {name} {expand} {a}")
    g, err = _gpu_variant(L, w.width_w, w.budget_b, roots, expand, a)
    assert err == 0
    for s in range(2):
        t = O.build_tree_variant(L[s].numpy(), w.width_w, w.budget_b, int(roots[s]), expand, a)
        assert t["margin"] >= _GAP and not t["cross_ties"]
        _check_seq(g, s, t)


def test_variant_reports_nan():
    L = torch.zeros((1, 2, 16))
    L[0, 1, 3] = float("nan")
    g, err = _gpu_variant(L, 2, 4, [0], "node_block", 0.5)
    assert err & B.DERR_BAD_LOGIT


@pytest.mark.parametrize("expand", ["candidate", "node_block"])
def test_variant_max_budget(expand):
    """B = 1023 (1024 nodes: every register slot of the search is used)."""
    rng = np.random.default_rng(1023 if expand == "candidate" else 1024)
    N, W, V, Bn = 12, 2, 64, 1023
    L = torch.from_numpy((rng.standard_normal((2, N, V)) * 2).astype(np.float32))
    roots = [5, 9]
    for a in (0.0, 0.5):
        g, err = _gpu_variant(L, W, Bn, roots, expand, a)
        assert err == 0
        for s in range(2):
            t = O.build_tree_variant(L[s].numpy(), W, Bn, roots[s], expand, a)
            assert t["n_nodes"] == 1024
            if t["margin"] < _GAP or t["cross_ties"]:
                continue
            _check_seq(g, s, t)


@pytest.mark.parametrize("expand", ["candidate", "node_block"])
def test_variant_cross_depth_entropy_ties(expand):
    """Pure entropy priority (a = 1) with draft rows repeated at several
    depths: a repeated row has the same entropy at every depth it sits at, on
    both sides (same data, same arithmetic), so entries of different depths
    tie exactly and the tie rule alone decides.  The trees must agree bit for
    bit, and the oracle must report such ties (the case is exercised)."""
    rng = np.random.default_rng(77 if expand == "candidate" else 78)
    N, W, V, Bn = 6, 3, 40, 60
    base = rng.standard_normal((3, V)) * 2
    rows = base[[0, 0, 1, 1, 2, 0]]  # depths 1, 2 and 6 share a row; 3 and 4 too
    L = torch.from_numpy(np.stack([rows, rows[::-1].copy()]).astype(np.float32))
    roots = [3, 7]
    g, err = _gpu_variant(L, W, Bn, roots, expand, 1.0)
    assert err == 0
    ties = 0
    for s in range(2):
        t = O.build_tree_variant(L[s].numpy(), W, Bn, roots[s], expand, 1.0)
        ties += t["cross_ties"]
        _check_seq(g, s, t)
    assert ties > 0
