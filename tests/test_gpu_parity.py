"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.  Tree build and acceptance must match bit for bit; attention within
max-abs 1e-5 (fp32) or max-abs 2e-2 and rel-L2 1e-2 (bf16, fp32 accumulate)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import tree_oracle as O
from tree_causal_attention_amd import binding as B
from tree_causal_attention_amd import workloads as WL

from gpu_util import (as_f64, check_attention, check_lse, dev, to_np)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ helpers

def _gpu_build(draft, W, B_, root):
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    t = B.jt_build_tree(draft.to(dev()), W, B_, root.to(dev()), err=err)
    torch.cuda.synchronize()
    out = {k: to_np(v) for k, v in t.items() if v is not None}
    out["err"] = int(err.item())
    return out


def _assert_tree_equal(g, ref, s, what):
    n = ref["n_nodes"]
    assert int(g["n_nodes"][s]) == n, f"{what} seq {s}: n_nodes {g['n_nodes'][s]} != {n}"
    T = ref["parent"].shape[0]
    for k in ("parent", "token", "depth"):
        assert np.array_equal(g[k][s][:T], ref[k][:T]), f"{what} seq {s}: {k} differs"
    gs = g["score"][s][:n]
    assert np.allclose(gs, ref["score"][:n], rtol=0, atol=1e-9), f"{what} seq {s}: score"


# ------------------------------------------------------------------ tree build

BUILD_CASES = ([("tiny_f32", 0), ("qwen3_8b_b16", 0)] + [("qwen3_8b_b256", i) for i in range(8)]
               + [("serving_b16", 0), ("serving_b32", 0), ("qwen3_30b_a3b_b8", 0)])


@pytest.mark.parametrize("name,instance", BUILD_CASES)
def test_build_tree_workloads(name, instance):
    w = WL.WORKLOADS[name]
    _say(f"build {name}#{instance}")
    x = WL.make_inputs(w, instance, with_target=False)
    g = _gpu_build(x.draft, w.width_w, w.budget_b, x.root_token)
    assert g["err"] == 0
    for s in range(x.draft.shape[0]):
        ref = O.build_tree(x.draft[s].numpy(), w.width_w, w.budget_b, int(x.root_token[s]),
                           check_exact=False)
        _assert_tree_equal(g, ref, s, f"{name}#{instance}")


def test_build_tree_golden_ties_and_neg_inf():
    data = json.load(open(os.path.join(GOLDEN, "build_ties.json")))
    for case in data["cases"]:
        L = torch.tensor([[float(v) for v in row] for row in case["logits"]], dtype=torch.float32)
        for Bs, exp in case["expect"].items():
            g = _gpu_build(L[None], case["width_w"], int(Bs),
                           torch.tensor([case["root_token"]], dtype=torch.int32))
            n = len(exp["parent"])
            assert int(g["n_nodes"][0]) == n
            assert list(g["parent"][0][:n]) == exp["parent"], case["name"]
            assert list(g["token"][0][:n]) == exp["token"], case["name"]
            assert list(g["depth"][0][:n]) == exp["depth"], case["name"]


@pytest.mark.parametrize("seed", range(12))
def test_build_tree_random_small(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 7))
    W = int(rng.integers(1, 9))
    V = int(rng.integers(W, 300))
    Bb = int(rng.integers(0, 120))
    b = int(rng.integers(1, 5))
    L = (rng.standard_normal((b, N, V)) * rng.uniform(0.3, 8)).astype(np.float32)
    if seed % 3 == 0:   # exact ties and excluded tokens
        L[:, :, rng.integers(0, V, V // 3)] = -np.inf
        L[:, :, 0] = L[:, :, 1] = np.float32(5.0)
        L[:, 0, :] = np.isfinite(L[:, 0, :]) * 1.0 + np.where(np.isfinite(L[:, 0, :]), 0, -np.inf)
    roots = rng.integers(0, V, b).astype(np.int32)
    g = _gpu_build(torch.from_numpy(L), W, Bb, torch.from_numpy(roots))
    for s in range(b):
        ref = O.build_tree(L[s], W, Bb, int(roots[s]), check_exact=False)
        _assert_tree_equal(g, ref, s, f"seed{seed}")


def test_build_tree_bf16_logits_and_budget_edges():
    rng = np.random.default_rng(5)
    Lb = torch.from_numpy((rng.standard_normal((2, 5, 777)) * 3).astype(np.float32)).to(torch.bfloat16)
    roots = torch.tensor([1, 2], dtype=torch.int32)
    for Bb, W in ((0, 3), (1, 3), (40, 3), (400, 3), (30, 1)):
        g = _gpu_build(Lb, W, Bb, roots)
        for s in range(2):
            ref = O.build_tree(Lb[s].float().numpy(), W, Bb, int(roots[s]), check_exact=False)
            _assert_tree_equal(g, ref, s, f"bf16 B={Bb} W={W}")



# Draft-scan shapes the workloads leave out: rows longer than 2^19 logits
# (128 a thread), and bf16 rows whose length is a multiple of 8 (16-byte
# loads of 8 logits) on a grid of at most 512 workgroups (512 threads of 16)
# and on a larger one (256 threads of 32).
@pytest.mark.parametrize("b,N,V,dtype", [(1, 3, (1 << 19) + 40, "f32"), (1, 2, (1 << 19) + 40, "bf16"),
                                         (1, 4, 151936, "bf16"), (4, 8, 151936, "bf16")])
def test_build_tree_scan_shapes(b, N, V, dtype):
    rng = np.random.default_rng(V + N + b)
    _say(f"build scan shape b={b} N={N} V={V} {dtype}")
    L = torch.from_numpy((rng.standard_normal((b, N, V)) * 2.5).astype(np.float32))
    if dtype == "bf16":
        L = L.to(torch.bfloat16)
    roots = torch.from_numpy(rng.integers(0, V, b).astype(np.int32))
    g = _gpu_build(L, 8, 64, roots)
    assert g["err"] == 0
    for s in range(b):
        ref = O.build_tree(L[s].float().numpy(), 8, 64, int(roots[s]), check_exact=False)
        _assert_tree_equal(g, ref, s, f"scan b={b} N={N} V={V} {dtype}")


# ------------------------------------------------------------------ tree meta

@pytest.mark.parametrize("T,b", [(1, 1), (17, 3), (257, 2), (1024, 1)])
def test_tree_meta_random_trees(T, b):
    gen = torch.Generator().manual_seed(T)
    parents, ns = [], []
    for s in range(b):
        n = int(torch.randint(1, T + 1, (1,), generator=gen)) if s else T
        p = WL.random_recursive_parents(n, gen)
        if s == b - 1 and n > 2:   # a chain tail
            p = [-1] + list(range(n - 1))
        parents.append(p + [-1] * (T - n))
        ns.append(n)
    par = torch.tensor(parents, dtype=torch.int32, device=dev())
    nn = torch.tensor(ns, dtype=torch.int32, device=dev())
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    anc = to_np(B.jt_tree_meta(par, nn, err=err)).view(np.uint32)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for s in range(b):
        ref = O.ancestor_words(parents[s], ns[s], T)
        assert np.array_equal(anc[s], ref), f"T={T} seq {s}"


def test_tree_meta_rejects_bad_parent_and_nnodes():
    T = 40
    p_ok = [-1] + list(range(T - 1))
    p_bad = list(p_ok)
    p_bad[7] = 9          # parent after child
    par = torch.tensor([p_ok, p_bad, p_ok], dtype=torch.int32, device=dev())
    nn = torch.tensor([T, T, 0], dtype=torch.int32, device=dev())
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    anc = to_np(B.jt_tree_meta(par, nn, err=err)).view(np.uint32)
    torch.cuda.synchronize()
    assert int(err.item()) == (B.DERR_BAD_PARENT | B.DERR_BAD_NNODES)
    assert np.array_equal(anc[0], O.ancestor_words(p_ok, T, T))
    assert not anc[1].any() and not anc[2].any()


# ------------------------------------------------------------------ attention

def _attn_case(rng, b, prefixes, ns, T, hq, hkv, D, dtype):
    """Random paged inputs with the generator's layout conventions."""
    pages_per = [(P + T + 15) // 16 for P in prefixes]
    num_pages = sum(pages_per) + 2
    perm = rng.permutation(num_pages)
    table = np.full((b, max(pages_per)), -1, dtype=np.int32)
    o = 0
    for s in range(b):
        table[s, :pages_per[s]] = perm[o:o + pages_per[s]]
        o += pages_per[s]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.from_numpy(rng.standard_normal((num_pages, hkv, 16, D)).astype(np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((num_pages, hkv, 16, D)).astype(np.float32)).to(tdt)
    # poison every slot past P + n and the spare pages
    for s in range(b):
        for t in range(prefixes[s] + ns[s], pages_per[s] * 16):
            k[table[s, t // 16], :, t % 16] = float("nan")
            v[table[s, t // 16], :, t % 16] = float("nan")
    used = set(table[table >= 0].tolist())
    for pg in range(num_pages):
        if pg not in used:
            k[pg] = float("nan")
            v[pg] = float("nan")
    q = torch.from_numpy((rng.standard_normal((b, T, hq, D)) / np.sqrt(D)).astype(np.float32)).to(tdt)
    parents = []
    for s in range(b):
        n = ns[s]
        p = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
        parents.append(p + [-1] * (T - n))
    return q, k, v, table, num_pages, parents


def _run_attention(q, k, v, table, num_pages, prefixes, parents, ns, scale):
    d = dev()
    par = torch.tensor(parents, dtype=torch.int32, device=d)
    nn = torch.tensor(ns, dtype=torch.int32, device=d)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    anc = B.jt_tree_meta(par, nn, err=err)
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device=d)       # sentinel for unwritten rows
    o, lse = B.jt_tree_attention(q.to(d), k.to(d), v.to(d), nn,
                                 torch.tensor(prefixes, dtype=torch.int32, device=d),
                                 torch.from_numpy(table).to(d), num_pages, anc, scale, err=err,
                                 out=out)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return o, lse


SMALL_ATTN = [
    # b, prefixes, ns, T, hq, hkv, D, dtype
    (2, [100, 0], [37, 1], 40, 8, 2, 128, "bf16"),
    (3, [1, 64, 333], [17, 5, 17], 17, 32, 8, 128, "bf16"),
    (2, [17, 250], [70, 64], 70, 4, 4, 64, "bf16"),
    (1, [0], [200], 257, 16, 1, 128, "bf16"),
    (2, [31, 150], [20, 9], 20, 6, 3, 64, "f32"),
    (1, [64], [17], 17, 4, 1, 64, "f32"),
    (1, [513], [129], 129, 8, 8, 128, "f32"),
    # one (sequence, KV head) group with a long prefix: both row tiles are
    # split over more than 64 key ranges, the merge loops over lane chunks
    (1, [20000], [40], 40, 8, 1, 128, "bf16"),
    (1, [20000], [20], 20, 4, 1, 64, "bf16"),
    # the largest trees the call takes (1024 nodes, 32 mask words) with the
    # largest GQA group (16): 64 full row tiles per (sequence, KV head)
    (1, [100], [1024], 1024, 16, 1, 128, "bf16"),
    (2, [0, 37], [1024, 999], 1024, 16, 1, 64, "bf16"),
    (1, [10], [1024], 1024, 16, 1, 64, "f32"),
    # small last row tiles beside full ones: 8 rows (and a sequence without
    # any), D = 64, 16 rows of one node, group 2 with no prefix
    (2, [100, 20], [257, 256], 257, 8, 1, 128, "bf16"),
    (1, [60], [257], 257, 4, 1, 64, "bf16"),
    (1, [30], [257], 257, 16, 1, 128, "bf16"),
    (1, [0], [257], 257, 4, 2, 128, "bf16"),
]


@pytest.mark.parametrize("case", SMALL_ATTN, ids=lambda c: f"{c[7]}-D{c[6]}-g{c[4] // c[5]}")
def test_attention_small_cases(case):
    b, prefixes, ns, T, hq, hkv, D, dtype = case
    rng = np.random.default_rng(sum(prefixes) + T)
    q, k, v, table, num_pages, parents = _attn_case(rng, b, prefixes, ns, T, hq, hkv, D, dtype)
    scale = 1.0 if dtype == "bf16" else 1 / np.sqrt(D)
    o, lse = _run_attention(q, k, v, table, num_pages, prefixes, parents, ns, scale)
    og, lg = as_f64(o), to_np(lse).astype(np.float64)
    kf, vf, qf = k.float().numpy(), v.float().numpy(), q.float().numpy()
    for s in range(b):
        n = ns[s]
        ro, rl = O.tree_attention_seq_fast(qf[s], kf, vf, table[s], prefixes[s], parents[s], n, scale)
        check_attention(og[s, :n], ro, dtype, f"seq {s}")
        check_lse(lg[s, :n], rl, dtype, f"seq {s}")
        assert (og[s, n:] == 7.0).all(), "rows past n_nodes must not be written"


@pytest.fixture(scope="module")
def oracle_trees():
    cache = {}

    def get(name, instance, x, w):
        key = (name, instance)
        if key not in cache:
            cache[key] = [O.build_tree(x.draft[s].numpy(), w.width_w, w.budget_b,
                                       int(x.root_token[s]), check_exact=False)
                          for s in range(x.draft.shape[0])]
        return cache[key]
    return get


def _workload_attention(name, instance, oracle_trees, full_seqs, sample):
    w = WL.WORKLOADS[name]
    _say(f"attention {name}#{instance}")
    x = WL.make_inputs(w, instance, with_target=False)
    trees = oracle_trees(name, instance, x, w)
    parents = [t["parent"].tolist() for t in trees]
    ns = [t["n_nodes"] for t in trees]
    prefixes = x.prefix_len.tolist()
    o, lse = _run_attention(x.q, x.k_pool, x.v_pool, x.page_table.numpy(), x.num_pages, prefixes,
                            parents, ns, w.scale)
    og, lg = as_f64(o), to_np(lse).astype(np.float64)
    kf = x.k_pool.float().numpy()
    vf = x.v_pool.float().numpy()
    qf = x.q.float().numpy()
    for s in full_seqs:
        ro, rl = O.tree_attention_seq_fast(qf[s], kf, vf, x.page_table[s].numpy(), prefixes[s],
                                           trees[s]["parent"], ns[s], w.scale)
        check_attention(og[s, :ns[s]], ro, w.dtype, f"{name} seq {s}")
        check_lse(lg[s, :ns[s]], rl, w.dtype, f"{name} seq {s}")
    for s, nodes, heads in sample:
        nodes = [min(i, ns[s] - 1) for i in nodes]
        ro, rl = O.tree_attention_seq(qf[s], kf, vf, x.page_table[s].numpy(), prefixes[s],
                                      trees[s]["parent"], ns[s], w.scale, nodes=nodes, heads=heads)
        for i in nodes:
            check_attention(og[s, i, heads], ro[i, heads], w.dtype, f"{name} seq {s} node {i}")
            check_lse(lg[s, i, heads], rl[i, heads], w.dtype, f"{name} seq {s} node {i}")


@pytest.mark.parametrize("name,instance,full",
                         [("tiny_f32", 0, [0]), ("qwen3_8b_b16", 0, [0])]
                         + [("qwen3_8b_b256", i, [0]) for i in range(8)])
def test_attention_workloads_full(name, instance, full, oracle_trees):
    _workload_attention(name, instance, oracle_trees, full, [])


@pytest.mark.parametrize("name,seqs", [("serving_b16", range(0, 16)),
                                       ("serving_b32", range(0, 16)),
                                       ("serving_b32", range(16, 32)),
                                       ("qwen3_30b_a3b_b8", range(0, 8))])
def test_attention_batched_workloads_every_row(name, seqs, oracle_trees):
    """Every node and head of every sequence of the batched workloads (the
    launch the benchmark times), against the oracle's dense per-head pass."""
    _workload_attention(name, 0, oracle_trees, list(seqs), [])


def test_attention_long_prefix_sampled_rows_reference_form(oracle_trees):
    """A few rows of the 32K-prefix batch against the oracle's plain
    per-(node, head) form, a second formulation of the same definition."""
    samp = [(s, [0, 3, 128, 255, 256], [0, 9, 31]) for s in (0, 7)]
    _workload_attention("qwen3_30b_a3b_b8", 0, oracle_trees, [], samp)


def test_attention_invariances_bitwise():
    """Masked K/V cannot change a node (bitwise), page order cannot change the
    result (bitwise), and two runs are bitwise identical."""
    rng = np.random.default_rng(77)
    b, prefixes, ns, T, hq, hkv, D = 1, [300], [60], 60, 8, 2, 128
    q, k, v, table, num_pages, parents = _attn_case(rng, b, prefixes, ns, T, hq, hkv, D, "bf16")
    o1, l1 = _run_attention(q, k, v, table, num_pages, prefixes, parents, ns, 1.0)
    o2, l2 = _run_attention(q, k, v, table, num_pages, prefixes, parents, ns, 1.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    node = 45
    anc = set(O.ancestors(parents[0], node))
    k2, v2 = k.clone(), v.clone()
    for j in range(ns[0]):
        if j not in anc:
            t = prefixes[0] + j
            k2[table[0, t // 16], :, t % 16] = 30.0
            v2[table[0, t // 16], :, t % 16] = -30.0
    o3, l3 = _run_attention(q, k2, v2, table, num_pages, prefixes, parents, ns, 1.0)
    assert torch.equal(o3[0, node], o1[0, node]) and torch.equal(l3[0, node], l1[0, node])
    perm = rng.permutation(num_pages)
    kp = torch.empty_like(k)
    vp = torch.empty_like(v)
    kp[torch.from_numpy(perm)] = k
    vp[torch.from_numpy(perm)] = v
    tp = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    o4, l4 = _run_attention(q, kp, vp, tp, num_pages, prefixes, parents, ns, 1.0)
    assert torch.equal(o4[0, :ns[0]], o1[0, :ns[0]]) and torch.equal(l4[0, :ns[0]], l1[0, :ns[0]])


# ------------------------------------------------------------------ acceptance

def _gpu_accept(target, depth_n, parent, token, depth, n_nodes):
    d = dev()
    err = torch.zeros(1, dtype=torch.int32, device=d)
    alen, anodes, bonus = B.jt_accept(
        target.to(d), depth_n, torch.as_tensor(parent, dtype=torch.int32).to(d),
        torch.as_tensor(token, dtype=torch.int32).to(d),
        torch.as_tensor(depth, dtype=torch.int32).to(d),
        torch.as_tensor(n_nodes, dtype=torch.int32).to(d), err=err)
    torch.cuda.synchronize()
    return to_np(alen), to_np(anodes), to_np(bonus), int(err.item())


@pytest.mark.parametrize("seed", range(6))
def test_accept_small_random_trees(seed):
    """Tiny vocabularies make matches common, so long paths and ties occur."""
    rng = np.random.default_rng(seed)
    b, T, V, N = 4, 60, 3, 64
    parents, tokens, depths, ns = [], [], [], []
    for s in range(b):
        n = int(rng.integers(1, T + 1))
        p = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
        dd = [0] * n
        for j in range(1, n):
            dd[j] = dd[p[j]] + 1
        parents.append(p + [-1] * (T - n))
        depths.append(dd + [-1] * (T - n))
        tokens.append([int(x) for x in rng.integers(0, V, T)])
        ns.append(n)
    X = torch.from_numpy(rng.integers(0, 3, (b, T, V)).astype(np.float32))
    alen, anodes, bonus, err = _gpu_accept(X, N, parents, tokens, depths, ns)
    assert err == 0
    for s in range(b):
        L, nodes, bb = O.accept(X[s].numpy(), parents[s], tokens[s], depths[s], ns[s], N)
        assert (alen[s], bonus[s]) == (L, bb)
        assert np.array_equal(anodes[s], nodes)


@pytest.mark.parametrize("name,instance,plant",
                         [("tiny_f32", 0, True), ("qwen3_8b_b16", 0, False),
                          ("qwen3_8b_b16", 0, True)]
                         + [("qwen3_8b_b256", i, True) for i in range(8)]
                         + [("qwen3_8b_b256", 1, False), ("serving_b16", 0, True),
                            ("serving_b32", 0, True), ("qwen3_30b_a3b_b8", 0, True),
                            ("qwen3_30b_a3b_b8", 0, False)])
def test_accept_workloads(name, instance, plant, oracle_trees):
    w = WL.WORKLOADS[name]
    _say(f"accept {name}#{instance}")
    x = WL.make_inputs(w, instance)
    trees = oracle_trees(name, instance, x, w)
    tgt = x.target.clone()
    gen = torch.Generator().manual_seed(instance)
    for s in range(len(trees)):
        if plant:
            t = trees[s]
            deepest = int(np.argmax(t["depth"][:t["n_nodes"]]))
            node = deepest if s % 2 == 0 else int(torch.randint(1, t["n_nodes"], (1,), generator=gen))
            WL.plant_path(tgt[s], t["parent"], t["token"], node)
    par = np.stack([t["parent"] for t in trees])
    tok = np.stack([t["token"] for t in trees])
    dep = np.stack([t["depth"] for t in trees])
    ns = [t["n_nodes"] for t in trees]
    alen, anodes, bonus, err = _gpu_accept(tgt, w.depth_n, par, tok, dep, ns)
    assert err == 0
    for s in range(len(trees)):
        L, nodes, bb = O.accept(tgt[s].numpy(), par[s], tok[s], dep[s], ns[s], w.depth_n)
        assert (int(alen[s]), int(bonus[s])) == (L, bb), f"{name} seq {s}"
        assert np.array_equal(anodes[s], nodes)
        if plant:
            assert L >= 1


def test_accept_bf16_logits():
    rng = np.random.default_rng(3)
    T, V = 17, 1000
    X = torch.from_numpy((rng.standard_normal((2, T, V)) * 3).astype(np.float32)).to(torch.bfloat16)
    p = [-1] + [0, 1, 2, 3] + [0] * (T - 5)
    d = [0, 1, 2, 3, 4] + [1] * (T - 5)
    Xf = X.float()
    tok = [0] + [int(Xf[0, p[j]].argmax()) if j < 5 else 0 for j in range(1, T)]
    alen, anodes, bonus, err = _gpu_accept(X, 4, [p, p], [tok, tok], [d, d], [T, T])
    assert err == 0
    for s in range(2):
        L, nodes, bb = O.accept(Xf[s].numpy(), p, tok, d, T, 4)
        assert (alen[s], bonus[s]) == (L, bb) and np.array_equal(anodes[s], nodes)
    assert alen[0] == 4


@pytest.mark.parametrize("N,W,Bb", [(24, 2, 100), (40, 1, 60), (17, 3, 200), (64, 1, 100),
                                    (64, 2, 120), (8, 16, 200)])
def test_build_tree_deep(N, W, Bb):
    """Depths past 16 take the kernel variant sized for up to 64 levels; the
    largest depth (64) and width (16) the call takes."""
    rng = np.random.default_rng(N * 100 + W)
    L = (rng.standard_normal((2, N, 500)) * rng.uniform(1, 10)).astype(np.float32)
    roots = np.array([3, 4], dtype=np.int32)
    g = _gpu_build(torch.from_numpy(L), W, Bb, torch.from_numpy(roots))
    for s in range(2):
        ref = O.build_tree(L[s], W, Bb, int(roots[s]), check_exact=False)
        _assert_tree_equal(g, ref, s, f"deep N={N}")


@pytest.mark.parametrize("seed", range(4))
def test_build_tree_ties_at_the_cut(seed):
    """Integer-valued logits make many exact score ties, including at the B-th
    score, where the selection's lower bound cuts the deeper levels."""
    rng = np.random.default_rng(900 + seed)
    N, W, V, b = 6, 4, 12, 3
    L = rng.integers(-3, 3, (b, N, V)).astype(np.float32)
    roots = rng.integers(0, V, b).astype(np.int32)
    for Bb in (50, 123, 300):
        g = _gpu_build(torch.from_numpy(L), W, Bb, torch.from_numpy(roots))
        assert g["err"] == 0
        for s in range(b):
            ref = O.build_tree(L[s], W, Bb, int(roots[s]), check_exact=False)
            _assert_tree_equal(g, ref, s, f"ties seed {seed} B={Bb}")


@pytest.mark.parametrize("case", [
    (2, [100, 20], [257, 256], 257, 8, 1, 128, "bf16"),   # nothing split: direct writes
    (1, [3000], [300], 300, 8, 2, 128, "bf16"),          # split tiles, merged
    (2, [31, 150], [20, 9], 20, 6, 3, 64, "f32"),        # fp32 path
], ids=["direct", "merged", "f32"])
def test_attention_without_lse_is_identical(case):
    """lse is optional: leaving it out changes no output bit."""
    b, prefixes, ns, T, hq, hkv, D, dtype = case
    rng = np.random.default_rng(4242 + T)
    q, k, v, table, num_pages, parents = _attn_case(rng, b, prefixes, ns, T, hq, hkv, D, dtype)
    d = dev()
    par = torch.tensor(parents, dtype=torch.int32, device=d)
    nn = torch.tensor(ns, dtype=torch.int32, device=d)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    anc = B.jt_tree_meta(par, nn, err=err)
    args = (q.to(d), k.to(d), v.to(d), nn, torch.tensor(prefixes, dtype=torch.int32, device=d),
            torch.from_numpy(table).to(d), num_pages, anc, 0.125)
    o1, l1 = B.jt_tree_attention(*args, err=err, with_lse=True)
    o2, l2 = B.jt_tree_attention(*args, err=err, with_lse=False)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and l1 is not None and l2 is None
    for s in range(b):
        assert torch.equal(o1[s, :ns[s]], o2[s, :ns[s]])


def test_step_with_optional_pointers_left_out():
    """The whole step with no error word, no score output and no lse gives
    the same results as with them (the optional pointers only add outputs)."""
    w = WL.WORKLOADS["qwen3_8b_b16"]
    x = WL.make_inputs(w)
    d = dev()
    draft, target, root = x.draft.to(d), x.target.to(d), x.root_token.to(d)
    args_attn = (x.q.to(d), x.k_pool.to(d), x.v_pool.to(d))
    pre, tab = x.prefix_len.to(d), x.page_table.to(d)

    def step(err, opt):
        t = B.jt_build_tree(draft, w.width_w, w.budget_b, root, err=err, with_score=opt)
        anc = B.jt_tree_meta(t["parent"], t["n_nodes"], err=err)
        o, lse = B.jt_tree_attention(*args_attn, t["n_nodes"], pre, tab, x.num_pages, anc,
                                     w.scale, err=err, with_lse=opt)
        acc = B.jt_accept(target, w.depth_n, t["parent"], t["token"], t["depth"], t["n_nodes"],
                          err=err)
        torch.cuda.synchronize()
        return t, anc, o, acc

    err = torch.zeros(1, dtype=torch.int32, device=d)
    t1, a1, o1, acc1 = step(err, True)
    assert int(err.item()) == 0
    t2, a2, o2, acc2 = step(None, False)
    assert t2["score"] is None
    for k in ("parent", "token", "depth", "n_nodes"):
        assert torch.equal(t1[k], t2[k]), k
    assert torch.equal(a1, a2)
    n = int(t1["n_nodes"][0])
    assert torch.equal(o1[:, :n], o2[:, :n])
    for r1, r2 in zip(acc1, acc2):
        assert torch.equal(r1, r2)



def test_build_and_accept_into_preallocated_outputs():
    """Outputs passed in (out=) receive the same results as freshly allocated
    ones, and are rejected when their shape or dtype is wrong."""
    w = WL.WORKLOADS["qwen3_8b_b16"]
    x = WL.make_inputs(w)
    d = dev()
    draft, target, root = x.draft.to(d), x.target.to(d), x.root_token.to(d)
    t1 = B.jt_build_tree(draft, w.width_w, w.budget_b, root)
    a1 = B.jt_accept(target, w.depth_n, t1["parent"], t1["token"], t1["depth"], t1["n_nodes"])
    b, T = draft.shape[0], w.budget_b + 1
    tout = {k: torch.full((b, T), -7, dtype=torch.int32, device=d) for k in ("parent", "token", "depth")}
    tout["score"] = torch.full((b, T), 3.0, dtype=torch.float64, device=d)
    tout["n_nodes"] = torch.full((b,), -7, dtype=torch.int32, device=d)
    t2 = B.jt_build_tree(draft, w.width_w, w.budget_b, root, out=tout)
    assert t2 is tout
    aout = tuple(torch.full(sh, -7, dtype=torch.int32, device=d) for sh in ((b,), (b, w.depth_n), (b,)))
    a2 = B.jt_accept(target, w.depth_n, t2["parent"], t2["token"], t2["depth"], t2["n_nodes"], out=aout)
    torch.cuda.synchronize()
    n = int(t1["n_nodes"][0])
    for k in ("parent", "token", "depth", "n_nodes"):
        assert torch.equal(t1[k][..., :n] if k != "n_nodes" else t1[k], t2[k][..., :n] if k != "n_nodes" else t2[k]), k
    assert torch.equal(t1["score"][:, :n], t2["score"][:, :n])
    for r1, r2, r3 in zip(a1, a2, aout):
        assert torch.equal(r1, r2) and r2 is r3
    bad = dict(tout)
    bad["parent"] = torch.empty((b, T + 1), dtype=torch.int32, device=d)
    with pytest.raises(ValueError):
        B.jt_build_tree(draft, w.width_w, w.budget_b, root, out=bad)
    with pytest.raises(ValueError):
        B.jt_accept(target, w.depth_n, t2["parent"], t2["token"], t2["depth"], t2["n_nodes"],
                    out=(aout[0], aout[1].to(torch.int64), aout[2]))


def test_step_on_a_side_stream():
    """Every call enqueues on the caller's stream: the step run on a second
    (default-priority) stream gives the default stream's results."""
    w = WL.WORKLOADS["qwen3_8b_b16"]
    x = WL.make_inputs(w, instance=1)
    d = dev()
    draft, target, root = x.draft.to(d), x.target.to(d), x.root_token.to(d)
    q, k, v = x.q.to(d), x.k_pool.to(d), x.v_pool.to(d)
    pre, tab = x.prefix_len.to(d), x.page_table.to(d)

    def step():
        err = torch.zeros(1, dtype=torch.int32, device=d)
        t = B.jt_build_tree(draft, w.width_w, w.budget_b, root, err=err)
        anc = B.jt_tree_meta(t["parent"], t["n_nodes"], err=err)
        o, lse = B.jt_tree_attention(q, k, v, t["n_nodes"], pre, tab, x.num_pages, anc, w.scale,
                                     err=err)
        acc = B.jt_accept(target, w.depth_n, t["parent"], t["token"], t["depth"], t["n_nodes"],
                          err=err)
        return [t["parent"], t["token"], t["n_nodes"], anc, o, lse, *acc, err]

    ref = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = step()
    torch.cuda.synchronize()
    assert int(ref[-1].item()) == 0 and int(got[-1].item()) == 0
    n = int(ref[2][0])
    for i, (a, b_) in enumerate(zip(ref, got)):
        if i in (4, 5):  # attention outputs: rows past n_nodes are not written
            a, b_ = a[:, :n], b_[:, :n]
        assert torch.equal(a, b_), i


def test_step_captured_in_a_graph():
    """The step captures into a HIP graph: the library calls enqueue kernels
    only (no allocation, memset or host synchronisation; the binding's output
    tensors come from the graph's memory pool).  Three replays, with eager
    work and synchronisations between them, each reproduce the eager results."""
    w = WL.WORKLOADS["qwen3_8b_b16"]
    x = WL.make_inputs(w, instance=2)
    d = dev()
    draft, target, root = x.draft.to(d), x.target.to(d), x.root_token.to(d)
    q, k, v = x.q.to(d), x.k_pool.to(d), x.v_pool.to(d)
    pre, tab = x.prefix_len.to(d), x.page_table.to(d)
    err = torch.zeros(1, dtype=torch.int32, device=d)

    def step():
        t = B.jt_build_tree(draft, w.width_w, w.budget_b, root, err=err)
        anc = B.jt_tree_meta(t["parent"], t["n_nodes"], err=err)
        o, lse = B.jt_tree_attention(q, k, v, t["n_nodes"], pre, tab, x.num_pages, anc, w.scale,
                                     err=err)
        acc = B.jt_accept(target, w.depth_n, t["parent"], t["token"], t["depth"], t["n_nodes"],
                          err=err)
        return [t["parent"], t["token"], t["n_nodes"], anc, o, lse, *acc]

    ref = [r.clone() for r in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    n = int(ref[2][0])
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for i, (a, b_) in enumerate(zip(ref, outs)):
            if i in (4, 5):
                a, b_ = a[:, :n], b_[:, :n]
            assert torch.equal(a, b_), i


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_bad_page_and_bad_prefix(dtype):
    """A page id outside the pool is reported and its keys and values read as
    zero (the oracle sees an all-zero page there); a sequence whose prefix
    and tree overflow its page table is reported and skipped (rows untouched);
    the other sequences are unaffected."""
    rng = np.random.default_rng(99 if dtype == "bf16" else 98)
    b, prefixes, ns, T, hq, hkv, D = 3, [200, 150, 100], [30, 30, 30], 30, 8, 2, 64
    q, k, v, table, num_pages, parents = _attn_case(rng, b, prefixes, ns, T, hq, hkv, D, dtype)
    bad_table = table.copy()
    bad_table[1, 3] = num_pages + 5          # positions 48..63 of sequence 1 (prefix)
    gpu_prefixes = [200, 150, table.shape[1] * 16]  # sequence 2 overflows its table
    d = dev()
    par = torch.tensor(parents, dtype=torch.int32, device=d)
    nn = torch.tensor(ns, dtype=torch.int32, device=d)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    anc = B.jt_tree_meta(par, nn, err=err)
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device=d)
    o, lse = B.jt_tree_attention(q.to(d), k.to(d), v.to(d), nn,
                                 torch.tensor(gpu_prefixes, dtype=torch.int32, device=d),
                                 torch.from_numpy(bad_table).to(d), num_pages, anc, 1 / np.sqrt(D),
                                 err=err, out=out)
    torch.cuda.synchronize()
    assert int(err.item()) == (B.DERR_BAD_PAGE | B.DERR_BAD_PREFIX)
    og, lg = as_f64(o), to_np(lse).astype(np.float64)
    kf, vf, qf = k.float().numpy(), v.float().numpy(), q.float().numpy()
    # the oracle reads an appended all-zero page where the bad id points
    kz = np.concatenate([kf, np.zeros_like(kf[:1])])
    vz = np.concatenate([vf, np.zeros_like(vf[:1])])
    zero_table = table.copy()
    zero_table[1, 3] = num_pages
    for s in (0, 1):
        ro, rl = O.tree_attention_seq_fast(qf[s], kz, vz, zero_table[s], prefixes[s], parents[s],
                                           ns[s], 1 / np.sqrt(D))
        check_attention(og[s, :ns[s]], ro, dtype, f"seq {s}")
        check_lse(lg[s, :ns[s]], rl, dtype, f"seq {s}")
    assert (og[2] == 7.0).all(), "the skipped sequence must not be written"


def test_accept_bad_depth_reported():
    """depth[v] != depth[parent] + 1, or a node deeper than depth_n: reported,
    that sequence's outputs are zero / -1, the others are unaffected."""
    rng = np.random.default_rng(515)
    T, V, N = 12, 5, 4
    p = [-1, 0, 1, 2, 3, 0, 5, -1, -1, -1, -1, -1]   # a chain of depth 4, then node 6 at depth 2
    dd = [0, 1, 2, 3, 4, 1, 2, -1, -1, -1, -1, -1]
    parents = [p, p, p]
    bad_rel = list(dd)
    bad_rel[6] = 3                                   # its parent 5 has depth 1
    depths = [dd, bad_rel, dd]
    ns = [7, 7, 7]
    tokens = [[int(x) for x in rng.integers(0, V, T)] for _ in range(3)]
    X = torch.from_numpy(rng.standard_normal((3, T, V)).astype(np.float32))
    alen, anodes, bonus, err = _gpu_accept(X, N, parents, tokens, depths, ns)
    assert err == B.DERR_BAD_DEPTH
    assert (alen[1], bonus[1]) == (0, -1) and (anodes[1] == -1).all()
    for s in (0, 2):
        L, nodes, bb = O.accept(X[s].numpy(), parents[s], tokens[s], depths[s], ns[s], N)
        assert (alen[s], bonus[s]) == (L, bb) and np.array_equal(anodes[s], nodes)
    # with depth_n = 3 the depth-4 node of every sequence is too deep
    alen3, anodes3, bonus3, err3 = _gpu_accept(X, 3, parents, tokens, depths, ns)
    assert err3 == B.DERR_BAD_DEPTH
    assert (alen3 == 0).all() and (bonus3 == -1).all() and (anodes3 == -1).all()
