"""Pins for the oracle's tree-causal mask and paged tree attention.

Checks against: torch's scaled_dot_product_attention in float64 (causal
chunked prefill for a chain tree, decode for a one-node tree, and single-query
attention over an explicitly concatenated root-to-node path for every
recursive tree of up to 8 nodes), torch.logsumexp, structural identities of
the mask, and invariances the definition implies (masked K/V cannot matter,
page order cannot matter, GQA equals MHA with repeated KV heads).
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import tree_oracle as O

PS = 16


def _pool(rng, n_rows, hkv, d, pages_extra=2):
    """Random paged pool holding n_rows logical rows, randomly permuted."""
    n_pages = (n_rows + PS - 1) // PS + pages_extra
    perm = rng.permutation(n_pages)
    table = perm[: (n_rows + PS - 1) // PS]
    k = rng.standard_normal((n_pages, hkv, PS, d))
    v = rng.standard_normal((n_pages, hkv, PS, d))
    return k, v, table


def _logical(pool, table, n):
    t = np.arange(n)
    return pool[table[t // PS], :, t % PS, :]  # [n, hkv, d]


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in float64. q [H, nq, d], k/v [H, nk, d], mask [nq, nk]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(mask), scale=scale)[0].numpy()


# ------------------------------------------------------------------- mask

def test_mask_structure():
    rng = np.random.default_rng(0)
    for n in (1, 2, 5, 40):
        par = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
        M = O.ancestor_mask(par, n)
        depth = [0] * n
        for j in range(1, n):
            depth[j] = depth[par[j]] + 1
        assert all(M[i].sum() == depth[i] + 1 for i in range(n))
        assert all(M[i, 0] and M[i, i] for i in range(n))
        assert not np.triu(M, 1).any()   # parent[j] < j keeps it lower-triangular
    chain = [-1] + list(range(0, 9))
    assert (O.ancestor_mask(chain, 10) == np.tril(np.ones((10, 10), bool))).all()
    star = [-1] + [0] * 9
    exp = np.eye(10, dtype=bool)
    exp[:, 0] = True
    assert (O.ancestor_mask(star, 10) == exp).all()


def test_mask_words_layout():
    par = [-1, 0, 1, 0, 3] + list(range(4, 40))
    n = len(par)
    W = O.ancestor_words(par, n, 50)
    M = O.ancestor_mask(par, n)
    assert W.shape == (50, 2) and W.dtype == np.uint32
    for i in range(50):
        for j in range(64):
            bit = (int(W[i, j // 32]) >> (j % 32)) & 1
            assert bit == (1 if (i < n and j < n and M[i, j]) else 0)


# ------------------------------------------------------------- attention

def _run(q, k, v, table, P, par, n, scale, fast=False):
    f = O.tree_attention_seq_fast if fast else O.tree_attention_seq
    return f(q, k, v, table, P, par, n, scale)


@pytest.mark.parametrize("P,n", [(0, 1), (0, 7), (13, 9), (40, 20), (16, 16)])
def test_chain_equals_causal_prefill(P, n):
    rng = np.random.default_rng(P * 31 + n)
    hq, hkv, d, scale = 4, 2, 8, 0.3
    k, v, table = _pool(rng, P + n, hkv, d)
    q = rng.standard_normal((n, hq, d))
    par = [-1] + list(range(n - 1))
    K = _logical(k, table, P + n).repeat(hq // hkv, axis=1).transpose(1, 0, 2)
    Vv = _logical(v, table, P + n).repeat(hq // hkv, axis=1).transpose(1, 0, 2)
    mask = np.arange(P + n)[None, :] <= (P + np.arange(n))[:, None]   # bottom-right aligned
    ref = _sdpa(np.ascontiguousarray(q.transpose(1, 0, 2)), K, Vv, mask, scale).transpose(1, 0, 2)
    for fast in (False, True):
        o, _ = _run(q, k, v, table, P, par, n, scale, fast)
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P", [0, 1, 31, 100])
def test_single_node_equals_decode(P):
    rng = np.random.default_rng(P)
    hq, hkv, d, scale = 6, 3, 16, 0.25
    k, v, table = _pool(rng, P + 1, hkv, d)
    q = rng.standard_normal((1, hq, d))
    K = _logical(k, table, P + 1).repeat(2, axis=1).transpose(1, 0, 2)
    Vv = _logical(v, table, P + 1).repeat(2, axis=1).transpose(1, 0, 2)
    ref = _sdpa(np.ascontiguousarray(q.transpose(1, 0, 2)), K, Vv,
                np.ones((1, P + 1), bool), scale).transpose(1, 0, 2)
    for fast in (False, True):
        o, lse = _run(q, k, v, table, P, [-1], 1, scale, fast)
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
        s = scale * np.einsum("hd,hkd->hk", q[0], K)
        np.testing.assert_allclose(lse[0], torch.logsumexp(torch.from_numpy(s), -1).numpy(),
                                   rtol=1e-13)


def _recursive_trees(n):
    for choice in itertools.product(*[range(j) for j in range(1, n)]):
        yield [-1] + list(choice)


@pytest.mark.slow
def test_every_small_tree_against_path_concatenation():
    """All 5914 recursive trees of 1..8 nodes: each node's output equals
    single-query attention over prefix K/V concatenated with the K/V of the
    node's root-to-node path (found here by walking parents)."""
    rng = np.random.default_rng(11)
    hq, hkv, d, scale, P = 2, 1, 4, 0.7, 5
    k, v, table = _pool(rng, P + 8, hkv, d)
    Kall = _logical(k, table, P + 8)[:, 0]
    Vall = _logical(v, table, P + 8)[:, 0]
    q = rng.standard_normal((8, hq, d))
    count = 0
    for n in range(1, 9):
        for par in _recursive_trees(n):
            count += 1
            o, lse = O.tree_attention_seq(q, k, v, table, P, par, n, scale)
            of, lsef = O.tree_attention_seq_fast(q, k, v, table, P, par, n, scale)
            np.testing.assert_allclose(of, o, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lsef, lse, rtol=1e-13, atol=1e-13)
            for i in range(n):
                path, u = [], i
                while u >= 0:
                    path.append(u)
                    u = par[u]
                rows = list(range(P)) + [P + u for u in reversed(path)]
                Kp = np.repeat(Kall[rows][None], hq, 0)
                Vp = np.repeat(Vall[rows][None], hq, 0)
                ref = _sdpa(np.ascontiguousarray(q[i][:, None, :]), Kp, Vp,
                            np.ones((1, len(rows)), bool), scale)[:, 0]
                np.testing.assert_allclose(o[i], ref, rtol=1e-12, atol=1e-13)
    assert count == 5914


def test_masked_kv_cannot_change_a_node():
    rng = np.random.default_rng(5)
    hq, hkv, d, scale, P, n = 4, 2, 8, 0.4, 21, 30
    k, v, table = _pool(rng, P + n, hkv, d)
    q = rng.standard_normal((n, hq, d))
    par = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
    for fast in (False, True):
        base, base_lse = _run(q, k, v, table, P, par, n, scale, fast)
        for i in (0, 7, n - 1):
            anc = set(O.ancestors(par, i))
            k2, v2 = k.copy(), v.copy()
            for j in range(n):
                if j not in anc:
                    t = P + j
                    k2[table[t // PS], :, t % PS] = rng.standard_normal((hkv, d)) * 100
                    v2[table[t // PS], :, t % PS] = rng.standard_normal((hkv, d)) * 100
            o2, lse2 = _run(q, k2, v2, table, P, par, n, scale, fast)
            assert np.array_equal(o2[i], base[i]) and np.array_equal(lse2[i], base_lse[i])


def test_gqa_equals_repeated_mha_and_page_order_invariance():
    rng = np.random.default_rng(9)
    hq, hkv, d, scale, P, n = 8, 2, 8, 0.5, 37, 12
    k, v, table = _pool(rng, P + n, hkv, d)
    q = rng.standard_normal((n, hq, d))
    par = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
    o, lse = O.tree_attention_seq(q, k, v, table, P, par, n, scale)
    o_mha, lse_mha = O.tree_attention_seq(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                          table, P, par, n, scale)
    assert np.array_equal(o, o_mha) and np.array_equal(lse, lse_mha)
    perm = rng.permutation(k.shape[0])       # new slot of every page
    k_p = np.empty_like(k)
    v_p = np.empty_like(v)
    k_p[perm] = k
    v_p[perm] = v
    o_p, lse_p = O.tree_attention_seq(q, k_p, v_p, perm[table], P, par, n, scale)
    assert np.array_equal(o, o_p) and np.array_equal(lse, lse_p)


def test_lse_is_log_normaliser():
    rng = np.random.default_rng(2)
    hq, hkv, d, scale, P, n = 2, 1, 8, 0.9, 9, 6
    k, v, table = _pool(rng, P + n, hkv, d)
    q = rng.standard_normal((n, hq, d))
    par = [-1, 0, 0, 1, 2, 2]
    o, lse = O.tree_attention_seq(q, k, v, table, P, par, n, scale)
    K = _logical(k, table, P + n)[:, 0]
    for i in range(n):
        rows = list(range(P)) + [P + u for u in O.ancestors(par, i)]
        for h in range(hq):
            s = torch.from_numpy(scale * K[rows] @ q[i, h])
            assert abs(lse[i, h] - float(torch.logsumexp(s, 0))) < 1e-13
