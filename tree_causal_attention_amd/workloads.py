"""Seeded synthetic workloads for the tree verify step.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no softmax, no tree building, no attention, no argmax).
The same CPU tensors feed both the HIP library and the CPU checker, so both
sides see identical bits.

Shapes follow the pages' workloads: Qwen3-8B attention (32 query heads, 8 KV
heads, head_dim 128) and Qwen3-30B-A3B attention (32/4/128), tree budgets 16
and 256 (JetSpec news piece, results paragraphs; JetSpec explainer section
六), serving batch sizes 1, 16 and 32 (explainer section 七), vocabulary
151936 (the Qwen3 tokenizer).  The pages' benchmark suites are not available;
these seeded draws stand in for them.

Recipe (fixed draw order, ``seed = 1000 * workload.index + instance``):

* main generator: per-sequence temperatures T = 2**u, u ~ U[-2, 2] (only for
  workloads with ``temperature``), prefix lengths, root tokens, the page
  permutation;
* one sub-generator per (tensor, sequence): draft logits N(0, sigma)/T,
  K and V rows N(0, 1), Q rows N(0, q_sigma), target logits N(0, sigma).
* sigma is a standard deviation.  bf16 workloads round Q/K/V to bf16
  (round-to-nearest-even); logits stay fp32.
* The pool is paged (16 tokens per page).  Each sequence owns
  ceil((P + B + 1) / 16) pages -- room for its prefix and a full tree tail --
  drawn from one global random permutation of the pool; two spare pages are
  never referenced.  Slots past P + B + 1 and the spare pages hold NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

PAGE_SIZE = 16

_TAG_DRAFT, _TAG_K, _TAG_V, _TAG_Q, _TAG_TARGET = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    dtype: str            # "f32" or "bf16" (attention inputs)
    batch: int
    prefix: int | tuple   # fixed length, or (lo, hi) inclusive uniform range
    hq: int
    hkv: int
    head_dim: int
    depth_n: int
    width_w: int
    budget_b: int
    vocab: int
    sigma: float          # draft and target logit standard deviation
    q_sigma: float
    scale: float
    temperature: bool
    instances: int = 1

    @property
    def max_nodes(self) -> int:
        return self.budget_b + 1


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 0, "f32", 1, 64, 4, 1, 64, 4, 4, 16, 1000, 3.0, 1.0, 0.125, False),
        Workload("qwen3_8b_b16", 1, "bf16", 1, 2048, 32, 8, 128, 8, 4, 16, 151936, 4.0,
                 1 / math.sqrt(128), 1.0, False),
        Workload("qwen3_8b_b256", 2, "bf16", 1, 4096, 32, 8, 128, 16, 8, 256, 151936, 4.0,
                 1 / math.sqrt(128), 1.0, True, instances=8),
        Workload("serving_b16", 3, "bf16", 16, (512, 8192), 32, 8, 128, 16, 8, 256, 151936, 4.0,
                 1 / math.sqrt(128), 1.0, True),
        Workload("serving_b32", 3, "bf16", 32, (512, 8192), 32, 8, 128, 16, 8, 256, 151936, 4.0,
                 1 / math.sqrt(128), 1.0, True),
        Workload("qwen3_30b_a3b_b8", 4, "bf16", 8, 32768, 32, 4, 128, 16, 8, 256, 151936, 4.0,
                 1 / math.sqrt(128), 1.0, False),
    ]
}


def _sub(seed: int, tag: int, seq: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 65536 + tag * 4096 + seq)


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.float()


@dataclass
class Inputs:
    """CPU tensors of one batch (see the module docstring for the recipe)."""
    workload: Workload
    seed: int
    temps: torch.Tensor        # [b] fp32
    prefix_len: torch.Tensor   # [b] int32
    root_token: torch.Tensor   # [b] int32
    page_table: torch.Tensor   # [b, max_pages] int32
    num_pages: int
    k_pool: torch.Tensor       # [num_pages, Hkv, 16, D]
    v_pool: torch.Tensor
    q: torch.Tensor            # [b, B+1, Hq, D]
    draft: torch.Tensor | None   # [b, N, V] fp32
    target: torch.Tensor | None  # [b, B+1, V] fp32


def make_inputs(w: Workload, instance: int = 0, *, with_draft: bool = True,
                with_target: bool = True, batch: int | None = None) -> Inputs:
    """Draw one batch of workload ``w``.  ``batch`` may truncate the batch
    (the first sequences are identical to the full batch's)."""
    seed = 1000 * w.index + instance
    b_full = w.batch
    b = b_full if batch is None else batch
    g = torch.Generator().manual_seed(seed)
    if w.temperature:
        temps = torch.pow(2.0, torch.rand(b_full, generator=g) * 4.0 - 2.0)
    else:
        temps = torch.ones(b_full)
    if isinstance(w.prefix, tuple):
        lo, hi = w.prefix
        prefix = torch.randint(lo, hi + 1, (b_full,), generator=g)
    else:
        prefix = torch.full((b_full,), w.prefix, dtype=torch.int64)
    root = torch.randint(0, w.vocab, (b_full,), generator=g)
    T = w.max_nodes
    pages_per = [(int(p) + T + PAGE_SIZE - 1) // PAGE_SIZE for p in prefix[:b]]
    num_pages = sum(pages_per) + 2
    perm = torch.randperm(num_pages, generator=g)
    max_pages = max(pages_per)
    page_table = torch.full((b, max_pages), -1, dtype=torch.int32)
    off = 0
    for s in range(b):
        page_table[s, :pages_per[s]] = perm[off:off + pages_per[s]].to(torch.int32)
        off += pages_per[s]

    pool_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = (num_pages, w.hkv, PAGE_SIZE, w.head_dim)
    k_pool = torch.full(shape, float("nan"), dtype=pool_dtype)
    v_pool = torch.full(shape, float("nan"), dtype=pool_dtype)
    for s in range(b):
        n_rows = int(prefix[s]) + T
        kr = torch.randn((w.hkv, n_rows, w.head_dim), generator=_sub(seed, _TAG_K, s))
        vr = torch.randn((w.hkv, n_rows, w.head_dim), generator=_sub(seed, _TAG_V, s))
        _scatter(k_pool, page_table[s], _cast(kr, w.dtype))
        _scatter(v_pool, page_table[s], _cast(vr, w.dtype))

    q = torch.empty((b, T, w.hq, w.head_dim), dtype=pool_dtype)
    for s in range(b):
        q[s] = _cast(torch.randn((T, w.hq, w.head_dim), generator=_sub(seed, _TAG_Q, s))
                     * w.q_sigma, w.dtype)

    draft = None
    if with_draft:
        draft = torch.empty((b, w.depth_n, w.vocab), dtype=torch.float32)
        for s in range(b):
            draft[s] = (torch.randn((w.depth_n, w.vocab), generator=_sub(seed, _TAG_DRAFT, s))
                        * w.sigma / temps[s])
    target = None
    if with_target:
        target = torch.empty((b, T, w.vocab), dtype=torch.float32)
        for s in range(b):
            target[s] = torch.randn((T, w.vocab), generator=_sub(seed, _TAG_TARGET, s)) * w.sigma
    return Inputs(w, seed, temps[:b].float(), prefix[:b].to(torch.int32),
                  root[:b].to(torch.int32), page_table, num_pages, k_pool, v_pool, q,
                  draft, target)


def _scatter(pool: torch.Tensor, table_row: torch.Tensor, rows: torch.Tensor) -> None:
    """Write logical rows [Hkv, n, D] of one sequence into its pages."""
    n = rows.shape[1]
    t = torch.arange(n)
    pages = table_row[(t // PAGE_SIZE)].long()
    slots = t % PAGE_SIZE
    pool[pages, :, slots, :] = rows.transpose(0, 1)


def plant_path(target: torch.Tensor, parent, token, node: int, bump: float = 50.0) -> None:
    """Make the target agree with the draft along the root->``node`` path.

    For every node u on the path (root excluded) adds ``bump`` to
    target[parent(u), token(u)], so that token(u) becomes the argmax of its
    parent's row (test input construction for long accepted paths).
    ``target`` is one sequence's [T, V] tensor, modified in place.
    """
    u = int(node)
    while u > 0:
        p = int(parent[u])
        target[p, int(token[u])] += bump
        u = p


def random_recursive_parents(n: int, gen: torch.Generator) -> list:
    """parent[0] = -1, parent[j] uniform in [0, j): a random recursive tree."""
    return [-1] + [int(torch.randint(0, j, (1,), generator=gen)) for j in range(1, n)]
