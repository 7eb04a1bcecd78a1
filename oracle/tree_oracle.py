"""Plain, slow, fp64 CPU oracle for the tree speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in the repository's
entry module, and the CPU-baseline leg of the benchmark use it.  It shares no
code with the HIP library and imports nothing from the product package.

What it computes (sources are the four web pages the method is described on):

* ``build_tree``   -- candidate tree: top-W tokens per depth, then best-first
  expansion by cumulative draft log-probability until the node budget B is
  spent.  JetSpec news piece (mlqm.cn/news/158889), paragraph on building the
  candidate tree each decode step (max depth N, width W, budget B, top-W per
  layer, greedy expansion by cumulative draft log-prob); JetSpec explainer
  (techwalker.com, "加速AI思考…"), section 五 (priority queue keyed by the
  path's cumulative log-probability, up to W children, stop at B).
* ``ancestor_mask`` -- the tree-causal mask: a node sees the prefix and the
  nodes on its own root-to-node branch (itself included), never siblings or
  descendants.  JetSpec news piece, paragraph on the one-forward solution
  (tree-causal attention mask); JetSpec explainer, section 三.
* ``tree_attention`` -- one-pass verification attention of every tree node
  over a paged KV cache: prefix plus the node's ancestors in the tree tail.
  JetSpec explainer, section 七 (paged tree attention with tree-tail masking);
  section 三 (the target verifies all candidate paths in one forward).
* ``accept``       -- greedy acceptance: a node is accepted when its parent is
  accepted and its token equals the target's argmax after the parent; the
  deepest accepted node ends the path.  JetSpec news piece (longest consistent
  prefix under the SD acceptance rule); explainer section 三 (longest accepted
  prefix along each path); SD overview (chooseai.io/news/6515), section on when
  "lossless" fails (at temperature 0 a draft token is accepted only when it
  equals the target's choice).

Readings where the pages leave a step open (numbered as in the design notes):

* B counts drafted nodes; node 0 is the root (the last accepted token), so a
  tree has up to B+1 nodes and the target has B+1 logit rows (row r is the
  target's prediction after node r).
* One queue pop adds ONE candidate to the tree; a popped node of depth < N
  then offers its W children as new candidates.
* Candidates are per depth: every depth-d node's children are the same top-W
  tokens of draft row d.
* score(node) = sum over its path of log-softmax(draft row depth)[token]; the
  root scores 0.  Arithmetic: raw = fp64 sum of the fp32 logits along the path
  (root to node, left to right), S_d = fp64 prefix sum of the per-depth
  log-sum-exp, score = raw - S_d.
* Top-W order: logit descending, then token id ascending.
* Queue order: key (-score, parent node index, candidate rank), ascending.
* Drafted nodes are numbered in pop order, so parent[j] < j.
* A node sees itself (ancestor-or-self set).
* The tree tail's K/V sit in the paged pool at logical positions
  prefix_len + j, in node-index order.
* Greedy argmax ties go to the lowest token id; the deepest accepted node wins,
  ties to the lower node index.

Precision: every floating-point step is fp64.  Inputs arrive as fp32 or bf16
values; both convert to fp64 exactly.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

PAGE_SIZE = 16


class OracleInputError(ValueError):
    """The inputs fall outside the operation's contract (NaN, +inf, ...)."""


# ---------------------------------------------------------------------------
# a1: per-depth log-sum-exp and top-W candidates
# ---------------------------------------------------------------------------

def draft_row_stats(row: np.ndarray, width: int):
    """Log-sum-exp (fp64) and the top-``width`` tokens of one draft logit row.

    Follows the JetSpec news piece's tree-construction paragraph (top-W per
    depth) with the readings above: order is logit descending, token id
    ascending.  Entries may be finite or -inf (an excluded token); NaN, +inf
    and rows with no finite entry are outside the contract.

    Returns (lse, cand_tok[int64, width], cand_val[fp64, width]).
    """
    x = np.asarray(row, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any():
        raise OracleInputError("draft logits must be finite or -inf")
    if not np.isfinite(x).any():
        raise OracleInputError("a draft row needs at least one finite logit")
    if not 1 <= width <= x.shape[0]:
        raise OracleInputError("need 1 <= W <= vocab")
    m = x.max()
    s = np.exp(x - m).sum()
    lse = m + np.log(s)
    ids = np.arange(x.shape[0])
    order = np.lexsort((ids, -x))  # primary: -logit ascending; secondary: id
    cand = order[:width]
    return float(lse), cand.astype(np.int64), x[cand].copy()


# ---------------------------------------------------------------------------
# a2: best-first tree construction
# ---------------------------------------------------------------------------

def build_tree(draft_logits: np.ndarray, width: int, budget: int, root_token: int,
               check_exact: bool = True):
    """Best-first candidate tree of one sequence.

    ``draft_logits``: [N, V] (row d-1 holds the logits of depth d).
    Returns a dict with parent/token/depth (int64, length B+1, -1 padded),
    score (fp64, -inf padded), raw (fp64), n_nodes, lse [N], cand_tok [N, W],
    plus ``margin`` (smallest non-zero score gap between adjacent decisions),
    ``cross_depth_ties`` (exact score ties decided across different depths)
    and ``raw_exact`` (every raw path sum equals the exact rational sum).

    Steps follow the JetSpec explainer, section 五, under the candidate-level
    reading: the frontier holds candidates (parent node, rank); the best one
    by (-score, parent, rank) is popped into the tree; if it is shallower than
    N its W children join the frontier; stop after B pops or when the
    frontier is empty.
    """
    L = np.asarray(draft_logits)
    n_depth, vocab = L.shape
    if budget < 0:
        raise OracleInputError("budget must be >= 0")
    lse = np.empty(n_depth)
    cand_tok = np.empty((n_depth, width), dtype=np.int64)
    cand_val = np.empty((n_depth, width))
    for d in range(n_depth):
        lse[d], cand_tok[d], cand_val[d] = draft_row_stats(L[d], width)
    # S[d] = lse_1 + ... + lse_d, added left to right; S[0] = 0 for the root.
    S = [0.0]
    for d in range(n_depth):
        S.append(S[-1] + float(lse[d]))

    parent = [-1]
    token = [int(root_token)]
    depth = [0]
    raw = [0.0]
    score = [0.0]
    logit = [0.0]  # the draft logit each node added to its path sum

    # Frontier as parallel lists; one entry per candidate (parent node, rank).
    f_parent, f_rank, f_raw, f_score = [], [], [], []

    def offer_children(p):
        dd = depth[p] + 1
        for k in range(width):
            r = raw[p] + float(cand_val[dd - 1, k])
            f_parent.append(p)
            f_rank.append(k)
            f_raw.append(r)
            f_score.append(r - S[dd])

    if n_depth >= 1:
        offer_children(0)

    pop_scores, pop_depths = [], []
    while len(parent) - 1 < budget and f_parent:
        sc = np.asarray(f_score)
        best = sc.max()
        tied = np.flatnonzero(sc == best)
        # linear scan over the tied entries for the smallest (parent, rank)
        i = min(tied, key=lambda t: (f_parent[t], f_rank[t]))
        p, k = f_parent[i], f_rank[i]
        dd = depth[p] + 1
        parent.append(p)
        depth.append(dd)
        token.append(int(cand_tok[dd - 1, k]))
        raw.append(f_raw[i])
        score.append(f_score[i])
        logit.append(float(cand_val[dd - 1, k]))
        pop_scores.append(f_score[i])
        pop_depths.append(dd)
        for lst in (f_parent, f_rank, f_raw, f_score):
            lst.pop(i)
        if dd < n_depth:
            offer_children(len(parent) - 1)

    n_nodes = len(parent)
    # decision margins: adjacent pops, plus the budget cut against the best
    # candidate left behind.
    seq_scores = list(pop_scores)
    seq_depths = list(pop_depths)
    if f_score:
        j = int(np.argmax(f_score))
        seq_scores.append(f_score[j])
        seq_depths.append(depth[f_parent[j]] + 1)
    margin = np.inf
    cross_ties = 0
    for a in range(len(seq_scores) - 1):
        gap = seq_scores[a] - seq_scores[a + 1]
        if gap > 0:
            margin = min(margin, gap)
        elif gap == 0 and seq_depths[a] != seq_depths[a + 1]:
            cross_ties += 1

    raw_exact = True
    if check_exact:
        for v in range(1, n_nodes):
            terms = []
            u = v
            while u != 0:
                terms.append(logit[u])
                u = parent[u]
            if not all(np.isfinite(terms)):
                if raw[v] != -np.inf:  # an excluded token makes the path -inf
                    raw_exact = False
                    break
                continue
            acc = sum((Fraction(x) for x in terms), Fraction(0))
            if Fraction(raw[v]) != acc:
                raw_exact = False
                break

    size = budget + 1
    out_parent = np.full(size, -1, dtype=np.int64)
    out_token = np.full(size, -1, dtype=np.int64)
    out_depth = np.full(size, -1, dtype=np.int64)
    out_score = np.full(size, -np.inf)
    out_raw = np.full(size, -np.inf)
    out_parent[:n_nodes] = parent
    out_token[:n_nodes] = token
    out_depth[:n_nodes] = depth
    out_score[:n_nodes] = score
    out_raw[:n_nodes] = raw
    return dict(parent=out_parent, token=out_token, depth=out_depth, score=out_score,
                raw=out_raw, n_nodes=n_nodes, lse=lse, cand_tok=cand_tok,
                cand_val=cand_val, margin=margin, cross_depth_ties=cross_ties,
                raw_exact=raw_exact)


def build_tree_batch(draft_logits: np.ndarray, width: int, budget: int, root_tokens):
    """``build_tree`` for each sequence of a [b, N, V] batch."""
    return [build_tree(draft_logits[s], width, budget, int(root_tokens[s]))
            for s in range(draft_logits.shape[0])]


# ---------------------------------------------------------------------------
# a3: tree-causal mask
# ---------------------------------------------------------------------------

def ancestors(parent, i):
    """Ancestor-or-self set of node ``i`` by walking parent pointers."""
    out = []
    while i != -1:
        out.append(int(i))
        i = int(parent[i])
    return out[::-1]


def ancestor_mask(parent, n_nodes):
    """Dense tail mask M[i, j] = (j is i or an ancestor of i), [n, n] bool.

    The tree-causal rule of the JetSpec news piece (one-forward solution
    paragraph) and the explainer's section 三, read with self-visibility.
    """
    M = np.zeros((n_nodes, n_nodes), dtype=bool)
    for i in range(n_nodes):
        M[i, ancestors(parent, i)] = True
    return M


def ancestor_words(parent, n_nodes, max_nodes):
    """The mask packed as uint32 words: bit (j % 32) of word j // 32 of row i.

    Rows at or past ``n_nodes`` are zero.  Shape [max_nodes, ceil(max_nodes/32)].
    """
    nw = (max_nodes + 31) // 32
    out = np.zeros((max_nodes, nw), dtype=np.uint32)
    M = ancestor_mask(parent, n_nodes)
    for i in range(n_nodes):
        for j in np.flatnonzero(M[i]):
            out[i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return out


# ---------------------------------------------------------------------------
# a4: paged tree attention
# ---------------------------------------------------------------------------

def gather_kv(pool, page_table_row, length):
    """Logical rows 0..length-1 of one sequence from a paged pool.

    pool: [num_pages, Hkv, PAGE_SIZE, D]; returns [Hkv, length, D] fp64.
    Row t lives in page page_table_row[t // 16], slot t % 16.
    """
    t = np.arange(length)
    pages = np.asarray(page_table_row)[t // PAGE_SIZE]
    slots = t % PAGE_SIZE
    rows = np.asarray(pool)[pages, :, slots, :]  # [length, Hkv, D]
    return np.ascontiguousarray(rows.transpose(1, 0, 2)).astype(np.float64)


def tree_attention_seq(q, k_pool, v_pool, page_table_row, prefix_len, parent, n_nodes,
                       scale, nodes=None, heads=None):
    """Tree attention of one sequence, straight from the definition.

    q: [T, Hq, D] (T >= n_nodes).  Returns (o [n, Hq, D], lse [n, Hq]) in fp64
    for the selected nodes (default all n_nodes) and heads (default all);
    unselected entries are NaN.

    For node i and query head h (KV head g = h // (Hq // Hkv)): the visible
    keys are the prefix positions t < P and the tail positions P + j for j in
    the ancestor-or-self set of i; masked keys are left out of the sum
    entirely.  s = scale * q.k, o = softmax(s) @ v, lse = log sum exp(s).
    """
    q = np.asarray(q)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = np.asarray(k_pool).shape[1]
    group = Hq // Hkv
    P = int(prefix_len)
    K = gather_kv(k_pool, page_table_row, P + n_nodes)
    V = gather_kv(v_pool, page_table_row, P + n_nodes)
    nodes = range(n_nodes) if nodes is None else nodes
    heads = range(Hq) if heads is None else heads
    o = np.full((n_nodes, Hq, D), np.nan)
    lse = np.full((n_nodes, Hq), np.nan)
    for i in nodes:
        keys = np.concatenate([np.arange(P), P + np.asarray(ancestors(parent, i))])
        for h in heads:
            g = h // group
            qv = q[i, h].astype(np.float64)
            s = scale * (K[g, keys] @ qv)
            m = s.max()
            e = np.exp(s - m)
            z = e.sum()
            o[i, h] = (e @ V[g, keys]) / z
            lse[i, h] = m + np.log(z)
    return o, lse


def tree_attention_seq_fast(q, k_pool, v_pool, page_table_row, prefix_len, parent, n_nodes,
                            scale):
    """The same quantity as ``tree_attention_seq``, organised per head.

    The prefix part is one dense product per head (every node sees every prefix
    key); the tail part uses the dense ancestor mask from ``ancestor_mask``.
    Masked tail scores never enter the exponentials (np.where selects 0 for
    them); masked V rows are multiplied by an exact 0, so for finite tail
    values this equals leaving them out.
    """
    q = np.asarray(q)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = np.asarray(k_pool).shape[1]
    group = Hq // Hkv
    P = int(prefix_len)
    n = int(n_nodes)
    K = gather_kv(k_pool, page_table_row, P + n)
    V = gather_kv(v_pool, page_table_row, P + n)
    M = ancestor_mask(parent, n)
    o = np.empty((n, Hq, D))
    lse = np.empty((n, Hq))
    for h in range(Hq):
        g = h // group
        Q = q[:n, h].astype(np.float64)
        s_pre = scale * (Q @ K[g, :P].T)            # [n, P]
        s_tail = scale * (Q @ K[g, P:P + n].T)      # [n, n]
        s_tail_m = np.where(M, s_tail, -np.inf)
        m = np.maximum(s_pre.max(axis=1, initial=-np.inf), s_tail_m.max(axis=1))
        e_pre = np.exp(s_pre - m[:, None])
        e_tail = np.where(M, np.exp(np.where(M, s_tail, 0.0) - m[:, None]), 0.0)
        z = e_pre.sum(axis=1) + e_tail.sum(axis=1)
        num = e_pre @ V[g, :P] + e_tail @ V[g, P:P + n]
        o[:, h] = num / z[:, None]
        lse[:, h] = m + np.log(z)
    return o, lse


# ---------------------------------------------------------------------------
# a5: greedy acceptance
# ---------------------------------------------------------------------------

def accept(target_logits, parent, token, depth, n_nodes, n_depth):
    """Greedy tree acceptance of one sequence.

    target_logits: [T, V]; row r is the target's next-token logits after node
    r.  a_r = argmax (first maximum = lowest id).  Node v > 0 is accepted when
    its parent is accepted and token[v] == a_{parent[v]}; the root is always
    accepted.  The path ends at the deepest accepted node (lowest index among
    equals).  Returns (accept_len, accept_nodes [n_depth], bonus_token).
    """
    X = np.asarray(target_logits)[:n_nodes].astype(np.float64)
    if np.isnan(X).any():
        raise OracleInputError("target logits must not be NaN")
    a = np.argmax(X, axis=1)
    acc = np.zeros(n_nodes, dtype=bool)
    acc[0] = True
    for v in range(1, n_nodes):
        p = int(parent[v])
        acc[v] = acc[p] and int(token[v]) == int(a[p])
    best = 0
    for v in range(1, n_nodes):
        if acc[v] and depth[v] > depth[best]:
            best = v
    path = ancestors(parent, best)[1:]
    nodes = np.full(n_depth, -1, dtype=np.int64)
    nodes[:len(path)] = path
    return int(depth[best]), nodes, int(a[best])


# ---------------------------------------------------------------------------
# f3: margin acceptance (AdaptiveSpec's per-step margin rule)
# ---------------------------------------------------------------------------

def accept_margin(target_logits, parent, token, depth, n_nodes, n_depth, logit_margin):
    """Margin acceptance of one sequence.

    AdaptiveSpec page (kongchang.com, "AdaptiveSpec：免训练推测解码方案提速56%的
    技术解析"), section on the per-step margin rule: a drafted token is kept
    when the target's probability of it, divided by the target's top-1
    probability, reaches a threshold theta, even if it is not the top-1 token.
    With p = softmax(L / T) the ratio is exp((L[x] - max L) / T), so the test
    is L[x] - max L >= T ln(theta) =: logit_margin (<= 0).

    Reading: the test is evaluated in fp64 on the stored logits (fp32 or bf16
    values, exact in fp64); the root is accepted; node v >= 1 is accepted when
    its parent is accepted and its token passes the test on the parent's row;
    the path ends at the deepest accepted node (lowest index among equals); the
    bonus token is the argmax (lowest id) of the end node's row.  With
    logit_margin = 0 only tokens tied with the maximum pass.
    Returns (accept_len, accept_nodes [n_depth], bonus_token).
    """
    X = np.asarray(target_logits)[:n_nodes].astype(np.float64)
    if np.isnan(X).any():
        raise OracleInputError("target logits must not be NaN")
    if not (logit_margin <= 0.0 and np.isfinite(logit_margin)):
        raise OracleInputError("logit_margin must be finite and <= 0")
    top = X.max(axis=1)
    a = np.argmax(X, axis=1)
    acc = [False] * n_nodes
    acc[0] = True
    for v in range(1, n_nodes):
        p = int(parent[v])
        acc[v] = acc[p] and (X[p, int(token[v])] - top[p] >= logit_margin)
    best = 0
    for v in range(1, n_nodes):
        if acc[v] and depth[v] > depth[best]:
            best = v
    path = ancestors(parent, best)[1:]
    nodes = np.full(n_depth, -1, dtype=np.int64)
    nodes[:len(path)] = path
    return int(depth[best]), nodes, int(a[best])


def margin_from_ratio(theta, temperature=1.0):
    """logit_margin = T ln(theta) for a probability-ratio threshold theta in (0, 1]."""
    import math
    return float(temperature) * math.log(float(theta))


# ---------------------------------------------------------------------------
# f1: committing the accepted path to the KV cache
# ---------------------------------------------------------------------------

def commit_kv(k_pool, v_pool, page_table_row, prefix_len, accept_len, accept_nodes):
    """KV commit of one sequence after acceptance (returns new pools and prefix).

    Follows from where the tree tail lives (node j at logical position P + j,
    design reading R10) and from the step the JetSpec news piece describes
    next: the next decode step starts from the state the verification accepted.
    The root (node 0, position P) stays; the k-th accepted node a_k
    (k = 1..L, depth order) moves from position P + a_k to P + k; positions
    past P + L are left as they are; the new prefix length is P + 1 + L.
    All source rows are read before any row is written.
    """
    k_pool = np.array(k_pool, copy=True)
    v_pool = np.array(v_pool, copy=True)
    P = int(prefix_len)
    L = int(accept_len)
    table = np.asarray(page_table_row)
    src = [P + int(accept_nodes[k]) for k in range(L)]
    rows_k = [k_pool[table[t // PAGE_SIZE], :, t % PAGE_SIZE, :].copy() for t in src]
    rows_v = [v_pool[table[t // PAGE_SIZE], :, t % PAGE_SIZE, :].copy() for t in src]
    for k in range(L):
        t = P + 1 + k
        k_pool[table[t // PAGE_SIZE], :, t % PAGE_SIZE, :] = rows_k[k]
        v_pool[table[t // PAGE_SIZE], :, t % PAGE_SIZE, :] = rows_v[k]
    return k_pool, v_pool, P + 1 + L


def decode_attention(q, k_pool, v_pool, page_table_row, length, scale):
    """Plain decode attention of one query over logical positions 0..length-1.

    q: [Hq, D].  Returns (o [Hq, D], lse [Hq]) in fp64: s = scale * q.k over
    every key, o = softmax(s) @ v, lse = log sum exp(s).
    """
    q = np.asarray(q)
    Hq = q.shape[0]
    Hkv = np.asarray(k_pool).shape[1]
    group = Hq // Hkv
    K = gather_kv(k_pool, page_table_row, length)
    V = gather_kv(v_pool, page_table_row, length)
    o = np.empty((Hq, q.shape[1]))
    lse = np.empty(Hq)
    for h in range(Hq):
        g = h // group
        s = scale * (K[g] @ q[h].astype(np.float64))
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        o[h] = (e @ V[g]) / z
        lse[h] = m + np.log(z)
    return o, lse


# ---------------------------------------------------------------------------
# f2: lossless stochastic verification of the tree (temperature sampling)
# ---------------------------------------------------------------------------

def softmax_t(row, temperature):
    """softmax(row / T) in fp64: exp((x - max) / T) / sum (fp64 throughout)."""
    x = np.asarray(row).astype(np.float64)
    m = x.max()
    e = np.exp((x - m) / float(temperature))
    return e / e.sum()


def sample_index(p, u):
    """Inverse-CDF draw: the smallest index y with cumsum(p)[y] > u * sum(p).

    cumsum in index order (fp64, left to right); u in [0, 1).
    """
    c = np.cumsum(np.asarray(p, dtype=np.float64))
    t = float(u) * c[-1]
    return int(np.searchsorted(c, t, side="right"))


def _check_stochastic_rows(rows):
    for arr in rows:
        arr = np.asarray(arr, dtype=np.float64)
        if np.isnan(arr).any() or np.isposinf(arr).any():
            raise OracleInputError("logits must not be NaN or +inf")
        if (arr.max(axis=-1) == -np.inf).any():
            raise OracleInputError("every logit row needs a finite entry")


def accept_stochastic(target_logits, draft_logits, parent, token, depth, n_nodes, n_depth,
                      temperature, u_accept, u_sample, margins=None, draft_mode="topw"):
    """Stochastic (temperature T > 0) verification of one sequence's tree.

    The SD overview (chooseai.io/news/6515), section on what speculative
    decoding is, and the AdaptiveSpec page (kongchang.com), section on the
    strict token-matching rule, state the rule for one drafted token x: with
    draft distribution q and target distribution p, accept x with probability
    min(1, p(x) / q(x)); on rejection draw from norm(max(0, p - q)).  The
    output then has the target's distribution.

    What q is depends on how the tree's tokens were proposed, so the rule
    takes the proposal as a mode:

    * ``draft_mode="topw"`` (the trees the build step makes).  The JetSpec
      news piece (tree-construction paragraph) and explainer (section 五)
      build each depth's siblings as the W most likely draft tokens: they are
      chosen, not sampled, so the proposal behind the k-th sibling, given
      that the earlier ones were rejected, is the point mass on its token.
      With q = point mass at x the rule reads: accept x with probability
      min(1, p(x) / 1) = p(x); on rejection the residual norm(max(0, p - q))
      is p with x removed, renormalised.  The draft logits are not used.
    * ``draft_mode="sampled"``.  Every child of a node was drawn
      independently from q = softmax(draft row of its depth / T); the rule
      is applied child after child with that same q, each rejection replacing
      p by norm(max(0, p - q)).  This is lossless only under that sampling
      assumption (it is not for top-W siblings).

    Common readings (the pages state the rule for one token):
    * p at node u is softmax(target row u / T).
    * The children of the current node are tried in node-index order (their
      candidate rank).  Child v with token x is accepted iff
      u_accept[v] * q(x) < p(x) (topw: u_accept[v] < p(x)), p being the
      current distribution.  An accepted child becomes the current node.
    * When no child is accepted (or there is none) the walk stops and the
      bonus token is drawn from the current p with u_sample (sample_index).
    * If a rejection leaves no mass (the residual sums to zero) the
      remaining children are not tried and the bonus is drawn from p as it
      was before that rejection.
    Randomness is passed in: u_accept [n_nodes] (one uniform per node, used
    when that node is tried), u_sample (one uniform), all in [0, 1).
    Returns (accept_len, accept_nodes [n_depth], bonus_token).

    margins: optional list; each decision appends how far it was from flipping,
    relative to the quantities compared (|u q(x) - p(x)| / max(p(x), u q(x))
    per tried child, and the distance of u_sample * sum from the neighbouring
    cumulative sums over the total for the bonus).  An implementation that sums
    in another order may take a different decision only where this is at the
    rounding level.
    """
    if draft_mode not in ("topw", "sampled"):
        raise OracleInputError(f"unknown draft mode {draft_mode!r}")
    X = np.asarray(target_logits)
    if draft_mode == "sampled":
        Dl = np.asarray(draft_logits)
        _check_stochastic_rows([X[:n_nodes], Dl])
    else:
        _check_stochastic_rows([X[:n_nodes]])
    if not (float(temperature) > 0.0 and np.isfinite(temperature)):
        raise OracleInputError("temperature must be positive and finite")
    u = 0
    path = []
    while True:
        p = softmax_t(X[u], temperature)
        kids = [v for v in range(1, n_nodes) if int(parent[v]) == u]
        nxt = None
        for v in kids:
            x = int(token[v])
            if draft_mode == "sampled":
                q = softmax_t(Dl[int(depth[v]) - 1], temperature)
            else:
                q = np.zeros_like(p)
                q[x] = 1.0
            lhs = float(u_accept[v]) * q[x]
            if margins is not None:
                den = max(p[x], lhs)
                margins.append(abs(lhs - p[x]) / den if den > 0.0 else 1.0)
            if lhs < p[x]:
                nxt = v
                break
            r = np.maximum(p - q, 0.0)
            if r.sum() == 0.0:
                break
            p = r / r.sum()
        if nxt is None:
            break
        path.append(nxt)
        u = nxt
    nodes = np.full(n_depth, -1, dtype=np.int64)
    nodes[:len(path)] = path
    y = sample_index(p, u_sample)
    if margins is not None:
        c = np.cumsum(p)
        t = float(u_sample) * c[-1]
        lo = c[y - 1] if y > 0 else 0.0
        margins.append(min(c[y] - t, t - lo) / c[-1])
    return len(path), nodes, y


# ---------------------------------------------------------------------------
# f4: build-mode variants (node-block expansion, entropy / mixed priority)
# ---------------------------------------------------------------------------

def draft_row_entropy(row) -> float:
    """Shannon entropy (nats, fp64) of softmax(row): -sum p log p over p > 0.

    The JetSpec explainer (techwalker.com), section 五, names the entropy of
    each position as an alternative priority.  -inf entries have p = 0.
    """
    x = np.asarray(row, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any() or not np.isfinite(x).any():
        raise OracleInputError("draft logits must be finite or -inf, one finite")
    e = np.exp(x - x.max())
    p = e / e.sum()
    nz = p > 0.0
    return float(-(p[nz] * np.log(p[nz])).sum())


def variant_key(score, ent, entropy_weight):
    """Priority of a node of cumulative score ``score`` at a depth of entropy
    ``ent``: (1 - a) * score - a * ent for a = entropy_weight in [0, 1]; a = 1
    is the pure per-position entropy priority (the score term is dropped)."""
    a = float(entropy_weight)
    if a == 1.0:
        return -ent
    return (1.0 - a) * score - a * ent


def build_tree_variant(draft_logits, width: int, budget: int, root_token: int,
                       expand: str = "candidate", entropy_weight: float = 0.0):
    """Best-first tree of one sequence under a build-mode variant.

    JetSpec explainer (techwalker.com), section 五: a priority queue of
    candidate nodes; the best is popped and given up to W children, which join
    the queue, until B nodes are placed.  The same section reports two other
    priorities, the per-position entropy and a weighted mix of cumulative
    probability and entropy.  Readings fixed here:

    * ``expand="candidate"`` (the default reading): the queue holds candidates
      (parent node, rank); a pop places one node; a placed node shallower than
      N offers its W children.  Ties: parent index, then rank.
    * ``expand="node_block"``: the queue holds placed nodes shallower than N
      (the root first); a pop attaches all of that node's W children (rank
      order, consecutive node indices), cut short when B nodes are placed.
      Ties: lower node index.
    * priority = variant_key(score, H_depth, a): score is the cumulative draft
      log-probability (as in build_tree); H_d is draft_row_entropy of depth d's
      row, the entropy of the position the node's token sits at.
    Candidates are per depth (top-W of row d, logit desc then id asc), as in
    build_tree.  Returns dict(parent, token, depth, score (-1 / -inf padded to
    B+1), n_nodes, entropy [N], margin, cross_ties): margin is the smallest
    positive gap between a pop's winner and the best entry left behind, and
    cross_ties counts pops whose winner tied with an entry of another depth.
    """
    L = np.asarray(draft_logits)
    n_depth = L.shape[0]
    a = float(entropy_weight)
    if not 0.0 <= a <= 1.0:
        raise OracleInputError("entropy_weight must lie in [0, 1]")
    if expand not in ("candidate", "node_block"):
        raise OracleInputError("expand must be 'candidate' or 'node_block'")
    if budget < 0:
        raise OracleInputError("budget must be >= 0")
    lse = np.empty(n_depth)
    ent = np.empty(n_depth)
    cand_tok = np.empty((n_depth, width), dtype=np.int64)
    cand_val = np.empty((n_depth, width))
    for d in range(n_depth):
        lse[d], cand_tok[d], cand_val[d] = draft_row_stats(L[d], width)
        ent[d] = draft_row_entropy(L[d])
    S = [0.0]
    for d in range(n_depth):
        S.append(S[-1] + float(lse[d]))

    parent, token, depth, raw, score = [-1], [int(root_token)], [0], [0.0], [0.0]
    margin, cross = np.inf, 0

    def place(p, k):
        dd = depth[p] + 1
        r = raw[p] + float(cand_val[dd - 1, k])
        parent.append(p)
        token.append(int(cand_tok[dd - 1, k]))
        depth.append(dd)
        raw.append(r)
        score.append(r - S[dd])

    def pick(keys, ties, depths):
        """Index of the best entry: key descending, then the tie key ascending."""
        nonlocal margin, cross
        kk = np.asarray(keys)
        best = kk.max()
        tied = np.flatnonzero(kk == best)
        i = int(min(tied, key=lambda t: ties[t]))
        if len(set(depths[t] for t in tied)) > 1:
            cross += 1
        rest = kk[kk < best]
        if rest.size:
            margin = min(margin, float(best - rest.max()))
        return i

    if expand == "candidate":
        f = []  # entries (parent, rank)
        if n_depth >= 1:
            f += [(0, k) for k in range(width)]
        while len(parent) - 1 < budget and f:
            keys = []
            for (p, k) in f:
                dd = depth[p] + 1
                sc = (raw[p] + float(cand_val[dd - 1, k])) - S[dd]
                keys.append(variant_key(sc, float(ent[dd - 1]), a))
            i = pick(keys, f, [depth[p] + 1 for (p, _) in f])
            p, k = f.pop(i)
            place(p, k)
            if depth[-1] < n_depth:
                v = len(parent) - 1
                f += [(v, kk) for kk in range(width)]
    else:
        q = [0] if n_depth >= 1 else []  # expandable placed nodes
        while len(parent) - 1 < budget and q:
            keys = [0.0 if v == 0 else variant_key(score[v], float(ent[depth[v] - 1]), a)
                    for v in q]
            i = pick(keys, q, [depth[v] for v in q])
            u = q.pop(i)
            for k in range(width):
                if len(parent) - 1 >= budget:
                    break
                place(u, k)
                if depth[-1] < n_depth:
                    q.append(len(parent) - 1)

    n = len(parent)
    size = budget + 1
    out = dict(parent=np.full(size, -1, dtype=np.int64), token=np.full(size, -1, dtype=np.int64),
               depth=np.full(size, -1, dtype=np.int64), score=np.full(size, -np.inf))
    out["parent"][:n] = parent
    out["token"][:n] = token
    out["depth"][:n] = depth
    out["score"][:n] = score
    out.update(n_nodes=n, entropy=ent, margin=margin, cross_ties=cross)
    return out
