"""Plain fp64 CPU oracle for MInference dynamic sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's compute
path never calls it, and it shares no code, constant or table with the HIP
sources or their Python binding.

It restates, slowly and in float64, what the method computes.  Sources, by
page (titles as printed on each page):

* [ABS]  arXiv 2407.02490 abstract, "MInference 1.0: Accelerating Pre-filling
         for Long-Context LLMs via Dynamic Sparse Attention": three per-head
         patterns (A-shape, Vertical-Slash, Block-Sparse), the pattern chosen
         offline per head, sparse indices built online per input.
* [SUM]  hotpaper.ai summary of the same paper, "key idea" section: Block-Sparse
         heads mean-pool in 64-token blocks to get block-level attention
         weights; Vertical-Slash heads use the last ``last_q`` queries against
         the keys to find the globally important indices.
* [GUIDE] aifetchly "MInference 1.0 Guide: Dynamic Sparse Attention for 1M
         Context": section "The Three Topological Attention Patterns" (sinks +
         local band; vertical lines and slash lines at fixed offsets i-j;
         coarse 64x64 tiles), section "2. The Block-Sparse Kernel Mechanics"
         (mean key of a 64-token block, query-block dot products, top-k key
         blocks, skipped tiles), section "1. The Vertical-Slash Kernel
         Mechanics" (online softmax with running max and normaliser).
* [REVIEW] hysenlabs review of the MInference repository, section "How
         MInference differs from xAttention, FlexPrefill and
         RetrievalAttention": xAttention scores blocks by antidiagonal sums.

Where the pages leave a step open the oracle takes one reading and the
function says "reading:".  Every reading is listed with its justification in
the design notes.

Conventions.  One (batch, head) slice at a time: q [N, d], k [N, d], v [N, d]
float64.  ``scale`` is the softmax scale (1/sqrt(d) unless stated).  Token
positions i (query) and j (key) run over [0, N).  A "block" is 64
consecutive tokens (parameter ``block``; tests use other sizes to reach
brute-force cases).  Query block a holds rows [block*a, block*(a+1)).
"""
from __future__ import annotations

import numpy as np

ASHAPE, VSLASH, BSPARSE, DENSE, VSLASH_EXACT = 0, 1, 2, 3, 4


# ----------------------------------------------------------------------------
# Attention given an allowed-key set per query (the definition every pattern
# reduces to): o_i = sum_{j in A(i)} softmax_j(scale q_i.k_j) v_j.
# ----------------------------------------------------------------------------

def dense_causal_attention(q, k, v, scale):
    """Dense causal attention, the quantity the sparse patterns approximate
    ([ABS]; [GUIDE] "The Prefill Phase" formula).  Returns (o [N,d], lse [N]).

    Builds the full N x N score matrix; for small N only.
    """
    n = q.shape[0]
    s = scale * (q @ k.T)
    s[np.triu_indices(n, 1)] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (m + np.log(l))[:, 0]


def attention_row_gather(q, k, v, scale, i, keys):
    """One query row attending to an explicit key list (softmax over that list).

    The per-row form of masked attention: gather the keys, score them, softmax,
    weight the values.  Returns (o_i [d], lse_i).
    """
    keys = np.asarray(keys, dtype=np.int64)
    s = scale * (k[keys] @ q[i])
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e @ v[keys]) / l, m + np.log(l)


def masked_rows_attention(q, k, v, scale, rows, cand, mask):
    """Masked attention for a group of query rows over a shared candidate list.

    rows [R] query positions, cand [C] key positions, mask [R, C] bool: row r
    attends to cand[c] iff mask[r, c].  Scores of excluded keys are -inf, so
    they get exactly zero weight.  Returns (o [R, d], lse [R]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    cand = np.asarray(cand, dtype=np.int64)
    s = scale * (q[rows] @ k[cand].T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v[cand]) / l, (m + np.log(l))[:, 0]


def union_attention(q, k, v, scale, rows, union_keys):
    """Attention where A(i) = U ∩ [0, i] for a key set U shared by the rows.

    This is how the tile/column index defines each query row's keys: a query
    block a attends to the union U(a) of its listed key blocks and its listed
    columns, restricted causally to keys j <= i.
    """
    cand = np.unique(np.asarray(union_keys, dtype=np.int64))
    rows = np.asarray(rows, dtype=np.int64)
    mask = cand[None, :] <= rows[:, None]
    return masked_rows_attention(q, k, v, scale, rows, cand, mask)


# ----------------------------------------------------------------------------
# Selection
# ----------------------------------------------------------------------------

def select_topk(score, k, forced=()):
    """F ∪ top-(k - |F|) of the remaining candidates, as an ascending list.

    Candidates are 0..M-1.  The remaining ones are ranked by score, larger
    first; reading: equal scores rank the lower index first.  k is clamped
    to M.  |F| <= k is required.  ([GUIDE] "top-k relevant key blocks";
    [SUM]: sink and diagonal are kept.)
    """
    score = np.asarray(score)
    m = score.shape[0]
    k = min(int(k), m)
    forced = sorted(set(int(f) for f in forced))
    if len(forced) > k:
        raise ValueError("more forced members than the budget")
    chosen = list(forced)
    need = k - len(forced)
    if need > 0:
        is_forced = np.zeros(m, bool)
        is_forced[forced] = True
        idx = np.arange(m)
        # lexsort: last key is primary -> by score descending, then index ascending
        order = np.lexsort((idx, -score))
        rest = order[~is_forced[order]]
        chosen.extend(int(x) for x in rest[:need])
    return np.array(sorted(chosen), dtype=np.int64)


# ----------------------------------------------------------------------------
# Vertical-Slash: estimate from the last last_q queries ([SUM] key idea)
# ----------------------------------------------------------------------------

def vs_estimate(q, k, scale, last_q):
    """Vertical and slash scores of one head.

    The last L = last_q queries, rows i_r = N - L + r, attend causally to all
    keys (reading: the softmax of row r runs over j <= i_r, so only the
    trailing L x L square is masked).  With P the L x N probability matrix:
        vertical[j] = sum_r P[r, j]           (column mass of key j)
        slash[o]    = sum_r P[r, i_r - o]     (mass on the diagonal at offset
                                               o = i - j, terms with i_r-o < 0
                                               omitted)
    Reading: scores are sums of probabilities (a mean ranks the same).
    Returns (vertical [N], slash [N]) float64.
    """
    n = k.shape[0]
    L = int(last_q)
    rows = np.arange(n - L, n)
    s = scale * (q[rows] @ k.T)
    s = np.where(np.arange(n)[None, :] <= rows[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    vertical = p.sum(axis=0)
    slash = np.zeros(n)
    for r, i in enumerate(rows):
        # offsets o = i - j for j = i, i-1, ..., 0  ->  o = 0, 1, ..., i
        slash[: i + 1] += p[r, i::-1]
    return vertical, slash


def vs_select(vertical, slash, n_vertical, n_slash, force_vertical=1, force_slash=1):
    """Vertical list V and slash list S (ascending).  Reading: the first
    ``force_vertical`` keys (the sink) and the first ``force_slash`` offsets
    (the main diagonal) are always kept and count inside the budgets."""
    V = select_topk(vertical, n_vertical, range(force_vertical))
    S = select_topk(slash, n_slash, range(force_slash))
    return V, S


def vs_block_list(a, S, block=64):
    """Key blocks query block a must compute for slash offsets S (brute force).

    Reading: each slash line is computed as whole aligned block x block tiles;
    a tile belongs to query block a when some row i of a has its diagonal
    key j = i - o (j >= 0) inside it.  Returns an ascending array.
    """
    rows = np.arange(block * a, block * (a + 1))
    S = np.asarray(S, dtype=np.int64)
    j = rows[:, None] - S[None, :]
    j = j[j >= 0]
    return np.unique(j // block)


def vs_column_list(a, V, blocks, block=64):
    """Vertical keys query block a reads as gathered columns: verticals that
    are causal for some row of a (j <= block*a + block - 1) and whose key
    block is not already a listed tile (reading: no key is counted twice)."""
    V = np.asarray(V, dtype=np.int64)
    V = V[V <= block * a + block - 1]
    return V[~np.isin(V // block, blocks)]


def vs_exact_allowed(i, V, S):
    """The per-element Vertical-Slash key set of row i ([GUIDE] "The
    Vertical-Slash Pattern"): vertical keys j in V and diagonal keys i - o for
    o in S, restricted to 0 <= j <= i.  Not the tile-level parity target; the
    tile index must contain it."""
    V = np.asarray(V, dtype=np.int64)
    S = np.asarray(S, dtype=np.int64)
    return np.union1d(V[V <= i], i - S[S <= i])


def vs_exact_attention(q, k, v, scale, rows, V, S):
    """Attention of query rows over their exact Vertical-Slash key sets
    ([GUIDE] "The Vertical-Slash Pattern"): row i attends to
    A(i) = {j in V : j <= i} u {i - o : o in S, o <= i}, each key once.

    This is the per-element pattern itself, not its tile covering: the
    element-masked variant of the sparse kernel is compared with it.
    Returns (o [R, d], lse [R])."""
    rows = np.asarray(rows, dtype=np.int64)
    V = np.unique(np.asarray(V, dtype=np.int64))
    S = np.unique(np.asarray(S, dtype=np.int64))
    hi = int(rows.max())
    diag = (rows[:, None] - S[None, :]).reshape(-1)
    cand = np.union1d(V[V <= hi], diag[diag >= 0])
    i = rows[:, None]
    causal = cand[None, :] <= i
    mask = causal & (np.isin(cand, V)[None, :] | np.isin(i - cand[None, :], S))
    return masked_rows_attention(q, k, v, scale, rows, cand, mask)


# ----------------------------------------------------------------------------
# Block-Sparse: mean pooling per 64-token block ([SUM]; [GUIDE] 2.)
# ----------------------------------------------------------------------------

def block_means(x, block=64):
    n, d = x.shape
    return x.reshape(n // block, block, d).mean(axis=1)


def bs_estimate(q, k, scale, top_blocks, block=64):
    """Block-level attention weights and kept key blocks of one head.

    Qbar_a, Kbar_c = means of the query/key rows of blocks a, c (reading: both
    queries and keys are pooled).  z[a, c] = scale * Qbar_a . Kbar_c for
    c <= a; w[a, :a+1] = softmax(z[a, :a+1]), w[a, c] = 0 for c > a.
    KB(a) = {0, a} ∪ top-(min(top, a+1) - |{0, a}|) of the other causal blocks
    by w (reading: first and diagonal block forced, inside the budget).
    Returns (w [nb, nb], list of ascending arrays KB(a)).
    """
    qb = block_means(q, block)
    kb = block_means(k, block)
    nb = qb.shape[0]
    z = scale * (qb @ kb.T)
    w = np.zeros((nb, nb))
    kept = []
    for a in range(nb):
        za = z[a, : a + 1]
        e = np.exp(za - za.max())
        w[a, : a + 1] = e / e.sum()
        kept.append(select_topk(w[a, : a + 1], min(top_blocks, a + 1), {0, a}))
    return w, kept


# ----------------------------------------------------------------------------
# Antidiagonal block scoring ([REVIEW] "How MInference differs from
# xAttention, FlexPrefill and RetrievalAttention": xAttention keeps the blocks
# whose antidiagonal sums score highest)
# ----------------------------------------------------------------------------

def antidiag_estimate(q, k, scale, top_blocks, block=64):
    """Block weights and kept key blocks of one head from antidiagonal sums.

    Reading: the score of (query block a, key block c) is the sum of the
    scaled logits along the block's main antidiagonal,
        x[a, c] = scale * sum_r q[block*a + r] . k[block*c + block-1-r],
    each query row and each key row of the pair entering once; for the
    diagonal block c = a only its causal half (block-1-r <= r) is summed.
    Then, as for the pooled estimate: w[a, :a+1] = softmax(x[a, :a+1]),
    w[a, c] = 0 for c > a, and KB(a) = {0, a} plus the highest-weight other
    causal blocks, min(top, a+1) in total.
    Returns (w [nb, nb], list of ascending arrays KB(a)).
    """
    n, d = q.shape
    nb = n // block
    qb = q[: nb * block].reshape(nb, block, d)
    kb = k[: nb * block].reshape(nb, block, d)[:, ::-1, :]  # row r of block c = key block*c + block-1-r
    # x[a, c] = scale * sum_r qb[a, r] . kb[c, r]: a matrix product over the
    # block's rows laid end to end
    x = scale * (qb.reshape(nb, block * d) @ kb.reshape(nb, block * d).T)
    r = np.arange(block)
    causal_half = (block - 1 - r) <= r
    xdiag = scale * (qb[:, causal_half] * kb[:, causal_half]).sum(axis=(1, 2))
    w = np.zeros((nb, nb))
    kept = []
    for a in range(nb):
        xa = x[a, : a + 1].copy()
        xa[a] = xdiag[a]
        e = np.exp(xa - xa.max())
        w[a, : a + 1] = e / e.sum()
        kept.append(select_topk(w[a, : a + 1], min(top_blocks, a + 1), {0, a}))
    return w, kept


# ----------------------------------------------------------------------------
# A-shape: sink tokens plus a local causal window ([GUIDE] 1. A-Shape Pattern)
# ----------------------------------------------------------------------------

def ashape_allowed(i, sink, local):
    """A(i) = {j <= i : j < sink or i - j < local} (reading: token-exact
    edges, the window holds ``local`` keys including i itself)."""
    j = np.arange(i + 1)
    return j[(j < sink) | (i - j < local)]


def ashape_block_list(a, sink, local, n, block=64):
    """Key blocks touched by some row of query block a (brute force)."""
    touched = set()
    for i in range(block * a, min(block * (a + 1), n)):
        touched.update(int(x) for x in np.unique(ashape_allowed(i, sink, local) // block))
    return np.array(sorted(touched), dtype=np.int64)


def ashape_attention(q, k, v, scale, rows, sink, local):
    rows = np.asarray(rows, dtype=np.int64)
    hi = int(rows.max())
    cand = ashape_allowed(hi, sink, local + (hi - int(rows.min())))
    i = rows[:, None]
    mask = (cand[None, :] <= i) & ((cand[None, :] < sink) | (i - cand[None, :] < local))
    return masked_rows_attention(q, k, v, scale, rows, cand, mask)


# ----------------------------------------------------------------------------
# Tile/column index -> per-block key union, and per-head dispatch
# ----------------------------------------------------------------------------

def block_union(blocks, cols, block=64):
    """Key set U(a) of a query block from its tile list and column list."""
    blocks = np.asarray(blocks, dtype=np.int64)
    tiles = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return np.union1d(tiles, np.asarray(cols, dtype=np.int64))


def attention_from_index(q, k, v, scale, a, blocks, cols, block=64):
    """Output rows of query block a for a tile list and a column list:
    A(i) = {j <= i : j in U(a)}."""
    rows = np.arange(block * a, block * (a + 1))
    return union_attention(q, k, v, scale, rows, block_union(blocks, cols, block))


class HeadIndex:
    """The oracle's own per-head index, built from its own estimates."""

    def __init__(self, pattern, n, block=64, V=None, S=None, kept=None, sink=0, local=0):
        self.pattern, self.n, self.block = pattern, n, block
        self.V, self.S, self.kept, self.sink, self.local = V, S, kept, sink, local

    def blocks(self, a):
        if self.pattern in (VSLASH, VSLASH_EXACT):
            return vs_block_list(a, self.S, self.block)
        if self.pattern == BSPARSE:
            return self.kept[a]
        if self.pattern == ASHAPE:
            return ashape_block_list(a, self.sink, self.local, self.n, self.block)
        return np.arange(a + 1)

    def cols(self, a):
        if self.pattern in (VSLASH, VSLASH_EXACT):
            return vs_column_list(a, self.V, self.blocks(a), self.block)
        return np.zeros(0, np.int64)


def head_attention(q, k, v, scale, idx: HeadIndex, blocks_a):
    """Output of one head on query blocks ``blocks_a`` per its pattern.
    Returns dict a -> (o [block, d], lse [block])."""
    out = {}
    bsz = idx.block
    for a in blocks_a:
        rows = np.arange(bsz * a, bsz * (a + 1))
        if idx.pattern == ASHAPE:
            out[a] = ashape_attention(q, k, v, scale, rows, idx.sink, idx.local)
        elif idx.pattern == DENSE:
            out[a] = union_attention(q, k, v, scale, rows, np.arange(rows[-1] + 1))
        elif idx.pattern == VSLASH_EXACT:
            out[a] = vs_exact_attention(q, k, v, scale, rows, idx.V, idx.S)
        else:
            out[a] = attention_from_index(q, k, v, scale, a, idx.blocks(a), idx.cols(a), bsz)
    return out


def build_head_index(pattern, q, k, scale, *, last_q=64, n_vertical=1000, n_slash=6096,
                     force_vertical=1, force_slash=1, top_blocks=100, sink=128, local=4096,
                     block=64):
    """Online index of one head from its own fp64 estimates.
    Returns (HeadIndex, scores dict)."""
    n = k.shape[0]
    if pattern in (VSLASH, VSLASH_EXACT):
        vert, sl = vs_estimate(q, k, scale, last_q)
        V, S = vs_select(vert, sl, n_vertical, n_slash, force_vertical, force_slash)
        return HeadIndex(pattern, n, block, V=V, S=S), dict(vertical=vert, slash=sl)
    if pattern == BSPARSE:
        w, kept = bs_estimate(q, k, scale, top_blocks, block)
        return HeadIndex(BSPARSE, n, block, kept=kept), dict(w=w)
    if pattern == ASHAPE:
        return HeadIndex(ASHAPE, n, block, sink=sink, local=local), {}
    return HeadIndex(DENSE, n, block), {}


def layer_attention(q, k, v, scale, indices, blocks_a):
    """All query heads of one layer: q [Hq, N, d], k, v [Hkv, N, d].

    Query head h reads key/value head h // (Hq / Hkv) (grouped-query
    attention); ``indices[h]`` is head h's HeadIndex.  Returns a list over
    heads of dict a -> (o, lse) for the query blocks in ``blocks_a``.
    """
    hq, hkv = q.shape[0], k.shape[0]
    g = hq // hkv
    return [head_attention(q[h], k[h // g], v[h // g], scale, indices[h], blocks_a)
            for h in range(hq)]
