"""DARTree tree construction: per-depth candidates, depth-wise fixed-width
expansion and deferred top-B pruning.

TEST INFRASTRUCTURE ONLY (see the package docstring).

DARTree paper, Methodology:
* Depth-Wise Parallel Supertree Construction and Algorithm 1: at every draft
  depth d only the drafter's top-K tokens C_d are candidate extensions; every
  retained prefix of depth d-1 is extended by every candidate, each child is
  scored by s(child) = s(parent) + log q~_d(token | parent) + beta, and the
  highest-scoring W children (over all parents) are retained as layer S_d.
  The union of the layers is the supertree S.
* Deferred Best-First Pruning, eq. 5: s_beta(u_1:d) = sum_i log q~_i(u_i) + beta d,
  and eq. 6 / Lemma 1: with beta <= 0 and ancestors preferred on ties, the
  best-first heap over S and the global top-B of S by s_beta return the same
  tree (Appendix C: a child never scores above its parent).

The correction head q~ needs trained weights; here it is an input: the
per-depth log-probabilities of every (parent, candidate) pair.

Readings (the pages do not fix them):
* Candidate log-probabilities are the log-softmax of the drafter's logits over
  the whole vocabulary, ranked by (logit desc, token index asc).
* Scores are evaluated in float32 exactly as Algorithm 1 accumulates them:
  ((s_parent + log q~) + beta), left to right. Selection compares these fp32
  values; ties go to the lower parent slot, then the lower candidate rank, so
  each layer's slots are in lexicographic (rank-tuple) order among equals.
* The verification budget B counts draft nodes; the pruned tree is the root
  plus B nodes, flattened in the order (score desc, depth asc, slot asc),
  which lists every parent before its children.
"""

import heapq

import numpy as np

F32 = np.float32


def topk_logprobs(logits, k):
    """Per row: the k largest logits ordered by (logit desc, index asc), and
    their log-softmax values (float64). Returns (tokens int64 [rows, k], logp float64 [rows, k])."""
    lg = np.asarray(logits)
    rows, vocab = lg.shape
    k = min(int(k), vocab)
    toks = np.empty((rows, k), np.int64)
    logp = np.empty((rows, k), np.float64)
    for r in range(rows):
        x = lg[r].astype(np.float64)
        order = np.lexsort((np.arange(vocab), -x))[:k]  # primary key -x (ascending), then index
        m = x.max()
        lse = m + np.log(np.sum(np.exp(x - m)))
        toks[r] = order
        logp[r] = x[order] - lse
    return toks, logp


def child_scores(parent_score, child_logq, beta):
    """s(child) = (s(parent) + log q~) + beta in float32, [w_prev, k]."""
    ps = np.asarray(parent_score, F32).reshape(-1, 1)
    lq = np.asarray(child_logq, F32)
    with np.errstate(invalid="ignore"):
        return (ps + lq) + F32(beta)


def expand_depth(parent_score, child_logq, beta, w):
    """Algorithm 1's expansion step for one sequence: score every (parent slot p,
    candidate c) child and keep the w best by (score desc, p asc, c asc).
    Parents with score -inf (absent slots) have no children. Returns
    (parent slot, candidate index, score) lists of length <= w."""
    s = child_scores(parent_score, child_logq, beta)
    wp, k = s.shape
    cands = [(-float(s[p, c]), p, c) for p in range(wp) for c in range(k) if np.isfinite(s[p, c])]
    cands.sort()
    keep = cands[:w]
    return [p for _, p, _ in keep], [c for _, _, c in keep], [F32(-ns) for ns, _, _ in keep]


def build_supertree(logq_per_depth, beta, w):
    """Algorithm 1's expansion loop for one sequence, with the head's outputs
    given: logq_per_depth[d] is a function (parent layer as a list of node ids,
    their token paths) -> float32 [len(layer), k] of log q~ for depth d + 1.
    Returns the supertree as layers: for depth d = 1.., lists of
    (parent slot in layer d-1, candidate index, score)."""
    layers = []
    prev_scores = [F32(0.0)]
    prev_paths = [()]
    for d, head in enumerate(logq_per_depth):
        lq = head(prev_paths)
        par, cand, sc = expand_depth(prev_scores, lq, beta, w)
        layers.append(list(zip(par, cand, sc)))
        prev_paths = [prev_paths[p] + (c,) for p, c in zip(par, cand)]
        prev_scores = sc
        if not par:
            break
    return layers


def flatten_nodes(layers):
    """Supertree layers -> node list [(node id, parent id, depth, slot, cand, score)],
    root = id 0 (depth 0, score 0)."""
    nodes = [(0, -1, 0, 0, -1, F32(0.0))]
    ids_prev = [0]
    for d, layer in enumerate(layers, start=1):
        ids = []
        for slot, (p, c, sc) in enumerate(layer):
            nid = len(nodes)
            nodes.append((nid, ids_prev[p], d, slot, c, F32(sc)))
            ids.append(nid)
        ids_prev = ids
    return nodes


def _order_key(node):
    nid, par, depth, slot, cand, score = node
    return (-float(score), depth, slot)


def prune_topb(layers, budget):
    """Eq. 6 right-hand side: the root plus the global top-B supertree nodes by
    (score desc, depth asc, slot asc). Returns the list of kept node ids in
    that order (root first)."""
    nodes = flatten_nodes(layers)
    rest = sorted(nodes[1:], key=_order_key)
    return [0] + [n[0] for n in rest[:budget]]


def best_first(layers, budget):
    """Eq. 6 left-hand side: a best-first max-heap over the supertree (pop the
    best frontier node, push its children), preferring ancestors on ties by
    the same (score desc, depth asc, slot asc) order. Returns kept node ids in
    pop order (root first)."""
    nodes = flatten_nodes(layers)
    children = {}
    for n in nodes[1:]:
        children.setdefault(n[1], []).append(n)
    out = [0]
    heap = [(_order_key(c), c[0]) for c in children.get(0, [])]
    heapq.heapify(heap)
    while heap and len(out) < budget + 1:
        _, nid = heapq.heappop(heap)
        out.append(nid)
        for c in children.get(nid, []):
            heapq.heappush(heap, (_order_key(c), c[0]))
    return out


def tree_arrays(layers, kept, cand_tokens):
    """The kept nodes as a verification tree in the given order: (parent,
    token, depth, score) arrays, parent indices into the kept order.
    cand_tokens[d-1][c] is the token of candidate c at depth d; the root's
    token is -1 (the caller's last committed token)."""
    nodes = flatten_nodes(layers)
    pos = {nid: i for i, nid in enumerate(kept)}
    parent, token, depth, score = [], [], [], []
    for nid in kept:
        _, par, d, _, c, sc = nodes[nid]
        parent.append(pos[par] if par >= 0 else -1)
        token.append(int(cand_tokens[d - 1][c]) if d > 0 else -1)
        depth.append(d)
        score.append(F32(sc))
    return np.array(parent), np.array(token), np.array(depth), np.array(score, F32)
