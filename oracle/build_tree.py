"""Best-first draft-tree construction (DDTree) and the optimum it reaches.

Objective (DARTree paper, Preliminaries > Tree Verification and DDTree, eq. 4):
choose a prefix tree T of at most B draft prefixes maximising the expected
acceptance length under the factorised drafting distribution. For a prefix
u = (u_1..u_d) its mass is the product of the per-position probabilities of
its tokens; the expectation decomposes into the sum of the masses of the
prefixes in T, and because an ancestor has at least the mass of any
descendant, the B prefixes of highest mass form an optimal tree.

Procedure (DARTree paper, Figure 3 caption; DDTree abstract): a max-heap over
frontier prefixes; each pop takes the prefix of highest mass, makes it a tree
node, and pushes that prefix's next sibling (same parent, next-ranked token at
the same depth) and its first child (highest-ranked token at the next depth).

Scores are log-masses: the sum of the candidates' log-probabilities, added in
float64 from the root down. Lemma 1 (DARTree paper, Deferred Best-First
Pruning, eq. 6; proof in Appendix C) states that when every step adds a
non-positive amount and ancestors win ties, best-first selection equals plain
top-B selection. Ties are broken by (score descending, depth ascending, rank
tuple ascending in lexicographic order); a child always sorts after its parent
and a next sibling after its elder sibling, so this total order is consistent
with the heap (a reading: the pages ask only that ancestors win ties).

Inputs: ``lp`` float [depths, k], each row sorted descending (ties by ascending
token); ``tok`` int [depths, k]; the root token; the node budget n_nodes
counting the root. Outputs: parent, token, depth, score lists of length
<= n_nodes (shorter only when fewer prefixes exist).
"""

import heapq
import itertools

import numpy as np


def build_tree_heap(lp, tok, root_token, n_nodes):
    lp = np.asarray(lp)
    tok = np.asarray(tok)
    depths, k = lp.shape
    parent, token, depth, score = [-1], [int(root_token)], [0], [0.0]
    heap = []
    if n_nodes > 1 and depths >= 1 and k >= 1:
        # entry: (-score, depth, rank tuple, parent node)
        heapq.heappush(heap, (-(0.0 + float(lp[0, 0])), 1, (0,), 0))
    while heap and len(parent) < n_nodes:
        neg, d, ranks, par = heapq.heappop(heap)
        node = len(parent)
        s = -neg
        r = ranks[-1]
        parent.append(par)
        token.append(int(tok[d - 1, r]))
        depth.append(d)
        score.append(s)
        if r + 1 < k:  # next sibling: same parent, next-ranked candidate at depth d
            heapq.heappush(heap, (-(score[par] + float(lp[d - 1, r + 1])), d, ranks[:-1] + (r + 1,), par))
        if d < depths:  # first child: best candidate at depth d + 1
            heapq.heappush(heap, (-(s + float(lp[d, 0])), d + 1, ranks + (0,), node))
    return parent, token, depth, score


def _all_prefixes(lp):
    """Every rank tuple of length 1..depths with its log-mass, accumulated from
    the root down in float64."""
    depths, k = lp.shape
    out = []
    for d in range(1, depths + 1):
        for ranks in itertools.product(range(k), repeat=d):
            s = 0.0
            for i, r in enumerate(ranks):
                s = s + float(lp[i, r])
            out.append((s, d, ranks))
    return out


def build_tree_bruteforce(lp, tok, root_token, n_nodes):
    """Enumerate every prefix, sort by (score desc, depth asc, ranks asc), keep
    the first n_nodes - 1, and number them in that order after the root."""
    lp = np.asarray(lp)
    tok = np.asarray(tok)
    allp = sorted(_all_prefixes(lp), key=lambda e: (-e[0], e[1], e[2]))[: max(0, n_nodes - 1)]
    node_of = {(): 0}
    parent, token, depth, score = [-1], [int(root_token)], [0], [0.0]
    for s, d, ranks in allp:
        node_of[ranks] = len(parent)
        parent.append(node_of[ranks[:-1]])  # KeyError here would mean a non-prefix-closed set
        token.append(int(tok[d - 1, ranks[-1]]))
        depth.append(d)
        score.append(s)
    return parent, token, depth, score


def best_total_mass(lp, n_nodes):
    """Exhaustive search over every prefix-closed set of n_nodes - 1 prefixes:
    the largest total mass sum(exp(log-mass)) (eq. 4's decomposed objective).
    Exponential; for depths <= 3 and k <= 3 only."""
    lp = np.asarray(lp)
    allp = _all_prefixes(lp)
    mass = {ranks: np.exp(s) for s, _, ranks in allp}
    best = -1.0
    for subset in itertools.combinations(mass.keys(), max(0, n_nodes - 1)):
        chosen = set(subset)
        if all(len(r) == 1 or r[:-1] in chosen for r in chosen):
            best = max(best, sum(mass[r] for r in chosen))
    return best
