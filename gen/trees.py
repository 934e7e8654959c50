"""Random draft-tree topologies.

A tree over ``n`` nodes is an int32 ``parent`` array with ``parent[0] == -1``
(node 0 is the root: the last committed token) and ``0 <= parent[i] < i`` for
every other node, i.e. nodes are numbered in a topological order. These
generators only draw shapes; they compute nothing the verifier computes.
"""

import itertools

import numpy as np


def chain(n):
    """The single-trajectory tree: ``parent[i] = i - 1``."""
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def bfs_tree(rng, n, depth):
    """A tree of ``n`` nodes and exact depth ``depth`` numbered in BFS order.

    Every depth 1..depth holds at least one node; the remaining nodes get a
    uniformly drawn depth. A node at depth d picks its parent uniformly among
    the nodes at depth d-1. Nodes are numbered by (depth, parent).
    Returns (parent, depth_of_node).
    """
    if n < 1:
        raise ValueError("n >= 1")
    depth = min(depth, n - 1)
    d_of = [0]
    if n > 1:
        extra = rng.integers(1, depth + 1, size=n - 1 - depth) if n - 1 - depth > 0 else np.zeros(0, np.int64)
        d_of += sorted(list(range(1, depth + 1)) + [int(x) for x in extra])
    by_depth = {}
    for i, d in enumerate(d_of):
        by_depth.setdefault(d, []).append(i)
    # draw parents by depth level, then renumber by (depth, parent) so that the
    # numbering is a breadth-first order
    draft_parent = [-1] * n
    for d in range(1, depth + 1):
        prev = by_depth[d - 1]
        for i in by_depth[d]:
            draft_parent[i] = prev[int(rng.integers(0, len(prev)))]
    order = [0]
    new_id = {0: 0}
    for d in range(1, depth + 1):
        level = sorted(by_depth[d], key=lambda i: (new_id[draft_parent[i]], i))
        for i in level:
            new_id[i] = len(order)
            order.append(i)
    parent = np.empty(n, np.int32)
    dep = np.empty(n, np.int32)
    for old in order:
        j = new_id[old]
        parent[j] = -1 if old == 0 else new_id[draft_parent[old]]
        dep[j] = d_of[old]
    return parent, dep


def random_recursive(rng, n):
    """``parent[i]`` uniform on ``[0, i)``: a shallow, bushy tree (depth ~ log n)."""
    p = np.empty(n, np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(0, i)
    return p


def random_deep(rng, n, stick=0.85):
    """A deep, narrow tree: with probability ``stick`` a node extends the
    previous node, otherwise it attaches to a uniformly drawn earlier node."""
    p = np.empty(n, np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = i - 1 if rng.random() < stick else rng.integers(0, i)
    return p


def all_topological(n):
    """Every parent array of ``n`` nodes with ``0 <= parent[i] < i``:
    (n-1)! trees (1, 1, 2, 6 for n = 1..4)."""
    choices = [range(i) for i in range(1, n)]
    for tail in itertools.product(*choices):
        yield np.array((-1,) + tuple(tail), np.int32)


def children_lists(parent):
    """Children of every node in increasing index order (input-side helper for planting)."""
    ch = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        ch[int(parent[i])].append(i)
    return ch


def distinct_sibling_tokens(rng, parent, vocab):
    """Draw a token for every node such that siblings carry distinct tokens."""
    n = len(parent)
    tok = np.empty(n, np.int32)
    tok[0] = rng.integers(0, vocab)
    for kids in children_lists(parent):
        if kids:
            tok[kids] = rng.choice(vocab, size=len(kids), replace=False)
    return tok
