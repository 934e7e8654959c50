"""Ancestor sets of a flattened draft tree.

DARTree paper, Preliminaries > Tree Verification and DDTree: a draft tree is a
prefix tree; for verification its nodes are flattened and a node may attend to
the verified context and to the tokens on its root-to-node path. The path of
node i is i itself, its parent, its parent's parent, ... up to the root, so
anc(i) = {i} U anc(parent[i]), with node 0 the root (parent -1).
"""

import numpy as np


def check(parent):
    """Raise ValueError unless ``parent`` describes one rooted tree numbered
    topologically: parent[0] == -1 and 0 <= parent[i] < i for i > 0."""
    parent = np.asarray(parent)
    n = len(parent)
    if n < 1:
        raise ValueError("a tree has at least its root")
    if parent[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    for i in range(1, n):
        if not (0 <= parent[i] < i):
            raise ValueError(f"parent[{i}] = {parent[i]} is not in [0, {i})")


def path_to_root(parent, i):
    """Node indices on the root-to-node path of ``i``, listed root first."""
    out = []
    j = int(i)
    while j != -1:
        out.append(j)
        j = int(parent[j])
    return out[::-1]


def ancestor_matrix(parent):
    """Dense bool [n, n]: entry (i, j) is True iff j lies on i's root-to-node
    path (j == i included)."""
    check(parent)
    n = len(parent)
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in path_to_root(parent, i):
            anc[i, j] = True
    return anc


def depths(parent):
    """Depth of every node (root = 0): the length of its path minus one."""
    return np.array([len(path_to_root(parent, i)) - 1 for i in range(len(parent))], dtype=np.int64)
