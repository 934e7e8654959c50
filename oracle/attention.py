"""Tree attention, float64, with an explicit dense ancestor-only mask.

Definition followed (DARTree paper, Preliminaries > Tree Verification and
DDTree; DDTree abstract): all draft-tree nodes are scored in one target forward
in which node i attends to the whole verified context (the KV-cached prefix of
P tokens) and to the tree nodes on its root-to-node path, and to nothing else.

For one sequence, node i and query head h:

    keys    = [prefix rows 0..P-1 ; tree nodes 0..n-1]
    visible = every prefix row, and tree node j iff j in anc(i)
    s_j     = scale * <q[i, h], k_j>            (-inf where not visible)
    p       = exp(s - max s) / sum exp(s - max s)
    o[i, h] = sum_j p_j v_j

Readings where the pages say nothing (each listed in the design notes):
grouped-query attention maps query head h to KV head h // (Hq / Hkv); the
softmax scale defaults to 1 / sqrt(head_dim); positions (RoPE) are already in
the Q/K operands.

Operands are read as given (bf16-valued float32 arrays in the parity tests)
and every product, sum and exponential is taken in float64. The matrix
products use numpy's BLAS.
"""

import numpy as np

from .tree import ancestor_matrix, path_to_root


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, parent, scale=None):
    """One sequence.

    q: [n, Hq, d]; k_tree, v_tree: [n, Hkv, d]; k_prefix, v_prefix: [P, Hkv, d];
    parent: [n] int (parent[0] = -1, 0 <= parent[i] < i). Returns o [n, Hq, d] float64.
    """
    q, k_tree, v_tree = _f64(q), _f64(k_tree), _f64(v_tree)
    k_prefix = _f64(k_prefix).reshape(-1, k_tree.shape[1], k_tree.shape[2])
    v_prefix = _f64(v_prefix).reshape(-1, k_tree.shape[1], k_tree.shape[2])
    n, Hq, d = q.shape
    Hkv = k_tree.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = Hq // Hkv
    P = k_prefix.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)

    # dense mask over [prefix ; tree]: the whole prefix, plus the ancestors
    visible = np.concatenate([np.ones((n, P), dtype=bool), ancestor_matrix(parent)], axis=1)
    keys = np.concatenate([k_prefix, k_tree], axis=0)  # [P+n, Hkv, d]
    vals = np.concatenate([v_prefix, v_tree], axis=0)

    out = np.empty((n, Hq, d), dtype=np.float64)
    for h in range(Hq):
        kv = h // g
        s = scale * (q[:, h, :] @ keys[:, kv, :].T)  # [n, P+n]
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals[:, kv, :]
    return out


def tree_attention_rows(q, k_tree, v_tree, k_prefix, v_prefix, parent, rows, scale=None):
    """The same definition evaluated for selected (node, query head) pairs only.

    ``rows`` is a sequence of (i, h). Returns float64 [len(rows), d]. Used for
    sampled checks at sizes where the full dense evaluation is too slow.
    """
    Hkv, d = k_tree.shape[1], k_tree.shape[2]
    Hq = q.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((len(rows), d), dtype=np.float64)
    for r, (i, h) in enumerate(rows):
        kv = h // g
        path = path_to_root(parent, i)
        keys = np.concatenate([_f64(k_prefix[:, kv, :]), _f64(k_tree[path, kv, :])], axis=0)
        vals = np.concatenate([_f64(v_prefix[:, kv, :]), _f64(v_tree[path, kv, :])], axis=0)
        s = scale * (keys @ _f64(q[i, h, :]))
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum()
        out[r] = p @ vals
    return out


def batch_tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, parent, node_offsets,
                         prefix_lens, prefix_row_starts, scale=None):
    """Packed multi-sequence form.

    Rows of sequence s are ``node_offsets[s] .. node_offsets[s+1]-1`` of q,
    k_tree, v_tree and parent (parent indices are local to the sequence);
    its prefix is rows ``prefix_row_starts[s] .. + prefix_lens[s] - 1`` of
    k_prefix / v_prefix. Returns o [N, Hq, d] float64.
    """
    out = np.empty(q.shape, dtype=np.float64)
    for s in range(len(prefix_lens)):
        a, b = int(node_offsets[s]), int(node_offsets[s + 1])
        p0, P = int(prefix_row_starts[s]), int(prefix_lens[s])
        out[a:b] = tree_attention(q[a:b], k_tree[a:b], v_tree[a:b], k_prefix[p0:p0 + P],
                                  v_prefix[p0:p0 + P], parent[a:b], scale)
    return out


def flops(nodes, prefix_lens, parents, Hq, d):
    """Algorithmic flops of tree attention: 4 * d * Hq per visible (query node, key)
    pair (2 for q.k, 2 for p.v), counting the whole prefix and the
    ancestor-or-self tree keys only."""
    total = 0
    for n, P, parent in zip(nodes, prefix_lens, parents):
        anc_pairs = sum(len(path_to_root(parent, i)) for i in range(n))
        total += 4 * d * Hq * (n * P + anc_pairs)
    return total
