"""Greedy acceptance of the longest matching root-to-leaf path.

DARTree paper, Preliminaries > Speculative Sampling (T = 0): verification
accepts consecutive draft tokens while each equals the target's greedy
prediction; at the first mismatch the target's prediction is emitted and the
round ends. Every round commits the accepted prefix plus that one extra target
token (the bonus token); tau (Experimental Setup) counts it, so tau = L + 1.
Preliminaries > Tree Verification and DDTree: after the single forward, the
accepted root-to-leaf prefix is selected according to the target model.

On a tree the draft token at the next position is not unique: from node u the
walk moves to the child whose token equals argmax[u]. Siblings carry distinct
tokens in a prefix tree; for a caller-built tree with duplicate sibling tokens
the lowest-index matching child is taken (a reading).
"""


def accept_path(parent, token, argmax):
    """Return (path, L, bonus) for one tree.

    path: node indices from the root (node 0) to the last accepted node;
    L = len(path) - 1 accepted draft tokens; bonus = argmax[last accepted node].
    """
    n = len(parent)
    cur = 0
    path = [0]
    while True:
        want = int(argmax[cur])
        matches = [c for c in range(n) if int(parent[c]) == cur and int(token[c]) == want]
        if not matches:
            break
        cur = min(matches)
        path.append(cur)
    return path, len(path) - 1, int(argmax[cur])


def batch_accept_path(parent, token, argmax, node_offsets):
    """Packed multi-sequence form: per sequence (path, L, bonus), node indices local."""
    out = []
    for s in range(len(node_offsets) - 1):
        a, b = int(node_offsets[s]), int(node_offsets[s + 1])
        out.append(accept_path(parent[a:b], token[a:b], argmax[a:b]))
    return out
