"""Committing the accepted path's keys and values to the KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

DARTree paper, Preliminaries > Speculative Sampling: every round commits the
accepted draft prefix followed by one bonus token; Figure 3 (overview) has
tree verification hand the accepted tokens and their features on to the next
round. The pages do not describe the cache itself. Reading taken here: the
verification forward has already computed the keys and values of every tree
node at position P + depth (the node's place if its path is accepted), so the
commit copies, for the accepted path root = path[0], path[1], ..., path[L], the
tree K/V rows of path[t] into cache row P + t. The root is the previous round's
last committed token, whose K/V the verification forward produced; the bonus
token's K/V do not exist yet (it is the next round's root). After the commit
the verified prefix of the sequence is P + L + 1 rows long.
"""

import numpy as np


def commit_kv(k_cache, v_cache, k_tree, v_tree, path, accept_len, node_offsets, prefix_lens, prefix_row_start):
    """One layer. k_cache/v_cache [rows, Hkv, d] are returned as updated copies;
    k_tree/v_tree [N, Hkv, d]; path [N] tree-local node indices (path[off_s + t]
    for t = 0..L_s); accept_len [S]; node_offsets [S+1]; prefix_lens and
    prefix_row_start [S]."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for s in range(len(prefix_lens)):
        off = int(node_offsets[s])
        row0 = int(prefix_row_start[s]) + int(prefix_lens[s])
        for t in range(int(accept_len[s]) + 1):
            node = off + int(path[off + t])
            kc[row0 + t] = k_tree[node]
            vc[row0 + t] = v_tree[node]
    return kc, vc
