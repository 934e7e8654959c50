"""Pins for the KV-commit oracle (CPU only).

* The committed cache is the accepted path's context: for the last accepted
  node u, tree attention of u (the attention oracle, itself pinned) equals plain
  causal attention of u's query over the committed cache rows 0 .. P + L.
* Row P + t holds the depth-t ancestor of u (positions follow depth, as the
  verification forward placed them), and every other row is untouched.
* Closed forms: a fully accepted chain lands as tree rows 0 .. n-1 in order; an
  immediate mismatch commits the root alone.
* Planted mistakes (off-by-one row, reversed path, bonus row appended) fail.
"""

import numpy as np
import pytest

from gen import rng as grng, tensors as gten, trees as gtrees
from oracle import argmax as oarg, attention as oatt, commit as ocommit, tree as otree, walk as owalk


def _case(seed, n, P, Hq=4, Hkv=2, d=16, vocab=40, gap=3):
    r = grng.stream(seed, "commit")
    parent = [gtrees.random_recursive, gtrees.random_deep][seed % 2](r, n)
    token = gtrees.distinct_sibling_tokens(r, parent, vocab)
    lg = gten.logits(r, n, vocab)
    gten.plant(r, lg, parent, token, p=0.9, pick="random")
    path, L, _ = owalk.accept_path(parent, token, oarg.argmax_rows(lg))
    ops = gten.attention_operands(r, n, P, Hq, Hkv, d)
    # cache with room: gap rows before the prefix start, capacity P + n + gap after it
    cache_rows = gap + P + n + gap
    kc = r.standard_normal((cache_rows, Hkv, d))
    vc = r.standard_normal((cache_rows, Hkv, d))
    kc[gap:gap + P] = ops["k_prefix"]
    vc[gap:gap + P] = ops["v_prefix"]
    full_path = np.full(n, -1, np.int64)
    full_path[:L + 1] = path
    return parent, path, L, ops, kc, vc, full_path, gap


@pytest.mark.parametrize("seed", range(10))
def test_committed_cache_is_the_accepted_context(seed):
    n, P = [1, 7, 30, 60][seed % 4], [0, 5, 33][seed % 3]
    parent, path, L, ops, kc, vc, full_path, gap = _case(seed, n, P)
    kc2, vc2 = ocommit.commit_kv(kc, vc, ops["k_tree"], ops["v_tree"], full_path, [L], [0, n], [P], [gap])
    u = path[-1]
    Hq, d = ops["q"].shape[1], ops["q"].shape[2]
    g = Hq // ops["k_tree"].shape[1]
    tree_out = oatt.tree_attention_rows(ops["q"], ops["k_tree"], ops["v_tree"], ops["k_prefix"], ops["v_prefix"],
                                        parent, [(u, h) for h in range(Hq)])
    ctx = slice(gap, gap + P + L + 1)
    for h in range(Hq):
        s = kc2[ctx, h // g, :] @ ops["q"][u, h].astype(np.float64) / np.sqrt(d)
        p = np.exp(s - s.max())
        causal = (p / p.sum()) @ vc2[ctx, h // g, :]
        np.testing.assert_allclose(causal, tree_out[h], rtol=0, atol=1e-12)
    # position order: row P + t is u's depth-t ancestor; nothing else changed
    anc = otree.path_to_root(parent, u)
    assert len(anc) == L + 1
    for t, node in enumerate(anc):
        np.testing.assert_array_equal(kc2[gap + P + t], ops["k_tree"][node])
        np.testing.assert_array_equal(vc2[gap + P + t], ops["v_tree"][node])
    keep = np.ones(kc.shape[0], bool)
    keep[gap + P:gap + P + L + 1] = False
    np.testing.assert_array_equal(kc2[keep], kc[keep])
    np.testing.assert_array_equal(vc2[keep], vc[keep])


def test_closed_forms():
    n, P, Hkv, d = 6, 3, 1, 4
    kt = np.arange(n * d, dtype=np.float64).reshape(n, Hkv, d)
    vt = -kt
    kc = np.zeros((P + n + 2, Hkv, d))
    vc = np.zeros_like(kc)
    chain_path = np.arange(n)
    kc2, vc2 = ocommit.commit_kv(kc, vc, kt, vt, chain_path, [n - 1], [0, n], [P], [0])
    np.testing.assert_array_equal(kc2[P:P + n], kt)
    np.testing.assert_array_equal(vc2[P:P + n], vt)
    assert not kc2[:P].any() and not kc2[P + n:].any()
    root_only = np.array([0, -1, -1, -1, -1, -1])
    kc3, _ = ocommit.commit_kv(kc, vc, kt, vt, root_only, [0], [0, n], [P], [0])
    np.testing.assert_array_equal(kc3[P], kt[0])
    assert not np.delete(kc3, P, axis=0).any()


def test_batch_equals_per_sequence():
    r = grng.stream(4, "commit-batch")
    Hkv, d = 2, 8
    nodes, plens, starts = [5, 1, 9], [4, 0, 7], [0, 20, 30]
    offs = np.concatenate([[0], np.cumsum(nodes)])
    kt = r.standard_normal((offs[-1], Hkv, d))
    vt = r.standard_normal((offs[-1], Hkv, d))
    kc = r.standard_normal((50, Hkv, d))
    vc = r.standard_normal((50, Hkv, d))
    path = np.full(offs[-1], -1)
    Ls = []
    for s, n in enumerate(nodes):
        parent = gtrees.random_deep(r, n)
        u = int(r.integers(0, n))
        p = otree.path_to_root(parent, u)
        path[offs[s]:offs[s] + len(p)] = p
        Ls.append(len(p) - 1)
    kb, vb = ocommit.commit_kv(kc, vc, kt, vt, path, Ls, offs, plens, starts)
    ks, vs = kc, vc
    for s in range(3):
        a, b = offs[s], offs[s + 1]
        ks, vs = ocommit.commit_kv(ks, vs, kt[a:b], vt[a:b], path[a:b], [Ls[s]], [0, b - a], [plens[s]], [starts[s]])
    np.testing.assert_array_equal(kb, ks)
    np.testing.assert_array_equal(vb, vs)


@pytest.mark.parametrize("kind", ["row-off-by-one", "reversed", "bonus-row"])
def test_planted_commit_mistakes_are_caught(kind):
    caught = False
    for seed in range(12):
        n, P = 40, 9
        parent, path, L, ops, kc, vc, full_path, gap = _case(seed + 100, n, P)
        if L < 2:
            continue
        kc2, vc2 = np.array(kc), np.array(vc)
        rows = list(range(gap + P, gap + P + L + 1))
        nodes = list(path)
        if kind == "row-off-by-one":
            rows = [x + 1 for x in rows]
        elif kind == "reversed":
            nodes = nodes[::-1]
        else:
            rows.append(rows[-1] + 1)
            nodes.append(nodes[-1])
        for row, node in zip(rows, nodes):
            kc2[row] = ops["k_tree"][node]
            vc2[row] = ops["v_tree"][node]
        want_k, _ = ocommit.commit_kv(kc, vc, ops["k_tree"], ops["v_tree"], full_path, [L], [0, n], [P], [gap])
        anc = otree.path_to_root(parent, path[-1])
        ordered = all(np.array_equal(kc2[gap + P + t], ops["k_tree"][a]) for t, a in enumerate(anc))
        keep = np.ones(kc.shape[0], bool)
        keep[gap + P:gap + P + L + 1] = False
        untouched = np.array_equal(kc2[keep], kc[keep])
        assert not (np.array_equal(kc2, want_k))
        if not (ordered and untouched):
            caught = True
            break
    assert caught
