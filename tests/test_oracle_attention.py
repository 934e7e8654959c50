"""Pins for the attention oracle (CPU only).

Each check ties ``oracle.attention`` to something other than itself:

* chain == causal: a chain tree (parent[i] = i-1) verifies a single drafted
  trajectory (DDTree abstract), whose target forward is ordinary causal
  attention; compared with torch's scaled_dot_product_attention (is_causal,
  enable_gqa, float64) over [prefix ; chain], last n rows.
* path-as-sequence: node i's output is plain (unmasked) attention of its query
  over [prefix ; tokens on its root-to-node path] (DARTree paper, Tree
  Verification and DDTree); computed with torch SDPA on the gathered keys.
* every tree of 1..4 nodes, non-ancestor perturbation invariance, relabelling,
  uniform keys (closed form: mean of the visible values), hand-worked fixture.
* planted mistakes in copies of the oracle are caught by these pins.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from gen import rng as grng, trees as gtrees
from oracle import attention as oatt, tree as otree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _operands(seed, n, P, Hq, Hkv, d, scale=1.0):
    r = grng.stream(seed, "oracle-att")
    f = lambda *s: r.standard_normal(s) * scale  # noqa: E731
    return f(n, Hq, d), f(n, Hkv, d), f(n, Hkv, d), f(P, Hkv, d), f(P, Hkv, d)


def _sdpa(q, k, v, causal=False):
    """q [Lq, Hq, d], k/v [Lk, Hkv, d] -> [Lq, Hq, d] via torch SDPA (float64, GQA)."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


def _path_as_sequence(q, kt, vt, kp, vp, parent):
    n, Hq, d = q.shape
    out = np.empty_like(q)
    for i in range(n):
        path = otree.path_to_root(parent, i)
        keys = np.concatenate([kp, kt[path]], axis=0)
        vals = np.concatenate([vp, vt[path]], axis=0)
        out[i] = _sdpa(q[i:i + 1], keys, vals)[0]
    return out


@pytest.mark.parametrize("n,P,Hq,Hkv,d", [(16, 128, 1, 1, 64), (9, 33, 4, 2, 16), (5, 0, 2, 1, 8), (12, 7, 8, 2, 32)])
def test_chain_equals_causal(n, P, Hq, Hkv, d):
    q, kt, vt, kp, vp = _operands(11 + n, n, P, Hq, Hkv, d)
    parent = gtrees.chain(n)
    got = oatt.tree_attention(q, kt, vt, kp, vp, parent)
    # a full causal pass over [prefix ; chain]; the prefix rows get throwaway queries
    extra_q = grng.stream(99, n, P).standard_normal((P, Hq, d))
    ref = _sdpa(np.concatenate([extra_q, q]), np.concatenate([kp, kt]), np.concatenate([vp, vt]), causal=True)[P:]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", ["bfs", "recursive", "deep"])
@pytest.mark.parametrize("P", [0, 1, 40])
def test_path_as_sequence(shape, P):
    n, Hq, Hkv, d = 24, 4, 2, 16
    r = grng.stream(7, shape, P)
    parent = {"bfs": lambda: gtrees.bfs_tree(r, n, 5)[0], "recursive": lambda: gtrees.random_recursive(r, n),
              "deep": lambda: gtrees.random_deep(r, n)}[shape]()
    q, kt, vt, kp, vp = _operands(3, n, P, Hq, Hkv, d, scale=0.7)
    got = oatt.tree_attention(q, kt, vt, kp, vp, parent)
    ref = _path_as_sequence(q, kt, vt, kp, vp, parent)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_every_tree_up_to_four_nodes():
    count = 0
    for n in range(1, 5):
        for parent in gtrees.all_topological(n):
            q, kt, vt, kp, vp = _operands(100 + count, n, 3, 2, 1, 8, scale=1.5)
            got = oatt.tree_attention(q, kt, vt, kp, vp, parent)
            ref = _path_as_sequence(q, kt, vt, kp, vp, parent)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
            count += 1
    assert count == 1 + 1 + 2 + 6


def test_non_ancestor_perturbation_is_invisible():
    n, P, Hq, Hkv, d = 20, 10, 4, 2, 16
    r = grng.stream(21)
    parent = gtrees.random_recursive(r, n)
    q, kt, vt, kp, vp = _operands(5, n, P, Hq, Hkv, d)
    base = oatt.tree_attention(q, kt, vt, kp, vp, parent)
    anc = otree.ancestor_matrix(parent)
    for i in range(n):
        others = ~anc[i]
        if not others.any():
            continue
        kt2, vt2 = kt.copy(), vt.copy()
        sign = np.where(r.random(others.sum()) < 0.5, -1.0, 1.0)[:, None, None]
        kt2[others] += 1e3 * sign
        vt2[others] -= 1e3 * sign
        got = oatt.tree_attention(q, kt2, vt2, kp, vp, parent)
        assert np.array_equal(got[i], base[i])
        # and the perturbation is visible to some node that does see those keys
        seen = anc[:, others].any(axis=1)
        assert not np.allclose(got[seen], base[seen])


def test_relabelling_permutes_outputs():
    n, P, Hq, Hkv, d = 15, 6, 2, 2, 8
    r = grng.stream(31)
    parent = gtrees.random_recursive(r, n)
    q, kt, vt, kp, vp = _operands(6, n, P, Hq, Hkv, d)
    base = oatt.tree_attention(q, kt, vt, kp, vp, parent)
    # a random topological renumbering: repeatedly pick any node whose parent is placed
    placed, order = {0}, [0]
    while len(order) < n:
        ready = [i for i in range(n) if i not in placed and parent[i] in placed]
        i = ready[int(r.integers(0, len(ready)))]
        placed.add(i)
        order.append(i)
    new_of = {old: new for new, old in enumerate(order)}
    parent2 = np.array([-1 if old == 0 else new_of[int(parent[old])] for old in order], np.int32)
    got = oatt.tree_attention(q[order], kt[order], vt[order], kp, vp, parent2)
    np.testing.assert_allclose(got, base[order], rtol=1e-13, atol=1e-13)


def test_uniform_keys_give_mean_of_visible_values():
    n, P, Hq, Hkv, d = 12, 5, 2, 1, 8
    r = grng.stream(41)
    parent = gtrees.random_deep(r, n)
    q, kt, vt, kp, vp = _operands(8, n, P, Hq, Hkv, d)
    kt[:] = kt[0]
    kp[:] = kt[0]
    got = oatt.tree_attention(q, kt, vt, kp, vp, parent)
    for i in range(n):
        path = otree.path_to_root(parent, i)
        mean = np.concatenate([vp, vt[path]]).mean(axis=0)  # [Hkv, d]
        for h in range(Hq):
            np.testing.assert_allclose(got[i, h], mean[h * Hkv // Hq], rtol=1e-12, atol=1e-13)


def test_empty_prefix_root_sees_only_itself():
    q, kt, vt, kp, vp = _operands(9, 4, 0, 2, 2, 8)
    got = oatt.tree_attention(q, kt, vt, kp, vp, np.array([-1, 0, 0, 1]))
    np.testing.assert_array_equal(got[0], vt[0])


def test_rows_variant_matches_dense():
    n, P, Hq, Hkv, d = 30, 50, 8, 2, 16
    r = grng.stream(51)
    parent = gtrees.bfs_tree(r, n, 6)[0]
    q, kt, vt, kp, vp = _operands(10, n, P, Hq, Hkv, d)
    dense = oatt.tree_attention(q, kt, vt, kp, vp, parent)
    rows = [(int(r.integers(0, n)), int(r.integers(0, Hq))) for _ in range(40)]
    got = oatt.tree_attention_rows(q, kt, vt, kp, vp, parent, rows)
    for (i, h), o in zip(rows, got):
        np.testing.assert_allclose(o, dense[i, h], rtol=1e-12, atol=1e-13)


def test_batch_form_is_per_sequence():
    r = grng.stream(61)
    nodes, plens = [5, 1, 9], [3, 0, 11]
    Hq, Hkv, d = 4, 2, 8
    parts = [_operands(70 + s, nodes[s], plens[s], Hq, Hkv, d) for s in range(3)]
    parents = [gtrees.random_recursive(r, m) for m in nodes]
    cat = [np.concatenate([p[j] for p in parts]) for j in range(5)]
    offs = np.concatenate([[0], np.cumsum(nodes)])
    starts = np.concatenate([[0], np.cumsum(plens)[:-1]])
    got = oatt.batch_tree_attention(*cat, np.concatenate(parents), offs, plens, starts)
    for s in range(3):
        want = _path_as_sequence(*parts[s], parents[s])
        np.testing.assert_allclose(got[offs[s]:offs[s + 1]], want, rtol=1e-12, atol=1e-12)


def test_hand_worked_fixture():
    """tests/golden/attention_worked.json: a 3-node tree over a 1-token prefix,
    head dim 1, scale 1, worked by hand from the definition."""
    with open(os.path.join(GOLDEN, "attention_worked.json")) as f:
        g = json.load(f)
    arr = lambda k: np.array(g[k], dtype=np.float64)  # noqa: E731
    got = oatt.tree_attention(arr("q"), arr("k_tree"), arr("v_tree"), arr("k_prefix"), arr("v_prefix"),
                              np.array(g["parent"]), scale=g["scale"])
    want = np.array([[[eval(x, {"math": math})] for x in row] for row in g["expected"]])  # rationals written by hand
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)


def test_flops_count():
    # chain of 3 over P=2: pairs = 3*2 + (1+2+3) = 12 -> 4*d*Hq*12
    assert oatt.flops([3], [2], [gtrees.chain(3)], Hq=2, d=8) == 4 * 8 * 2 * 12


# ---- planted mistakes: mutated copies of the oracle must fail the pins ----------------------

def _mutant(kind):
    def f(q, k_tree, v_tree, k_prefix, v_prefix, parent, scale=None):
        n, Hq, d = q.shape
        Hkv = k_tree.shape[1]
        g = Hq // Hkv
        P = k_prefix.shape[0]
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        anc = otree.ancestor_matrix(parent)
        if kind == "no-self":
            anc = anc & ~np.eye(n, dtype=bool)
            anc[0, 0] = True
        if kind == "parent-only":
            anc = np.eye(n, dtype=bool)
            for i in range(1, n):
                anc[i, parent[i]] = True
        vis = np.concatenate([np.ones((n, P), bool), anc], axis=1)
        keys = np.concatenate([k_prefix, k_tree])
        vals = np.concatenate([v_prefix, v_tree])
        out = np.empty((n, Hq, d))
        for h in range(Hq):
            kv = h % Hkv if kind == "gqa-modulo" else h // g
            sc = 1.0 if kind == "no-scale" else scale
            s = np.where(vis, sc * q[:, h] @ keys[:, kv].T, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            out[:, h] = (p / p.sum(1, keepdims=True)) @ vals[:, kv]
        return out
    return f


@pytest.mark.parametrize("kind", ["no-self", "parent-only", "gqa-modulo", "no-scale"])
def test_planted_mistakes_are_caught(kind):
    n, P, Hq, Hkv, d = 10, 4, 4, 2, 8
    parent = gtrees.random_deep(grng.stream(81), n)
    q, kt, vt, kp, vp = _operands(12, n, P, Hq, Hkv, d)
    bad = _mutant(kind)(q, kt, vt, kp, vp, parent)
    good = _mutant("none")(q, kt, vt, kp, vp, parent)
    ref = _path_as_sequence(q, kt, vt, kp, vp, parent)
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-12)
    assert not np.allclose(bad, ref, rtol=1e-6, atol=1e-9)
