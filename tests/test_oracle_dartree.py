"""Pins for the DARTree construction oracle (CPU only).

* topk_logprobs: a full sort (numpy argsort on negated values, stable) and
  scipy's logsumexp; the log-probabilities of a whole row exponentiate to 1;
  ties keep the lowest token ids.
* expand_depth: brute-force enumeration of all children; a width covering every
  child keeps them all; absent parents (-inf) have no children.
* Lemma 1 (eq. 6): best-first heap == global top-B on random supertrees with
  beta <= 0, including exact ties; a constructed beta > 0 case breaks it, and
  so does a dropped ancestor tie rule; top-B is prefix-closed.
* DDTree as a special case: with the factorised head (every parent sees the
  same per-depth log-probabilities), beta = 0 and a width that keeps every
  prefix, deferred top-B equals the independently pinned best-first builder
  (oracle.build_tree), node for node.
* The depth bonus: a very negative beta prunes breadth-first (all of depth 1
  before any of depth 2).
"""

import numpy as np
import pytest
from scipy.special import logsumexp

from gen import rng as grng
from oracle import build_tree as obt, dartree as odt, tree as otree

F32 = np.float32


def test_topk_matches_full_sort_and_logsumexp():
    r = grng.stream(1, "topk")
    x = r.standard_normal((7, 1000)).astype(np.float32)
    x[3, [5, 17, 900]] = 9.0     # a three-way tie at the top: lowest ids first
    toks, logp = odt.topk_logprobs(x, 64)
    for i in range(7):
        want = np.argsort(-x[i].astype(np.float64), kind="stable")[:64]
        np.testing.assert_array_equal(toks[i], want)
        np.testing.assert_allclose(logp[i], x[i][want].astype(np.float64) - logsumexp(x[i].astype(np.float64)),
                                   rtol=0, atol=1e-12)
    assert list(toks[3, :3]) == [5, 17, 900]
    full_t, full_lp = odt.topk_logprobs(x, 1000)
    np.testing.assert_allclose(np.exp(full_lp).sum(axis=1), 1.0, rtol=1e-12)
    t1, _ = odt.topk_logprobs(x, 5000)  # k beyond the vocabulary is clipped
    assert t1.shape == (7, 1000)


def test_expand_depth_brute_force():
    r = grng.stream(2, "expand")
    for trial in range(20):
        wp, k, w = int(r.integers(1, 6)), int(r.integers(1, 7)), int(r.integers(1, 12))
        ps = np.sort(-r.integers(0, 8, size=wp).astype(F32) * F32(0.25))[::-1]
        lq = -r.integers(0, 6, size=(wp, k)).astype(F32) * F32(0.5)
        beta = F32(-0.2) if trial % 2 else F32(0.0)
        par, cand, sc = odt.expand_depth(ps, lq, beta, w)
        allc = sorted(((-(float((ps[p] + lq[p, c]) + beta)), p, c) for p in range(wp) for c in range(k)))
        want = allc[:w]
        assert par == [p for _, p, _ in want] and cand == [c for _, _, c in want]
        assert [float(s) for s in sc] == [-s for s, _, _ in want]
        if w >= wp * k:
            assert len(par) == wp * k


def test_expand_depth_absent_parents():
    ps = np.array([0.0, -np.inf, -1.0], F32)
    lq = np.zeros((3, 2), F32)
    par, cand, sc = odt.expand_depth(ps, lq, 0.0, 10)
    assert par == [0, 0, 2, 2] and cand == [0, 1, 0, 1]


def _random_supertree(r, depths, w, k, beta, tie_levels=None):
    def head(paths):
        if tie_levels:
            v = -r.integers(0, tie_levels, size=(len(paths), k)).astype(F32) * F32(0.5)
        else:
            v = np.log(r.dirichlet(np.ones(k) * 0.7, size=len(paths))).astype(F32)
        return v
    return odt.build_supertree([head] * depths, beta, w)


@pytest.mark.parametrize("seed", range(24))
def test_lemma1_best_first_equals_top_b(seed):
    r = grng.stream(seed, "lemma1")
    depths, w, k = int(r.integers(1, 8)), int(r.integers(1, 13)), int(r.integers(1, 9))
    beta = [0.0, -0.2, -1.0][seed % 3]
    layers = _random_supertree(r, depths, w, k, beta, tie_levels=3 if seed % 4 == 0 else None)
    total = sum(len(x) for x in layers)
    for B in sorted({0, 1, 5, total // 2, total, total + 3}):
        top = odt.prune_topb(layers, B)
        assert top == odt.best_first(layers, B)
        nodes = odt.flatten_nodes(layers)
        kept = set(top)
        assert all(nodes[i][1] in kept for i in top[1:])  # prefix-closed


def test_lemma1_fails_for_positive_beta():
    # depth 1: one child of score log 0.9; its child adds log 0.9 + beta with beta > 0 large
    lq1 = np.log(np.array([[0.9, 0.1]], F32)).astype(F32)
    lq2 = np.log(np.array([[0.9, 0.1], [0.9, 0.1]], F32)).astype(F32)
    layers = odt.build_supertree([lambda p: lq1, lambda p: lq2], beta=2.0, w=4)
    assert odt.prune_topb(layers, 1) != odt.best_first(layers, 1)


def test_ancestor_tie_rule_matters():
    # parent and child with equal scores: without the depth tie-break the child could come first
    lq1 = np.zeros((1, 1), F32)
    layers = odt.build_supertree([lambda p: lq1, lambda p: np.zeros((1, 1), F32)], beta=0.0, w=1)
    nodes = odt.flatten_nodes(layers)
    assert nodes[1][5] == nodes[2][5]                    # equal scores
    assert odt.prune_topb(layers, 1) == [0, 1]           # the ancestor wins
    mutant = sorted(nodes[1:], key=lambda n: (-float(n[5]), -n[2]))[:1]  # deeper first: not prefix-closed
    assert mutant[0][0] == 2 and nodes[2][1] not in {0}


@pytest.mark.parametrize("seed", range(8))
def test_factorised_head_is_the_ddtree_heap(seed):
    r = grng.stream(seed, "ddtree-special")
    depths, k = int(r.integers(1, 4)), int(r.integers(1, 5))
    # dyadic log-probs: float32 and float64 sums agree exactly
    lp = np.sort(-r.integers(1, 1 << 14, size=(depths, k)).astype(np.float64) / (1 << 12), axis=1)[:, ::-1]
    lp = lp.astype(np.float32)
    tok = np.stack([r.choice(500, size=k, replace=False) for _ in range(depths)]).astype(np.int32)
    for d in range(depths):
        order = np.lexsort((tok[d], -lp[d]))
        lp[d], tok[d] = lp[d][order], tok[d][order]
    heads = [(lambda d: (lambda paths: np.tile(lp[d], (len(paths), 1))))(d) for d in range(depths)]
    layers = odt.build_supertree(heads, beta=0.0, w=k ** depths)
    total = sum(len(x) for x in layers)
    assert total == sum(k ** d for d in range(1, depths + 1))
    scores = [float(n[5]) for n in odt.flatten_nodes(layers)[1:]]
    if len(set(scores)) < len(scores):
        pytest.skip("exact score tie: the two builders order equal scores differently (slot vs rank tuple)")
    for n in sorted({1, 2, total // 2 + 1, total + 1}):
        kept = odt.prune_topb(layers, n - 1)
        parent, token, depth, score = odt.tree_arrays(layers, kept, tok)
        hp, ht, hd, hs = obt.build_tree_heap(lp, tok, -1, n)
        assert list(parent) == list(hp) and list(token) == list(ht) and list(depth) == list(hd)
        np.testing.assert_array_equal(score.astype(np.float64), np.array(hs))


def test_very_negative_beta_prunes_breadth_first():
    r = grng.stream(9, "bfs-beta")
    layers = _random_supertree(r, 4, 6, 3, beta=-100.0)
    kept = odt.prune_topb(layers, 10)
    nodes = odt.flatten_nodes(layers)
    depths = [nodes[i][2] for i in kept]
    # the root has k = 3 children; with beta = -100 every depth-1 node outranks every depth-2 node
    assert depths == [0] + [1] * 3 + [2] * 6 + [3]  # widths: 3 children of the root, then w = 6 per depth


def test_tree_arrays_form_a_valid_tree():
    r = grng.stream(10, "arrays")
    layers = _random_supertree(r, 6, 12, 8, beta=-0.2)
    toks = r.integers(0, 1000, size=(6, 8))
    kept = odt.prune_topb(layers, 64)
    parent, token, depth, score = odt.tree_arrays(layers, kept, toks)
    otree.check(parent)
    np.testing.assert_array_equal(depth, otree.depths(parent))
    assert all(score[i] <= score[parent[i]] for i in range(1, len(parent)))
