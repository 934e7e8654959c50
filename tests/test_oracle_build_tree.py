"""Pins for the best-first tree builder oracle (CPU only).

* heap == brute force: the heap's output equals the first n-1 prefixes of the
  full enumeration sorted by (score desc, depth asc, rank tuple asc), node for
  node, also when many prefixes tie exactly (Lemma 1 of the DARTree paper:
  best-first equals top-B for non-positive steps with ancestors first).
* optimality: on tiny instances, an exhaustive search over every prefix-closed
  set of the same size finds no larger total mass (Tree Verification and
  DDTree, eq. 4 and the mass decomposition after it).
* invariants on full-size inputs; k = 1 gives a chain; a hand-worked fixture.
"""

import json
import os

import numpy as np
import pytest

from gen import draft as gdraft, rng as grng
from oracle import build_tree as obt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_table(r, depths, k, vocab=1000):
    lp = np.sort(np.log(r.dirichlet(np.ones(k + 3), size=depths)[:, :k]).astype(np.float32), axis=1)[:, ::-1]
    tok = np.stack([r.choice(vocab, size=k, replace=False) for _ in range(depths)]).astype(np.int32)
    return np.ascontiguousarray(lp), tok


@pytest.mark.parametrize("seed", range(10))
def test_heap_equals_bruteforce(seed):
    r = grng.stream(seed, "bt")
    depths, k = int(r.integers(1, 5)), int(r.integers(1, 5))
    lp, tok = _random_table(r, depths, k)
    total = sum(k ** d for d in range(1, depths + 1))
    for n in sorted({1, 2, 3, min(total + 1, 9), total + 1, total + 4}):
        assert obt.build_tree_heap(lp, tok, 5, n) == obt.build_tree_bruteforce(lp, tok, 5, n)


@pytest.mark.parametrize("seed", range(6))
def test_heap_equals_bruteforce_with_ties(seed):
    r = grng.stream(seed, "ties")
    lp, tok = gdraft.tied_candidates(r, depths=3, k=3, vocab=40, levels=2)
    for n in (2, 5, 9, 14, 40):
        assert obt.build_tree_heap(lp, tok, 1, n) == obt.build_tree_bruteforce(lp, tok, 1, n)


@pytest.mark.parametrize("seed", range(6))
def test_heap_reaches_exhaustive_optimum(seed):
    r = grng.stream(seed, "opt")
    depths, k = (3, 2) if seed % 2 else (2, 3)
    lp, tok = _random_table(r, depths, k)
    for n in (2, 4, 6):
        _, _, _, score = obt.build_tree_heap(lp, tok, 0, n)
        got = float(np.sum(np.exp(score[1:])))
        assert got == pytest.approx(obt.best_total_mass(lp, n), rel=1e-12)


def _check_invariants(parent, token, depth, score):
    n = len(parent)
    assert parent[0] == -1 and depth[0] == 0 and score[0] == 0.0
    kids = {}
    for i in range(1, n):
        p = parent[i]
        assert 0 <= p < i
        assert depth[i] == depth[p] + 1
        assert score[i] <= score[p]              # non-increasing along every path (Lemma 1)
        assert score[i] <= score[i - 1] or i == 1  # popped in non-increasing score order
        kids.setdefault(p, []).append(token[i])
    for toks in kids.values():
        assert len(set(toks)) == len(toks)       # a prefix tree: distinct sibling tokens


@pytest.mark.parametrize("n,k", [(128, 2), (256, 2), (512, 2), (128, 127)])
def test_full_size_invariants(n, k):
    lp, tok = gdraft.candidates(grng.stream(n, k, "full"), depths=16, vocab=151936, k=k)
    out = obt.build_tree_heap(lp, tok, 17, n)
    assert len(out[0]) == n
    _check_invariants(*out)
    assert max(out[2]) <= 16                   # the drafting depth cap


def test_k1_gives_chain():
    lp = np.full((5, 1), -0.5, np.float32)
    tok = np.arange(5, dtype=np.int32)[:, None]
    parent, token, depth, _ = obt.build_tree_heap(lp, tok, 9, 100)
    assert parent == [-1, 0, 1, 2, 3, 4] and depth == [0, 1, 2, 3, 4, 5] and token == [9, 0, 1, 2, 3, 4]


def test_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "heap_worked.json")) as f:
        g = json.load(f)
    lp = np.log(np.array(g["probs"], np.float64)).astype(np.float32)
    tok = np.array(g["tokens"], np.int32)
    for case in g["cases"]:
        parent, token, depth, score = obt.build_tree_heap(lp, tok, g["root_token"], case["n_nodes"])
        assert parent == case["parent"] and token == case["token"] and depth == case["depth"]
        np.testing.assert_allclose(np.exp(score), case["mass"], rtol=1e-6)
