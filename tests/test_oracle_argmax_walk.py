"""Pins for the argmax and acceptance-walk oracles (CPU only).

* argmax: numpy's routine against an explicit scan, planted rows with known
  answers, constructed ties (lowest index wins), signed zeros.
* walk: brute force over all nodes (the deepest node whose every edge matches
  the target's greedy prediction at its parent), closed forms (a fully planted
  chain accepts everything; a root mismatch accepts nothing), a hand-worked
  fixture, and planted mistakes in copies of the walk.
"""

import json
import os

import numpy as np
import pytest

from gen import rng as grng, tensors as gten, trees as gtrees
from oracle import argmax as oarg, tree as otree, walk as owalk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_argmax_matches_explicit_scan():
    x = grng.stream(1).standard_normal((17, 257)).astype(np.float32)
    np.testing.assert_array_equal(oarg.argmax_rows(x), oarg.argmax_rows_loop(x))


def test_argmax_planted_and_ties():
    x = np.zeros((5, 64), np.float32)
    x[0, 17] = 1.0                      # planted single max
    x[1, [3, 40]] = 2.0                 # tie: lowest index
    x[2, :] = -1.0                      # all equal: index 0
    x[3, 0], x[3, 5] = -0.0, 0.0        # signed zeros compare equal: index 0 (rest are +0 too)
    x[4, 63] = np.float32(np.finfo(np.float32).max)
    want = [17, 3, 0, 0, 63]
    np.testing.assert_array_equal(oarg.argmax_rows(x), want)
    np.testing.assert_array_equal(oarg.argmax_rows_loop(x), want)


def _brute_force_walk(parent, token, argmax):
    """Deepest node whose whole root path matches; unique when sibling tokens are distinct."""
    best = 0
    for i in range(len(parent)):
        path = otree.path_to_root(parent, i)
        if all(int(token[c]) == int(argmax[int(parent[c])]) for c in path[1:]):
            if len(path) > len(otree.path_to_root(parent, best)):
                best = i
    path = otree.path_to_root(parent, best)
    return path, len(path) - 1, int(argmax[best])


@pytest.mark.parametrize("seed", range(12))
def test_walk_matches_brute_force(seed):
    r = grng.stream(seed, "walk")
    n = int(r.integers(1, 60))
    parent = [gtrees.random_recursive, gtrees.random_deep][seed % 2](r, n)
    token = gtrees.distinct_sibling_tokens(r, parent, 50)
    lg = gten.logits(r, n, 50)
    gten.plant(r, lg, parent, token, p=0.9, pick="random")
    am = oarg.argmax_rows(lg)
    assert owalk.accept_path(parent, token, am) == _brute_force_walk(parent, token, am)


def test_walk_closed_forms():
    n = 16
    parent = gtrees.chain(n)
    token = np.arange(100, 100 + n)
    am = np.append(token[1:], 7)                      # every prediction matches the next chain token
    path, L, bonus = owalk.accept_path(parent, token, am)
    assert path == list(range(n)) and L == n - 1 and bonus == 7
    am2 = am.copy()
    am2[0] = 5                                        # root mismatch
    assert owalk.accept_path(parent, token, am2) == ([0], 0, 5)
    assert owalk.accept_path([-1], [3], [9]) == ([0], 0, 9)   # root-only tree


def test_walk_duplicate_siblings_take_lowest_index():
    parent = [-1, 0, 0, 2]
    token = [0, 5, 5, 6]
    am = [5, 1, 6, 2]
    assert owalk.accept_path(parent, token, am) == ([0, 1], 1, 1)


def test_walk_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "walk_worked.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        path, L, bonus = owalk.accept_path(case["parent"], case["token"], case["argmax"])
        assert [path, L, bonus] == [case["path"], case["L"], case["bonus"]], case["name"]


def test_batch_walk():
    offs = [0, 3, 4]
    parent = [-1, 0, 0, -1]
    token = [9, 4, 5, 1]
    am = [5, 0, 0, 2]
    assert owalk.batch_accept_path(parent, token, am, offs) == [([0, 2], 1, 0), ([0], 0, 2)]


@pytest.mark.parametrize("kind", ["first-mismatch-continues", "highest-index", "bonus-from-parent"])
def test_planted_walk_mistakes_are_caught(kind):
    def mutant(parent, token, argmax):
        n, cur, path = len(parent), 0, [0]
        while True:
            m = [c for c in range(n) if parent[c] == cur and token[c] == argmax[cur]]
            if not m:
                if kind == "first-mismatch-continues":
                    kids = [c for c in range(n) if parent[c] == cur]
                    if kids and len(path) < 3:
                        cur = kids[0]
                        path.append(cur)
                        continue
                break
            cur = max(m) if kind == "highest-index" else min(m)
            path.append(cur)
        bonus = argmax[parent[cur]] if kind == "bonus-from-parent" and cur else argmax[cur]
        return path, len(path) - 1, int(bonus)

    caught = False
    for seed in range(30):
        r = grng.stream(seed, "mut")
        parent = gtrees.random_recursive(r, 25)
        token = r.integers(0, 4, size=25)  # small vocab: duplicate siblings and mismatches happen
        am = r.integers(0, 4, size=25)
        if mutant(parent, token, am) != owalk.accept_path(parent, token, am):
            caught = True
            break
    assert caught
