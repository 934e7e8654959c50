"""Pins for the sampling oracle (CPU only).

* Philox4x32-10 against the generator's published known-answer values
  (tests/golden/philox_kat.json), in both the scalar and the numpy form; planted
  changes to the round function miss those values.
* The uniform map's closed form at its extreme inputs.
* Uniformity (chi-square) and lag-1 independence of the uniforms.
* The Gumbel law of -ln(-ln U): mean Euler's gamma, variance pi^2/6, and a
  Kolmogorov-Smirnov test against exp(-exp(-x)).
* The Gumbel-max theorem: sampled frequencies against softmax(l / T) at three
  temperatures, and planted mistakes (sign of the noise, T multiplied instead of
  divided, one logarithm dropped) are rejected by the same test.
* T -> 0 reduces to the greedy rule (the argmax oracle), the T = 0 case of
  DARTree, Preliminaries > Speculative Sampling.
"""

import json
import os

import numpy as np
import pytest
from scipy import stats

from gen import rng as grng
from oracle import argmax as oarg, sample as osmp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
P_MIN = 1e-6  # a deterministic seed either passes or fails; this threshold only needs to reject real mistakes


def _kat():
    with open(os.path.join(GOLDEN, "philox_kat.json")) as f:
        return [([int(x, 16) for x in c["counter"]], [int(x, 16) for x in c["key"]], [int(x, 16) for x in c["out"]])
                for c in json.load(f)["cases"]]


def test_philox_known_answers():
    for ctr, key, out in _kat():
        assert list(osmp.philox4x32_10(ctr, key)) == out
        got = osmp.philox4x32_10_np(*ctr, *key)
        assert [int(w) for w in got] == out


def test_philox_numpy_matches_scalar():
    r = grng.stream(5, "philox")
    c = r.integers(0, 1 << 32, size=(200, 4), dtype=np.uint64)
    k = r.integers(0, 1 << 32, size=(200, 2), dtype=np.uint64)
    for i in range(200):
        want = osmp.philox4x32_10(c[i], k[i])
        got = osmp.philox4x32_10_np(*c[i], *k[i])
        assert [int(w) for w in got] == list(want)


def _mutant_philox(counter, key, kind):
    m0, m1, w0, w1, mask = osmp.M0, osmp.M1, osmp.W0, osmp.W1, osmp.MASK32
    c0, c1, c2, c3 = counter
    k0, k1 = key
    rounds = 9 if kind == "nine-rounds" else 10
    for rnd in range(rounds):
        if rnd > 0 and kind != "no-key-bump":
            k0, k1 = (k0 + w0) & mask, (k1 + w1) & mask
        if kind == "swapped-multipliers":
            p0, p1 = m1 * c0, m0 * c2
        else:
            p0, p1 = m0 * c0, m1 * c2
        if kind == "swapped-outputs":
            c0, c1, c2, c3 = (p0 >> 32) ^ c1 ^ k0, p0 & mask, (p1 >> 32) ^ c3 ^ k1, p1 & mask
        else:
            c0, c1, c2, c3 = (p1 >> 32) ^ c1 ^ k0, p1 & mask, (p0 >> 32) ^ c3 ^ k1, p0 & mask
    return [c0, c1, c2, c3]


@pytest.mark.parametrize("kind", ["nine-rounds", "no-key-bump", "swapped-multipliers", "swapped-outputs"])
def test_planted_philox_mistakes_miss_the_known_answers(kind):
    assert any(_mutant_philox(ctr, key, kind) != out for ctr, key, out in _kat())


def test_uniform_map_closed_form():
    b = np.array([0, 511, 512, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = osmp.uniform_from_bits(b)
    want = np.array([1, 1, 3, (1 << 24) - 1, (1 << 23) + 1], np.float64) / (1 << 24)
    np.testing.assert_array_equal(u, want)
    assert (u > 0).all() and (u < 1).all()
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)  # exact in float32


def _many_uniforms():
    return osmp.uniforms(np.arange(16), 1 << 16, seed=0x1234_5678_9ABC, offset=77).reshape(-1)


def test_uniforms_are_uniform_and_serially_independent():
    u = _many_uniforms()
    n = u.size
    counts = np.bincount(np.floor(u * 256).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > P_MIN
    x = u - 0.5
    rho = float(np.dot(x[:-1], x[1:]) / np.dot(x, x))
    assert abs(rho) < 6 / np.sqrt(n)
    # each of the four output words of a block is uniform on its own
    for w in range(4):
        cw = np.bincount(np.floor(u[w::4] * 64).astype(np.int64), minlength=64)
        assert stats.chisquare(cw).pvalue > P_MIN


def test_gumbel_law():
    g = osmp.gumbel(_many_uniforms())
    n = g.size
    sd = np.pi / np.sqrt(6)
    assert abs(g.mean() - np.euler_gamma) < 6 * sd / np.sqrt(n)
    # sd of the sample variance: sigma^2 * sqrt((kurtosis - 1) / n), Gumbel kurtosis 5.4
    assert abs(g.var() - np.pi ** 2 / 6) < 6 * sd ** 2 * np.sqrt(4.4 / n)
    assert stats.kstest(g, "gumbel_r").pvalue > P_MIN


def _law_logits():
    return (grng.stream(3, "law").standard_normal(12) * 1.5).astype(np.float32)


def _freq(picks, vocab):
    return np.bincount(picks, minlength=vocab)


def _chi2_p(counts, p):
    n = counts.sum()
    return stats.chisquare(counts, n * p).pvalue


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_gumbel_max_draws_from_the_target_distribution(T):
    lg = _law_logits()
    rows = 30000
    picks = osmp.sample_rows(np.tile(lg, (rows, 1)), T, seed=11, offset=int(T * 4), block=4096)
    assert _chi2_p(_freq(picks, lg.size), osmp.target_distribution(lg, T)) > P_MIN


@pytest.mark.parametrize("kind", ["noise-sign", "T-multiplies", "single-log"])
def test_planted_sampling_mistakes_fail_the_law(kind):
    lg = _law_logits().astype(np.float64)
    rows, T = 30000, 0.5
    u = osmp.uniforms(np.arange(rows), lg.size, seed=11, offset=2)
    if kind == "noise-sign":
        s = lg / T + np.log(-np.log(u))
    elif kind == "T-multiplies":
        s = lg * T - np.log(-np.log(u))
    else:
        s = lg / T - np.log(u)
    picks = np.argmax(s, axis=1)
    assert _chi2_p(_freq(picks, lg.size), osmp.target_distribution(lg, T)) < P_MIN


def test_small_temperature_is_the_greedy_rule():
    r = grng.stream(8, "cold")
    x = r.standard_normal((8, 5000)).astype(np.float32)
    for i in range(8):
        x[i, r.integers(0, 5000)] = x[i].max() + np.float32(0.05)
    np.testing.assert_array_equal(osmp.sample_rows(x, 1e-4, seed=1, offset=0), oarg.argmax_rows(x))


def test_streams_are_keyed_by_row_seed_and_offset():
    base = osmp.bits([0, 1, 2], 64, seed=5, offset=9)
    np.testing.assert_array_equal(base, osmp.bits([0, 1, 2], 64, seed=5, offset=9))
    np.testing.assert_array_equal(base[1], osmp.bits([1], 64, seed=5, offset=9)[0])
    for other in (osmp.bits([0, 1, 2], 64, seed=6, offset=9), osmp.bits([0, 1, 2], 64, seed=5, offset=10),
                  osmp.bits([0, 1, 2], 64, seed=5 + (1 << 32), offset=9),
                  osmp.bits([0, 1, 2], 64, seed=5, offset=9 + (1 << 32))):
        assert (other != base).mean() > 0.99
    assert (base[0] != base[1]).mean() > 0.99
    # vocabulary index j uses word j % 4 of block j // 4: a row's first block is the scalar generator's output
    assert [int(v) for v in base[2, :4]] == list(osmp.philox4x32_10((2, 0, 9, 0), (5, 0)))
