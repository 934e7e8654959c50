"""The target's sample at every tree node, for verification at temperature T > 0.

TEST INFRASTRUCTURE ONLY (see the package docstring).

DARTree paper, Preliminaries > Speculative Sampling: exact target-sample
matching (the DFlash rule) accepts consecutive draft tokens while each equals
the target's sample at that position, and emits the target's sample at the
first mismatch; Experimental Setup > Evaluation Details applies the same rule
on a tree at T = 1: the longest sampled prefix in the tree is accepted. The
target distribution at temperature T is p_T(j) proportional to exp(l_j / T)
(the "p_T" of the same passage).

How the sample is drawn is not fixed by the pages. Reading taken here:
Gumbel-max. With G_j = -ln(-ln U_j) for independent uniforms U_j, the index
argmax_j (l_j / T + G_j) is distributed exactly as p_T (Gumbel 1954; the
"Gumbel-max trick"). Its uniforms come from a counter-based generator so that
every (row, vocabulary index) has its own reproducible draw:

  Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
  Easy as 1, 2, 3", SC 2011): a 128-bit counter (c0, c1, c2, c3) and a 64-bit
  key (k0, k1); ten rounds, each multiplying c0 by 0xD2511F53 and c2 by
  0xCD9E8D57 into 64-bit products, then
      (c0, c1, c2, c3) <- (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)),
  with the key bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85) before
  every round after the first.

Stream layout (a choice of this library, stated with its entry point): for
row r, vocabulary index j, seed s and offset o,
  bits = Philox4x32-10(counter = (r, j // 4, o mod 2^32, o // 2^32),
                       key = (s mod 2^32, s // 2^32))[j mod 4]
  U    = (2 * (bits >> 9) + 1) / 2^24          (an odd multiple of 2^-24 in (0, 1))
The oracle evaluates the score l_j / T - ln(-ln U_j) in float64 and takes the
lowest index among the maxima.
"""

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Scalar Philox4x32-10 on Python integers: four 32-bit words out."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = (p1 >> 32) ^ c1 ^ k0, p1 & MASK32, (p0 >> 32) ^ c3 ^ k1, p0 & MASK32
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """The same generator on numpy arrays (broadcast); returns four uint64 arrays
    holding 32-bit words. Products of two 32-bit values fit uint64 exactly."""
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(MASK32) for x in (c0, c1, c2, c3)]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    k0 = int(k0) & MASK32
    k1 = int(k1) & MASK32
    m32 = np.uint64(MASK32)
    s32 = np.uint64(32)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = c0 * np.uint64(M0)
        p1 = c2 * np.uint64(M1)
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ np.uint64(k0), p1 & m32, (p0 >> s32) ^ c3 ^ np.uint64(k1), p0 & m32)
    return c0, c1, c2, c3


def uniform_from_bits(bits):
    """(2 * (bits >> 9) + 1) / 2^24 in float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint64) >> np.uint64(9)
    return (2.0 * b.astype(np.float64) + 1.0) / float(1 << 24)


def bits(row_ids, vocab, seed, offset):
    """The 32-bit draw of every (row, vocabulary index): uint64 array [len(row_ids), vocab]."""
    rows = np.asarray(row_ids, dtype=np.uint64).reshape(-1, 1)
    blocks = (int(vocab) + 3) // 4
    j4 = np.arange(blocks, dtype=np.uint64).reshape(1, -1)
    words = philox4x32_10_np(rows, j4, int(offset) & MASK32, (int(offset) >> 32) & MASK32,
                             int(seed) & MASK32, (int(seed) >> 32) & MASK32)
    # word w of block b belongs to vocabulary index 4 * b + w
    return np.stack(words, axis=2).reshape(rows.shape[0], 4 * blocks)[:, :vocab]


def uniforms(row_ids, vocab, seed, offset):
    """U for every (row, vocabulary index), float64 [len(row_ids), vocab]."""
    return uniform_from_bits(bits(row_ids, vocab, seed, offset))


def gumbel(u):
    """Standard Gumbel variates -ln(-ln u) for uniforms u in (0, 1), float64."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u))


def perturbed_scores(logits, temperature, row_ids, seed, offset):
    """l / T + G for rows of logits (float64 [len(row_ids), vocab]); row k of
    ``logits`` draws from the stream of row index row_ids[k]."""
    lg = np.asarray(logits, dtype=np.float64)
    return lg / float(temperature) + gumbel(uniforms(row_ids, lg.shape[1], seed, offset))


def sample_rows(logits, temperature, seed, offset, return_scores=False, block=32):
    """Gumbel-max sample of every row: the lowest index among the maxima of
    l / T + G, row r drawing from the stream of row index r. Returns int64
    [rows] (and the float64 score matrix when return_scores). Rows are handled
    ``block`` at a time only to bound memory."""
    lg = np.asarray(logits)
    rows = lg.shape[0]
    out = np.empty(rows, np.int64)
    scores = np.empty(lg.shape, np.float64) if return_scores else None
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        s = perturbed_scores(lg[r0:r1], temperature, np.arange(r0, r1), seed, offset)
        out[r0:r1] = np.argmax(s, axis=1)
        if return_scores:
            scores[r0:r1] = s
    return (out, scores) if return_scores else out


def target_distribution(logits_row, temperature):
    """p_T = softmax(l / T) in float64 (for distribution checks)."""
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()
