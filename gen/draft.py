"""Synthetic drafter output: per-depth ranked candidate lists.

A block-parallel drafter emits one distribution per draft position (the
factorised drafting distribution of the DARTree paper, Preliminaries >
Parallel Drafting and Causal Correction, eq. 3). Here those distributions are
synthetic: position d gets ``softmax(scale * z_d)`` with ``z_d ~ N(0, 1)`` over
the whole vocabulary. The tree builder consumes, per depth, the ``k`` most
likely tokens in descending log-probability (ties by ascending token id), as a
``float32 [depths][k]`` log-prob table and an ``int32 [depths][k]`` token table.
"""

import numpy as np


def candidates(rng, depths=16, vocab=151936, k=64, scale=3.0):
    """Return ``(cand_logprob float32 [depths, k], cand_token int32 [depths, k])``."""
    if k > vocab:
        raise ValueError("k must not exceed the vocabulary")
    lp = np.empty((depths, k), np.float32)
    tok = np.empty((depths, k), np.int32)
    ids = np.arange(vocab)
    for d in range(depths):
        z = rng.standard_normal(vocab) * scale
        m = z.max()
        logp = (z - (m + np.log(np.exp(z - m).sum()))).astype(np.float32)
        order = np.lexsort((ids, -logp))[:k]
        lp[d] = logp[order]
        tok[d] = order.astype(np.int32)
    return lp, tok


def tied_candidates(rng, depths, k, vocab, levels=3):
    """Candidate rows drawn from a few distinct log-prob levels, so that many
    prefixes tie exactly (exercises the tie-breaking rules)."""
    base = np.sort(-rng.integers(0, levels, size=(depths, k)).astype(np.float32) * 0.5 - 0.25, axis=1)[:, ::-1]
    tok = np.stack([rng.choice(vocab, size=k, replace=False) for _ in range(depths)]).astype(np.int32)
    # within equal log-probs order tokens ascending, as the contract asks
    for d in range(depths):
        order = np.lexsort((tok[d], -base[d]))
        base[d] = base[d][order]
        tok[d] = tok[d][order]
    return np.ascontiguousarray(base), np.ascontiguousarray(tok)
