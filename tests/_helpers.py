"""Shared helpers for the GPU parity tests (not a test module)."""

import numpy as np
import pytest

from gen import configs as gconf, draft as gdraft, rng as grng, tensors as gten, trees as gtrees
from oracle import build_tree as obt


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def dev_bf16(a, device="cuda:0"):
    """Host float32 array of bf16-representable values -> bf16 CUDA tensor (exact)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(torch.bfloat16)


def dev_i32(a, device="cuda:0"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host_f64(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_attention_close(got, ref, atol=2e-2, rel=1e-2, what=""):
    """Attention tolerance: max |got - ref| <= atol, and for every (node, head)
    row, max |got - ref| / max |ref| <= rel (element-wise relative error is
    meaningless near zero; the row-relative bound rejects e.g. an all-zero
    output on small-magnitude rows)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    assert err.max() <= atol, f"{what}: max abs err {err.max():.3e} > {atol}"
    scale = np.abs(ref).max(axis=-1)
    row_rel = err.max(axis=-1) / np.maximum(scale, 1e-30)
    worst = np.unravel_index(np.argmax(row_rel), row_rel.shape)
    assert row_rel.max() <= rel, f"{what}: row-relative err {row_rel.max():.3e} > {rel} at {worst}"


def tree(shape, n, seed, vocab=151936, depths=16):
    """(parent, token) of a tree of n nodes for the given shape recipe.
    Heap trees are built with the oracle's builder."""
    r = grng.stream(seed, "tree", shape, n)
    if shape == "chain":
        parent = gtrees.chain(n)
    elif shape == "bfs":
        parent = gtrees.bfs_tree(r, n, min(4, max(n - 1, 0)))[0]
    elif shape == "recursive":
        parent = gtrees.random_recursive(r, n)
    elif shape == "deep":
        parent = gtrees.random_deep(r, n)
    elif shape in ("heap", "heap-narrow"):
        k = 2 if shape == "heap-narrow" else max(1, n - 1)
        lp, tok = gdraft.candidates(r, depths=depths, vocab=vocab, k=k)
        p, t, _, _ = obt.build_tree_heap(lp, tok, int(r.integers(0, vocab)), n)
        return np.array(p, np.int32), np.array(t, np.int32)
    else:
        raise ValueError(shape)
    return parent, gtrees.distinct_sibling_tokens(r, parent, vocab)


def workload_inputs(w, seed_extra=0):
    """Host inputs of a (small enough) workload: per-sequence trees and packed
    bf16-valued operands."""
    nodes, plens = w.nodes, w.prefix_lens
    parents, tokens = [], []
    for s, n in enumerate(nodes):
        p, t = tree(w.tree if w.tree != "bfs" else "bfs", n, w.seed * 1000 + s + seed_extra, vocab=w.vocab)
        parents.append(p)
        tokens.append(t)
    r = grng.stream(w.seed, "operands", seed_extra)
    ops = [gten.attention_operands(r, n, P, w.Hq, w.Hkv, w.d, scale=w.operand_scale) for n, P in zip(nodes, plens)]
    cat = {k: np.concatenate([o[k] for o in ops]) for k in ops[0]}
    return parents, tokens, cat
