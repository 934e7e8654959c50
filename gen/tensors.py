"""Seeded attention operands and target logits.

Attention operands are bf16 on the device. Host-side generators return
float32 arrays whose every value is exactly representable in bf16 (rounded to
nearest-even), so that the device copy and the host copy hold the same numbers.
Big timing-only tensors are drawn directly on the device with a seeded torch
generator (:func:`device_randn_bf16`, :func:`device_logits`).
"""

import numpy as np

from .rng import torch_seed
from .trees import children_lists


def bf16_round(x):
    """Round a float32 array to the nearest bf16 value (ties to even); returns float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal_bf16(rng, shape, scale=1.0):
    """N(0, scale^2) samples rounded to bf16 (float32 array)."""
    return bf16_round(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def attention_operands(rng, n, P, Hq, Hkv, d, scale=None):
    """Q [n,Hq,d], K_tree/V_tree [n,Hkv,d], K_prefix/V_prefix [P,Hkv,d], all
    ~ N(0, scale^2) rounded to bf16. ``scale`` defaults to 1/sqrt(d) (the
    Qwen-shaped distribution); ``scale=1`` gives the "sharp" variant."""
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return {
        "q": normal_bf16(rng, (n, Hq, d), scale),
        "k_tree": normal_bf16(rng, (n, Hkv, d), scale),
        "v_tree": normal_bf16(rng, (n, Hkv, d), scale),
        "k_prefix": normal_bf16(rng, (P, Hkv, d), scale),
        "v_prefix": normal_bf16(rng, (P, Hkv, d), scale),
    }


def logits(rng, rows, vocab):
    """Target logits ~ N(0, 1), float32 [rows, vocab]."""
    return rng.standard_normal((rows, vocab), dtype=np.float32)


def plant(rng, logits_rows, parent, token, p=0.8, pick="first"):
    """Plant the greedy prediction on draft children, in place.

    For each node u that has children, with probability ``p`` the logit of one
    child's token is raised to ``max(logits[u]) + 1`` so that the target's
    greedy prediction at u equals that child's token. ``pick="first"`` takes the
    lowest-index child (for a best-first tree, its highest-scoring child);
    ``pick="random"`` takes a uniformly drawn child. Returns the planted node list.
    """
    planted = []
    for u, kids in enumerate(children_lists(parent)):
        if not kids:
            continue
        if rng.random() < p:
            c = kids[0] if pick == "first" else kids[int(rng.integers(0, len(kids)))]
            logits_rows[u, token[c]] = logits_rows[u].max() + np.float32(1.0)
            planted.append(u)
    return planted


def device_randn_bf16(shape, seed, *path, scale=1.0, device="cuda"):
    """bf16 tensor ~ N(0, scale^2) drawn on ``device`` with a seeded generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, *path))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch.bfloat16)


def device_logits(rows, vocab, seed, *path, device="cuda"):
    """float32 logits ~ N(0, 1) [rows, vocab] drawn on ``device``."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, *path))
    return torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32)


def device_plant(rng, logits_dev, row0, parent, token, p=0.8):
    """:func:`plant` with pick="first" for a device tensor whose rows
    ``row0 .. row0+len(parent)-1`` belong to one tree."""
    import torch

    kids = children_lists(parent)
    rows, cols = [], []
    for u, ks in enumerate(kids):
        if ks and rng.random() < p:
            rows.append(row0 + u)
            cols.append(int(token[ks[0]]))
    if not rows:
        return []
    r = torch.tensor(rows, device=logits_dev.device, dtype=torch.long)
    c = torch.tensor(cols, device=logits_dev.device, dtype=torch.long)
    mx = logits_dev[r].max(dim=1).values
    logits_dev[r, c] = mx + 1.0
    return [x - row0 for x in rows]
