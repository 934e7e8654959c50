"""The synthetic workloads.

Shapes follow a Qwen3-4B-sized target (32 query heads, 8 KV heads, head dim
128, 36 layers, vocabulary 151936), the model the DARTree paper measures on
(Experimental Setup), at the tree budgets the paper sweeps and beyond.

Each workload lists, per sequence, the prefix length P (tokens already in the
KV cache) and the node count n of its draft tree (root included). Trees come
either from a fixed recipe (``bfs``: a random BFS-numbered tree of given depth;
``chain``) or from the best-first builder over synthetic per-depth candidate
lists for a 16-position draft block (``heap``: k = n-1 candidates per depth
from softmax(3 N(0,1)) over the full vocabulary, so the heap never runs short
of siblings; ``heap-narrow``: the same distributions cut to k = 2 candidates
per depth, which gives deeper, binary-like trees). "Depth 16" is the drafting
depth cap; the realized depth of ``heap`` trees is small because these
synthetic distributions are flat. Building the tree is the caller's job (the
library's builder, or the oracle's in tests).
"""

from dataclasses import dataclass, field

import numpy as np

from .rng import stream


@dataclass
class Workload:
    name: str
    Hq: int
    Hkv: int
    d: int
    prefix_lens: list
    nodes: list
    vocab: int
    tree: str = "heap"
    depths: int = 16
    layers: int = 1
    plant_p: float = 0.8
    plant_pick: str = "first"
    operand_scale: float = None  # None -> 1/sqrt(d)
    seed: int = 0
    notes: str = ""

    @property
    def num_seqs(self):
        return len(self.nodes)

    @property
    def g(self):
        return self.Hq // self.Hkv

    def node_offsets(self):
        return np.concatenate([[0], np.cumsum(self.nodes)]).astype(np.int32)

    def prefix_row_starts(self):
        return np.concatenate([[0], np.cumsum(self.prefix_lens)[:-1]]).astype(np.int64)

    def cache_row_starts(self):
        """First cache row of every sequence when each keeps room for its tree
        after its prefix (P_s + n_s rows), so that accepted rows can be committed."""
        room = np.asarray(self.prefix_lens, np.int64) + np.asarray(self.nodes, np.int64)
        return np.concatenate([[0], np.cumsum(room)[:-1]]).astype(np.int64)

    @property
    def total_cache_rows(self):
        return int(sum(self.prefix_lens) + sum(self.nodes))

    @property
    def total_nodes(self):
        return int(sum(self.nodes))

    @property
    def total_prefix(self):
        return int(sum(self.prefix_lens))

    def cand_k(self, n):
        return 2 if self.tree == "heap-narrow" else max(1, n - 1)


def _ragged_prefixes(seed, count, lo, hi):
    r = stream(seed, "ragged-prefix")
    return [int(x) for x in r.integers(lo, hi + 1, size=count)]


def tiny():
    return Workload("tiny", Hq=1, Hkv=1, d=64, prefix_lens=[128], nodes=[16], vocab=1024,
                    tree="bfs", depths=4, plant_pick="random", operand_scale=1.0, seed=1,
                    notes="fp32 N(0,1) operands rounded to bf16 for the device")


def qwen_b128():
    return Workload("qwen3-4b-layer-P2048-B128", Hq=32, Hkv=8, d=128, prefix_lens=[2048], nodes=[128],
                    vocab=151936, seed=2)


def qwen_b256():
    return Workload("qwen3-4b-layer-P8192-B256", Hq=32, Hkv=8, d=128, prefix_lens=[8192], nodes=[256],
                    vocab=151936, seed=3)


def qwen_b256_round():
    w = qwen_b256()
    w.name = "qwen3-4b-verify-round-P8192-B256-36L"
    w.layers = 36
    return w


def chain16():
    return Workload("qwen3-4b-layer-P8192-chain16", Hq=32, Hkv=8, d=128, prefix_lens=[8192], nodes=[16],
                    vocab=151936, tree="chain", seed=4)


def ragged():
    return Workload("ragged-8seq-P1k-16k-B256", Hq=32, Hkv=8, d=128,
                    prefix_lens=_ragged_prefixes(5, 8, 1024, 16384), nodes=[256] * 8, vocab=151936, seed=5)


def long_context():
    return Workload("long-4seq-P32768-B512-36L", Hq=32, Hkv=8, d=128, prefix_lens=[32768] * 4,
                    nodes=[512] * 4, vocab=151936, layers=36, seed=6)


ALL = {
    "tiny": tiny,
    "b128": qwen_b128,
    "b256": qwen_b256,
    "round": qwen_b256_round,
    "chain16": chain16,
    "ragged": ragged,
    "long": long_context,
}


def get(name):
    return ALL[name]()
