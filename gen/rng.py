"""Seed plumbing: one independent PCG64 stream per (workload, tensor, sequence).

A stream is addressed by an integer workload seed plus a path of small integers
or strings (for example ``stream(3, "k_prefix", 5)``). Strings are hashed with
a fixed, platform-independent function so that the mapping never changes.
"""

import zlib

import numpy as np


def _key(part):
    if isinstance(part, (int, np.integer)):
        return int(part) & 0xFFFFFFFF
    return zlib.crc32(str(part).encode("utf-8")) & 0xFFFFFFFF


def stream(seed, *path):
    """Return a numpy Generator for ``seed`` and the spawn path ``path``."""
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(_key(p) for p in path))
    return np.random.Generator(np.random.PCG64(ss))


def torch_seed(seed, *path):
    """A 63-bit integer seed for a torch generator, derived like :func:`stream`."""
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(_key(p) for p in path))
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)
