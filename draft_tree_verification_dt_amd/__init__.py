"""Draft-tree verification on MI355X: Python binding of libdtree.

Same names as the C ABI (include/dtree.h). These wrappers only marshal
arguments: numpy arrays for host data, torch CUDA tensors for device memory,
the current torch stream as the HIP stream. Every step of the computation runs
in libdtree (host C++ for the tree builder, HIP kernels for the rest).

    dt_build_tree       best-first (DDTree) draft-tree construction, host
    dt_tree_attention   ancestor-only tree attention over a KV-cached prefix
    dt_tree_attention_noalloc  the same without a workspace (a static device buffer)
    dt_argmax_rows      per-node greedy prediction (row arg-max, lowest index on ties)
    dt_sample_rows      per-node target sample at temperature T > 0 (Gumbel-max, Philox4x32-10)
    dt_accept_path      longest accepted root-to-leaf path and bonus token
    dt_commit_kv        accepted path's keys and values into the KV cache, all layers
    dt_topk_rows        per-depth top-K draft candidates with log-softmax values
    dt_expand_depth     one depth of DARTree's fixed-width supertree
    dt_prune_topb       deferred top-B pruning of the supertree into the verification tree
"""

import ctypes

import numpy as np

from . import _lib
from ._lib import dt_attn_desc  # noqa: F401

__all__ = [
    "DtError", "dt_status_string", "dt_abi_version", "dt_build_tree", "dt_validate_tree",
    "AttnLayout", "dt_tree_attention_workspace_size", "dt_tree_attention", "dt_tree_attention_noalloc",
    "dt_argmax_rows_workspace_size", "dt_argmax_rows", "dt_sample_rows_workspace_size", "dt_sample_rows",
    "dt_accept_path", "dt_commit_kv", "CommitArgs", "dt_topk_rows_workspace_size", "dt_topk_rows",
    "dt_expand_depth", "dt_prune_topb", "library_path",
]


class DtError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {dt_status_string(status)} (status {status})")


def library_path():
    return _lib.LIB_PATH


def _check(status, where):
    if status != _lib.DT_OK:
        raise DtError(status, where)


def dt_status_string(status):
    return _lib.load().dt_status_string(int(status)).decode()


def dt_abi_version():
    return _lib.load().dt_abi_version()


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def dt_build_tree(cand_logprob, cand_token, root_token, n_nodes, with_score=True):
    """Best-first tree over per-depth ranked candidates (host).

    cand_logprob float32 [depths, k] (rows non-increasing, entries <= 0),
    cand_token int32 [depths, k]. Returns (parent, token, depth, score) numpy
    arrays of the realised node count (score is None if with_score=False).
    """
    lib = _lib.load()
    lp = np.ascontiguousarray(cand_logprob, dtype=np.float32)
    tok = _i32(cand_token)
    if lp.ndim != 2 or lp.shape != tok.shape:
        raise ValueError("cand_logprob and cand_token must be 2-D and of equal shape")
    depths, k = lp.shape
    n_nodes = int(n_nodes)
    size = max(n_nodes, 1)
    parent = np.empty(size, np.int32)
    token = np.empty(size, np.int32)
    depth = np.empty(size, np.int32)
    score = np.empty(size, np.float64) if with_score else None
    n_out = ctypes.c_int32(0)
    st = lib.dt_build_tree(depths, k, _ptr(lp, ctypes.c_float), _ptr(tok, ctypes.c_int32), int(root_token), n_nodes,
                           _ptr(parent, ctypes.c_int32), _ptr(token, ctypes.c_int32), _ptr(depth, ctypes.c_int32),
                           _ptr(score, ctypes.c_double) if with_score else None, ctypes.byref(n_out))
    _check(st, "dt_build_tree")
    m = n_out.value
    return parent[:m], token[:m], depth[:m], (score[:m] if with_score else None)


def dt_validate_tree(parent):
    """Status code (0 = valid) of a host parent array."""
    p = _i32(parent)
    return _lib.load().dt_validate_tree(_ptr(p, ctypes.c_int32) if p.size else None, int(p.size))


class AttnLayout:
    """Host-side sequence metadata of a (possibly ragged) batch of trees.

    node_offsets int32 [S+1]; prefix_lens int32 [S]; prefix_row_start int64 [S]
    (first cache row of each sequence; defaults to the packed layout).
    """

    def __init__(self, node_offsets, prefix_lens, prefix_row_start=None):
        self.node_offsets = _i32(node_offsets)
        self.prefix_lens = _i32(prefix_lens)
        if prefix_row_start is None:
            prefix_row_start = np.concatenate([[0], np.cumsum(self.prefix_lens, dtype=np.int64)[:-1]])
        self.prefix_row_start = np.ascontiguousarray(prefix_row_start, dtype=np.int64)
        if len(self.node_offsets) != len(self.prefix_lens) + 1 or len(self.prefix_row_start) != len(self.prefix_lens):
            raise ValueError("node_offsets must have one more entry than prefix_lens / prefix_row_start")

    @property
    def num_seqs(self):
        return len(self.prefix_lens)


def _row_stride(t, minimum):
    """Row stride to pass for a tensor's first dimension: a single row may carry
    any stride (numpy and torch give size-1 dimensions arbitrary ones)."""
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), minimum)


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _req(t, name, dtype, device=None, min_len=None, flat=False):
    """Check a device argument before its pointer reaches the library, which
    cannot check dtypes, devices or extents itself: a torch CUDA tensor of
    ``dtype`` (on ``device`` when given), with at least ``min_len`` entries along
    its first dimension; ``flat`` asks for a unit-stride 1-D view of them.
    Returns the tensor's device."""
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a CUDA tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, other operands on {device}")
    if flat and (t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1)):
        raise ValueError(f"{name}: expected a contiguous 1-D tensor")
    if min_len is not None and (t.dim() == 0 or t.shape[0] < min_len):
        raise ValueError(f"{name}: needs at least {min_len} entries, has {t.shape[0] if t.dim() else 0}")
    return t.device


def _req_workspace(ws, name, device):
    if ws is not None:
        _req(ws, name, ws.dtype, device)
        if not ws.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")


def _desc(layout, Hq, Hkv, d, scale, split_keys, q_rs, out_rs, tree_rs, p_rs, p_hs):
    desc = dt_attn_desc()
    desc.num_seqs = layout.num_seqs
    desc.num_q_heads = Hq
    desc.num_kv_heads = Hkv
    desc.head_dim = d
    desc.softmax_scale = float(scale)
    desc.split_keys = int(split_keys)
    desc.node_offsets = _ptr(layout.node_offsets, ctypes.c_int32)
    desc.prefix_lens = _ptr(layout.prefix_lens, ctypes.c_int32)
    desc.prefix_row_start = _ptr(layout.prefix_row_start, ctypes.c_int64)
    desc.q_row_stride = q_rs
    desc.out_row_stride = out_rs
    desc.tree_row_stride = tree_rs
    desc.prefix_row_stride = p_rs
    desc.prefix_head_stride = p_hs
    return desc


def _attn_geometry(q, k_tree, k_prefix, layout, scale, split_keys):
    N, Hq, d = q.shape
    Hkv = k_tree.shape[1]
    for t, name in ((q, "q"), (k_tree, "k_tree")):
        if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != d):
            raise ValueError(f"{name}: heads must be contiguous [rows][heads][d]")
    if k_prefix is not None and (k_prefix.stride(2) != 1):
        raise ValueError("k_prefix: head_dim must be contiguous")
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    p_rs = k_prefix.stride(0) if k_prefix is not None else 0
    p_hs = k_prefix.stride(1) if k_prefix is not None else 0
    return _desc(layout, Hq, Hkv, d, scale, split_keys, _row_stride(q, Hq * d), 0, _row_stride(k_tree, Hkv * d),
                 p_rs, p_hs)


def dt_tree_attention_workspace_size(q, k_tree, k_prefix, layout, scale=None, split_keys=0):
    desc = _attn_geometry(q, k_tree, k_prefix, layout, scale, split_keys)
    n = ctypes.c_size_t(0)
    _check(_lib.load().dt_tree_attention_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "dt_tree_attention_workspace_size")
    return n.value


def _check_attention(q, k_tree, v_tree, k_prefix, v_prefix, parent, layout, out):
    """Dtypes, devices, shapes and extents of dt_tree_attention's tensors
    (out may be None); returns the device."""
    import torch

    bf = torch.bfloat16
    dev = _req(q, "q", bf)
    if q.dim() != 3 or k_tree.dim() != 3 or tuple(k_tree.shape) != tuple(v_tree.shape):
        raise ValueError("q [N, Hq, d]; k_tree and v_tree [N, Hkv, d] of one shape")
    N, Hq, d = q.shape
    if k_tree.shape[0] != N or k_tree.shape[2] != d:
        raise ValueError("k_tree/v_tree must have q's rows and head_dim")
    _req(k_tree, "k_tree", bf, dev)
    _req(v_tree, "v_tree", bf, dev)
    if int(layout.node_offsets[-1]) != N:
        raise ValueError(f"layout covers {int(layout.node_offsets[-1])} rows, q has {N}")
    _req(parent, "parent", torch.int32, dev, N, flat=True)
    if (k_prefix is None) != (v_prefix is None):
        raise ValueError("k_prefix and v_prefix are both given or both None")
    if k_prefix is not None:
        _req(k_prefix, "k_prefix", bf, dev)
        _req(v_prefix, "v_prefix", bf, dev)
        if k_prefix.dim() != 3 or tuple(k_prefix.shape) != tuple(v_prefix.shape) or \
                tuple(k_prefix.shape[1:]) != tuple(k_tree.shape[1:]):
            raise ValueError("k_prefix/v_prefix: [rows, Hkv, d] of one shape, heads and d as k_tree")
        ends = layout.prefix_row_start + layout.prefix_lens.astype(np.int64)
        if len(ends) and int(ends.max()) > k_prefix.shape[0]:
            raise ValueError(f"a prefix ends at row {int(ends.max())}, the cache has {k_prefix.shape[0]} rows")
        if k_prefix.stride() != v_prefix.stride():
            raise ValueError("k_prefix and v_prefix must share strides")
    elif (layout.prefix_lens > 0).any():
        raise ValueError("non-empty prefixes need k_prefix and v_prefix")
    if k_tree.stride() != v_tree.stride():
        raise ValueError("k_tree and v_tree must share strides")
    if out is not None:
        _req(out, "out", bf, dev)
        if tuple(out.shape) != tuple(q.shape) or out.stride(2) != 1 or (Hq > 1 and out.stride(1) != d):
            raise ValueError("out: [N, Hq, d] like q, with contiguous heads")
    return dev


def dt_tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, parent, layout, scale=None, split_keys=0,
                      out=None, workspace=None, stream=None, phase_stamps=None):
    """Ancestor-only tree attention (GPU).

    q [N, Hq, d], k_tree/v_tree [N, Hkv, d], k_prefix/v_prefix [rows, Hkv, d]
    (any row/head strides, d contiguous; may be None when every prefix is
    empty), parent int32 [N] tree-local, all torch CUDA tensors (bf16 for the
    operands). Returns out [N, Hq, d] bf16. phase_stamps (profiling, optional):
    a contiguous int64 CUDA tensor [rows, 8] that receives every workgroup's
    real-time counter stamps (the descriptor's phase_stamps).
    """
    import torch

    dev = _check_attention(q, k_tree, v_tree, k_prefix, v_prefix, parent, layout, out)
    desc = _attn_geometry(q, k_tree, k_prefix, layout, scale, split_keys)
    if phase_stamps is not None:
        _req(phase_stamps, "phase_stamps", torch.int64, dev)
        if phase_stamps.dim() != 2 or phase_stamps.shape[1] != 8 or not phase_stamps.is_contiguous():
            raise ValueError("phase_stamps: expected a contiguous [rows, 8] tensor")
        desc.phase_stamps = phase_stamps.data_ptr()
        desc.phase_stamp_rows = phase_stamps.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    _req_workspace(workspace, "workspace", dev)
    desc.out_row_stride = _row_stride(out, q.shape[1] * q.shape[2])
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    _check(lib.dt_tree_attention_workspace_size(ctypes.byref(desc), ctypes.byref(need)),
           "dt_tree_attention_workspace_size")
    if need.value and workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.dt_tree_attention(ctypes.byref(desc), q.data_ptr(), k_tree.data_ptr(), v_tree.data_ptr(),
                               k_prefix.data_ptr() if k_prefix is not None else None,
                               v_prefix.data_ptr() if v_prefix is not None else None,
                               parent.data_ptr(), out.data_ptr(), ws_ptr, ws_len, _stream(stream))
    _check(st, "dt_tree_attention")
    return out


def dt_tree_attention_noalloc(q, k_tree, v_tree, k_prefix, v_prefix, parent, layout, out, scale=None,
                              split_keys=0, stream=None):
    """dt_tree_attention without a workspace, for callers that cannot allocate
    (HIP graph capture, serving loops): the library keeps the split partials in
    a static device buffer of DT_NOALLOC_SCRATCH_BYTES per GPU. ``out`` is the
    caller's (this wrapper allocates nothing either). Calls that overlap on one
    GPU share that buffer and must be serialised by the caller."""
    if out is None:
        raise ValueError("dt_tree_attention_noalloc needs the caller's out tensor")
    _check_attention(q, k_tree, v_tree, k_prefix, v_prefix, parent, layout, out)
    desc = _attn_geometry(q, k_tree, k_prefix, layout, scale, split_keys)
    desc.out_row_stride = _row_stride(out, q.shape[1] * q.shape[2])
    st = _lib.load().dt_tree_attention_noalloc(ctypes.byref(desc), q.data_ptr(), k_tree.data_ptr(),
                                               v_tree.data_ptr(),
                                               k_prefix.data_ptr() if k_prefix is not None else None,
                                               v_prefix.data_ptr() if v_prefix is not None else None,
                                               parent.data_ptr(), out.data_ptr(), _stream(stream))
    _check(st, "dt_tree_attention_noalloc")
    return out


def dt_argmax_rows_workspace_size(rows, vocab):
    n = ctypes.c_size_t(0)
    _check(_lib.load().dt_argmax_rows_workspace_size(int(rows), int(vocab), ctypes.byref(n)),
           "dt_argmax_rows_workspace_size")
    return n.value


def dt_argmax_rows(logits, out=None, workspace=None, stream=None):
    """Per-row arg-max (lowest index on ties) of a [rows, vocab] float32 CUDA tensor
    with unit column stride. Returns int32 [rows]."""
    import torch

    dev = _req(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits: expected [rows, vocab]")
    rows, vocab = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits: vocab dimension must be contiguous")
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=dev)
    _req(out, "out", torch.int32, dev, rows, flat=True)
    _req_workspace(workspace, "workspace", dev)
    need = dt_argmax_rows_workspace_size(rows, vocab)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().dt_argmax_rows(logits.data_ptr(), rows, vocab, _row_stride(logits, vocab), out.data_ptr(), ws_ptr,
                                    ws_len, _stream(stream))
    _check(st, "dt_argmax_rows")
    return out


def dt_sample_rows_workspace_size(rows, vocab):
    n = ctypes.c_size_t(0)
    _check(_lib.load().dt_sample_rows_workspace_size(int(rows), int(vocab), ctypes.byref(n)),
           "dt_sample_rows_workspace_size")
    return n.value


def dt_sample_rows(logits, temperature, seed, offset, out=None, workspace=None, stream=None):
    """Per-row sample from softmax(logits / temperature) by Gumbel-max with
    Philox4x32-10 noise keyed by (seed, offset, row, vocabulary index), for a
    [rows, vocab] float32 CUDA tensor with unit column stride. Returns int32 [rows]."""
    import torch

    dev = _req(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits: expected [rows, vocab]")
    rows, vocab = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits: vocab dimension must be contiguous")
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=dev)
    _req(out, "out", torch.int32, dev, rows, flat=True)
    _req_workspace(workspace, "workspace", dev)
    need = dt_sample_rows_workspace_size(rows, vocab)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().dt_sample_rows(logits.data_ptr(), rows, vocab, _row_stride(logits, vocab), float(temperature),
                                    int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFFFFFFFFFF, out.data_ptr(),
                                    ws_ptr, ws_len, _stream(stream))
    _check(st, "dt_sample_rows")
    return out


def dt_accept_path(node_offsets, parent, token, argmax_idx, path=None, accept_len=None, bonus=None, stream=None):
    """Longest accepted path per tree (GPU). node_offsets: host int32 [S+1];
    parent/token/argmax_idx: int32 CUDA tensors [N]. Returns (path [N], accept_len [S], bonus [S])."""
    import torch

    offs = _i32(node_offsets)
    S = len(offs) - 1
    N = int(offs[-1]) if S >= 1 else 0
    dev = _req(parent, "parent", torch.int32, None, N, flat=True)
    _req(token, "token", torch.int32, dev, N, flat=True)
    _req(argmax_idx, "argmax_idx", torch.int32, dev, N, flat=True)
    if path is None:
        path = torch.empty(max(parent.shape[0], N), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(S, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(S, dtype=torch.int32, device=dev)
    _req(path, "path", torch.int32, dev, N, flat=True)
    _req(accept_len, "accept_len", torch.int32, dev, S, flat=True)
    _req(bonus, "bonus", torch.int32, dev, S, flat=True)
    st = _lib.load().dt_accept_path(S, _ptr(offs, ctypes.c_int32), parent.data_ptr(), token.data_ptr(),
                                    argmax_idx.data_ptr(), path.data_ptr(), accept_len.data_ptr(), bonus.data_ptr(),
                                    _stream(stream))
    _check(st, "dt_accept_path")
    return path, accept_len, bonus


class CommitArgs:
    """Marshalled arguments of dt_commit_kv, built once and reusable across
    rounds (the pointer tables and host arrays stay alive with this object).

    layout: AttnLayout (node offsets, prefix lengths before the commit, first
    cache row per sequence); cache_rows: rows of room per sequence from its
    first row; k_tree/v_tree/k_cache/v_cache: per-layer lists of bf16 CUDA
    tensors ([N, Hkv, d] trees with unit head/dim strides, caches with any row
    and head stride and unit dim stride, all layers alike); max_path: 0 or a
    bound on accepted length + 1.
    """

    def __init__(self, layout, cache_rows, k_tree, v_tree, k_cache, v_cache, max_path=0):
        L = len(k_tree)
        if not (len(v_tree) == len(k_cache) == len(v_cache) == L) or L < 1:
            raise ValueError("one tree K/V and cache K/V tensor per layer")
        import torch

        kt0, kc0 = k_tree[0], k_cache[0]
        dev = _req(kt0, "k_tree[0]", torch.bfloat16)
        for name, ts in (("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache), ("v_cache", v_cache)):
            for i, t in enumerate(ts):
                _req(t, f"{name}[{i}]", torch.bfloat16, dev)
                if t.dim() != 3:
                    raise ValueError(f"{name}[{i}]: expected [rows, Hkv, d]")
        _, Hkv, d = kt0.shape
        N = int(layout.node_offsets[-1])
        for t in list(k_tree) + list(v_tree):
            if tuple(t.shape) != tuple(kt0.shape) or t.shape[0] < N:
                raise ValueError(f"tree K/V: [N >= {N}, Hkv, d], all layers alike")
        for t in list(k_cache) + list(v_cache):
            if tuple(t.shape[1:]) != (Hkv, d):
                raise ValueError("cache K/V: [rows, Hkv, d] with the tree's heads and head_dim")
        for t in list(k_tree) + list(v_tree):
            if t.stride() != kt0.stride() or t.stride(2) != 1 or (Hkv > 1 and t.stride(1) != d):
                raise ValueError("tree K/V: [rows][heads][d] with contiguous heads, all layers alike")
        for t in list(k_cache) + list(v_cache):
            if t.stride() != kc0.stride() or t.stride(2) != 1:
                raise ValueError("cache K/V: d contiguous, all layers alike")
        self.layout = layout
        self.cache_rows = np.ascontiguousarray(cache_rows, dtype=np.int64)
        if len(self.cache_rows) != layout.num_seqs:
            raise ValueError("cache_rows needs one entry per sequence")
        ends = layout.prefix_row_start + self.cache_rows
        if len(ends) and int(ends.max()) > min(t.shape[0] for t in list(k_cache) + list(v_cache)):
            raise ValueError("a sequence's cache room ends past the cache's last row")
        self.device = dev
        self.num_nodes = N
        desc = _lib.dt_commit_desc()
        desc.num_seqs = layout.num_seqs
        desc.num_layers = L
        desc.num_kv_heads = Hkv
        desc.head_dim = d
        desc.max_path = int(max_path)
        desc.node_offsets = _ptr(layout.node_offsets, ctypes.c_int32)
        desc.prefix_lens = _ptr(layout.prefix_lens, ctypes.c_int32)
        desc.prefix_row_start = _ptr(layout.prefix_row_start, ctypes.c_int64)
        desc.cache_rows = _ptr(self.cache_rows, ctypes.c_int64)
        desc.tree_row_stride = _row_stride(kt0, Hkv * d)
        desc.cache_row_stride = kc0.stride(0)
        desc.cache_head_stride = kc0.stride(1)
        self.desc = desc
        arr = ctypes.c_void_p * L
        self.k_tree = arr(*[t.data_ptr() for t in k_tree])
        self.v_tree = arr(*[t.data_ptr() for t in v_tree])
        self.k_cache = arr(*[t.data_ptr() for t in k_cache])
        self.v_cache = arr(*[t.data_ptr() for t in v_cache])
        self._keep = (k_tree, v_tree, k_cache, v_cache)


def dt_commit_kv(args, path, accept_len, stream=None):
    """Copy every layer's accepted-path K/V rows into the cache (GPU). ``args``:
    CommitArgs; path int32 [N] and accept_len int32 [S] CUDA tensors as
    dt_accept_path leaves them."""
    import torch

    _req(path, "path", torch.int32, args.device, args.num_nodes, flat=True)
    _req(accept_len, "accept_len", torch.int32, args.device, args.layout.num_seqs, flat=True)
    st = _lib.load().dt_commit_kv(ctypes.byref(args.desc), args.k_tree, args.v_tree, args.k_cache, args.v_cache,
                                  path.data_ptr(), accept_len.data_ptr(), _stream(stream))
    _check(st, "dt_commit_kv")


def dt_topk_rows_workspace_size(rows, vocab, k):
    n = ctypes.c_size_t(0)
    _check(_lib.load().dt_topk_rows_workspace_size(int(rows), int(vocab), int(k), ctypes.byref(n)),
           "dt_topk_rows_workspace_size")
    return n.value


def dt_topk_rows(logits, k, out_token=None, out_logprob=None, workspace=None, stream=None):
    """The k best entries of every row of a [rows, vocab] float32 CUDA tensor
    (unit column stride), ordered by (logit desc, index asc), with their
    log-softmax values. Returns (tokens int32 [rows, k], logprob float32 [rows, k])."""
    import torch

    dev = _req(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits: expected [rows, vocab]")
    rows, vocab = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits: vocab dimension must be contiguous")
    if out_token is None:
        out_token = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if out_logprob is None:
        out_logprob = torch.empty((rows, k), dtype=torch.float32, device=dev)
    _req(out_token, "out_token", torch.int32, dev)
    _req(out_logprob, "out_logprob", torch.float32, dev)
    _req_workspace(workspace, "workspace", dev)
    for t in (out_token, out_logprob):
        if not t.is_contiguous() or tuple(t.shape) != (rows, k):
            raise ValueError("outputs must be contiguous [rows, k]")
    if workspace is None:
        workspace = torch.empty(max(dt_topk_rows_workspace_size(rows, vocab, k), 256), dtype=torch.uint8, device=dev)
    st = _lib.load().dt_topk_rows(logits.data_ptr(), rows, vocab, _row_stride(logits, vocab), int(k), out_token.data_ptr(),
                                  out_logprob.data_ptr(), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "dt_topk_rows")
    return out_token, out_logprob


def dt_expand_depth(parent_score, child_logq, cand_token, w, beta, out=None, stream=None):
    """One depth of the fixed-width supertree (GPU). parent_score float32 [S, w_prev]
    (any row stride), child_logq float32 [S, w_prev, k] (each sequence's block
    contiguous), cand_token int32 [S, k] (any row stride). ``out``: optional
    (sel_parent, sel_cand, sel_token, sel_score) of shape [S, w] sharing one row
    stride (e.g. views of a [S, depths, w] supertree). Returns that tuple."""
    import torch

    dev = _req(child_logq, "child_logq", torch.float32)
    if child_logq.dim() != 3 or parent_score.dim() != 2 or cand_token.dim() != 2:
        raise ValueError("parent_score [S, w_prev], child_logq [S, w_prev, k], cand_token [S, k]")
    S, w_prev, k = child_logq.shape
    _req(parent_score, "parent_score", torch.float32, dev, S)
    _req(cand_token, "cand_token", torch.int32, dev, S)
    if parent_score.shape[1] < w_prev or cand_token.shape[1] < k:
        raise ValueError("parent_score needs w_prev columns and cand_token k columns")
    if child_logq.stride(2) != 1 or (w_prev > 1 and child_logq.stride(1) != k):
        raise ValueError("child_logq: each sequence's [w_prev, k] block must be contiguous")
    for t in (parent_score, cand_token):
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError("parent_score / cand_token rows must be contiguous")
    if out is None:
        out = (torch.empty((S, w), dtype=torch.int32, device=dev), torch.empty((S, w), dtype=torch.int32, device=dev),
               torch.empty((S, w), dtype=torch.int32, device=dev), torch.empty((S, w), dtype=torch.float32, device=dev))
    for t, name, ty in zip(out, ("sel_parent", "sel_cand", "sel_token", "sel_score"),
                           (torch.int32, torch.int32, torch.int32, torch.float32)):
        _req(t, name, ty, dev, S)
        if t.dim() != 2 or t.shape[1] < w:
            raise ValueError(f"{name}: expected [S, w]")
    rs = _row_stride(out[0], w)
    if any(_row_stride(t, w) != rs or (w > 1 and t.stride(1) != 1) for t in out):
        raise ValueError("outputs must share one row stride with contiguous rows")
    st = _lib.load().dt_expand_depth(S, w_prev, k, int(w), float(beta), parent_score.data_ptr(),
                                     _row_stride(parent_score, w_prev), child_logq.data_ptr(),
                                     _row_stride(child_logq, w_prev * k), cand_token.data_ptr(),
                                     _row_stride(cand_token, k), out[0].data_ptr(), out[1].data_ptr(),
                                     out[2].data_ptr(), out[3].data_ptr(), rs, _stream(stream))
    _check(st, "dt_expand_depth")
    return out


def dt_prune_topb(sel_parent, sel_token, sel_score, root_token, budget, out=None, stream=None):
    """Deferred top-B pruning (GPU). sel_* [S, depths, w] contiguous (dt_expand_depth's
    per-depth outputs stacked), root_token int32 [S]. Returns (parent, token, depth,
    score) [S, budget + 1] and n_out [S]."""
    import torch

    dev = _req(sel_parent, "sel_parent", torch.int32)
    if sel_parent.dim() != 3:
        raise ValueError("sel_parent: expected [S, depths, w]")
    S, depths, w = sel_parent.shape
    _req(sel_token, "sel_token", torch.int32, dev)
    _req(sel_score, "sel_score", torch.float32, dev)
    _req(root_token, "root_token", torch.int32, dev, S, flat=True)
    for t in (sel_parent, sel_token, sel_score):
        if not t.is_contiguous() or tuple(t.shape) != (S, depths, w):
            raise ValueError("supertree arrays must be contiguous [S, depths, w]")
    n = int(budget) + 1
    if out is None:
        out = (torch.empty((S, n), dtype=torch.int32, device=dev), torch.empty((S, n), dtype=torch.int32, device=dev),
               torch.empty((S, n), dtype=torch.int32, device=dev), torch.empty((S, n), dtype=torch.float32, device=dev),
               torch.empty(S, dtype=torch.int32, device=dev))
    for t, name, ty in zip(out, ("parent", "token", "depth", "score", "n_out"),
                           (torch.int32, torch.int32, torch.int32, torch.float32, torch.int32)):
        _req(t, name, ty, dev, S)
        if not t.is_contiguous() or (name != "n_out" and tuple(t.shape) != (S, n)):
            raise ValueError(f"{name}: expected a contiguous [S, {n}] tensor" if name != "n_out" else
                             "n_out: expected a contiguous [S] tensor")
    st = _lib.load().dt_prune_topb(S, depths, w, int(budget), sel_parent.data_ptr(), sel_token.data_ptr(),
                                   sel_score.data_ptr(), root_token.data_ptr(), *[t.data_ptr() for t in out],
                                   _stream(stream))
    _check(st, "dt_prune_topb")
    return out
