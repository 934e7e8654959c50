"""Benchmark: one draft-tree verification round per step, on one MI355X.

A step runs the whole verification path over one synthetic round:
  1. dt_build_tree      best-first tree from this round's per-depth candidates (host)
  2. upload parent/token (pinned host -> HBM, async)
  3. dt_tree_attention  x L layers, each with its own KV cache
  4. dt_argmax_rows     greedy prediction at every node over the full vocabulary
                        (dt_sample_rows instead with --temperature T > 0)
  5. dt_accept_path     accepted path, length and bonus token
  6. dt_commit_kv       only with --commit: the accepted rows into every layer's cache
Inputs (KV caches, Q/K/V of the tree, logits) are resident in HBM before the
timed region; only the tree itself is built per step, as a round would. After
the timed steps the T = 1 target-sampling kernel and the KV commit are timed on
their own as well (fields "sample" and "commit").

Default workload: Qwen3-4B-shaped target (32 query heads, 8 KV heads, head dim
128, 36 layers, vocabulary 151936), one sequence with an 8192-token verified
prefix and a 256-node tree. Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify TFLOP/s + % MFMA/HBM roofline; us per round at B=256"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
N_TABLES = 4  # distinct draft-candidate tables cycled through the steps


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="round", help="gen.configs name (round, b128, b256, chain16, ragged, long)")
    ap.add_argument("--layers", type=int, default=0,
                    help="independent per-layer KV caches the step cycles through (0: the workload's own; "
                         "enough of them keep one workload's caches out of the 256 MB last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the attention-only timings of the b128, ragged and long workloads")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="0: greedy verification (dt_argmax_rows); > 0: exact target-sample matching (dt_sample_rows)")
    ap.add_argument("--commit", action="store_true", help="commit the accepted K/V rows in every step")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="print the forward kernel's per-workgroup phase stamps for the workload and exit")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (a known-size reference "
                         "for hardware byte counters)")
    return ap.parse_args()


class Round:
    """Device-resident inputs of one workload and the launches of one step."""

    def __init__(self, w, device, temperature=0.0, commit=False):
        import torch

        import draft_tree_verification_dt_amd as dt
        from gen import draft as gdraft, rng as grng, tensors as gten

        self.w, self.dt, self.torch = w, dt, torch
        self.dev = device
        self.temperature, self.do_commit = float(temperature), bool(commit)
        S, Hq, Hkv, d, L = w.num_seqs, w.Hq, w.Hkv, w.d, w.layers
        N, CR = w.total_nodes, w.total_cache_rows
        sc = 1.0 / np.sqrt(d)
        self.offs = w.node_offsets()
        # each sequence's cache keeps room for its tree after the prefix (rows a commit writes)
        self.starts = w.cache_row_starts()
        self.layout = dt.AttnLayout(self.offs, w.prefix_lens, self.starts)
        # per-layer operands; every layer has its own KV cache
        self.kp = [gten.device_randn_bf16((CR, Hkv, d), w.seed, "kp", l, scale=sc) for l in range(L)]
        self.vp = [gten.device_randn_bf16((CR, Hkv, d), w.seed, "vp", l, scale=sc) for l in range(L)]
        self.q = [gten.device_randn_bf16((N, Hq, d), w.seed, "q", l, scale=sc) for l in range(L)]
        self.kt = [gten.device_randn_bf16((N, Hkv, d), w.seed, "kt", l, scale=sc) for l in range(L)]
        self.vt = [gten.device_randn_bf16((N, Hkv, d), w.seed, "vt", l, scale=sc) for l in range(L)]
        self.out = [torch.empty((N, Hq, d), dtype=torch.bfloat16, device=device) for _ in range(L)]

        # per-round draft candidates (host) and the planted target logits that go with them
        self.tables = []
        self.logits = []
        self.trees = []
        for t in range(N_TABLES):
            per_seq = []
            for s, n in enumerate(w.nodes):
                r = grng.stream(w.seed, "cand", t, s)
                lp, tok = gdraft.candidates(r, depths=w.depths, vocab=w.vocab, k=w.cand_k(n))
                per_seq.append((lp, tok, int(r.integers(0, w.vocab)), n))
            self.tables.append(per_seq)
            trees = [dt.dt_build_tree(lp, tok, root, n, with_score=False) for lp, tok, root, n in per_seq]
            self.trees.append(trees)
            lg = gten.device_logits(N, w.vocab, w.seed, "logits", t)
            for s, (p, tk, _, _) in enumerate(trees):
                gten.device_plant(grng.stream(w.seed, "plant", t, s), lg, int(self.offs[s]), p, tk, p=w.plant_p)
            self.logits.append(lg)

        # tree upload buffers (pinned host, double-buffered) and device copies
        self.h_tree = [torch.empty((2, N), dtype=torch.int32).pin_memory() for _ in range(2)]
        self.d_tree = torch.empty((2, N), dtype=torch.int32, device=device)
        self.am = torch.empty(N, dtype=torch.int32, device=device)
        self.path = torch.empty(N, dtype=torch.int32, device=device)
        self.acc = torch.empty(S, dtype=torch.int32, device=device)
        self.bonus = torch.empty(S, dtype=torch.int32, device=device)
        ws_att = dt.dt_tree_attention_workspace_size(self.q[0], self.kt[0], self.kp[0], self.layout)
        self.ws_att = torch.empty(max(ws_att, 256), dtype=torch.uint8, device=device)
        ws_am = max(dt.dt_argmax_rows_workspace_size(N, w.vocab), dt.dt_sample_rows_workspace_size(N, w.vocab))
        self.ws_am = torch.empty(max(ws_am, 256), dtype=torch.uint8, device=device)  # greedy and sampled scans
        self.upload_done = [None, None]
        self.commit_args = dt.CommitArgs(self.layout, np.asarray(w.prefix_lens) + np.asarray(w.nodes), self.kt,
                                         self.vt, self.kp, self.vp, max_path=w.depths + 1)
        self.sample_seed = 0x5EED_0000 + w.seed
        self._prepare_raw_calls()
        self.step_idx = 0

    def _prepare_raw_calls(self):
        """Marshal the per-layer C-ABI arguments once (the timed loop then only
        issues the calls)."""
        import ctypes

        from draft_tree_verification_dt_amd import _lib

        dt, w = self.dt, self.w
        self.lib = _lib.load()
        self.desc = dt._attn_geometry(self.q[0], self.kt[0], self.kp[0], self.layout, None, 0)
        self.desc.out_row_stride = self.out[0].stride(0)
        self.desc_ref = ctypes.byref(self.desc)
        self.stream = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        self.att_args = [(self.q[l].data_ptr(), self.kt[l].data_ptr(), self.vt[l].data_ptr(), self.kp[l].data_ptr(),
                          self.vp[l].data_ptr(), self.d_tree[0].data_ptr(), self.out[l].data_ptr(),
                          self.ws_att.data_ptr(), self.ws_att.numel()) for l in range(w.layers)]
        self.offs_c = np.ascontiguousarray(self.offs, dtype=np.int32)
        self.offs_ptr = self.offs_c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def build_and_upload(self):
        t = self.step_idx % N_TABLES
        slot = self.step_idx % 2
        if self.upload_done[slot] is not None:
            self.upload_done[slot].synchronize()  # the pinned slot's previous copy has finished
        h = self.h_tree[slot]
        for s, (lp, tok, root, n) in enumerate(self.tables[t]):
            p, tk, _, _ = self.dt.dt_build_tree(lp, tok, root, n, with_score=False)
            a = int(self.offs[s])
            h[0, a:a + n] = self.torch.from_numpy(p)
            h[1, a:a + n] = self.torch.from_numpy(tk)
        self.d_tree.copy_(h, non_blocking=True)
        ev = self.torch.cuda.Event()
        ev.record()
        self.upload_done[slot] = ev
        return t

    def attention(self, l):
        st = self.lib.dt_tree_attention(self.desc_ref, *self.att_args[l], self.stream)
        if st != 0:
            raise self.dt.DtError(st, "dt_tree_attention")

    def step(self, events=None):
        """One round. `events` (start, end), if given, bracket the round's
        attention calls on the stream they run on."""
        t = self.build_and_upload()
        self.device_part(t, events)
        self.advance()

    def device_part(self, t, events=None):
        """The round's GPU calls for candidate table t (the tree already on the device)."""
        if events is not None:
            events[0].record()
        for l in range(self.w.layers):
            self.attention(l)
        if events is not None:
            events[1].record()
        lg = self.logits[t]
        if self.temperature > 0:
            self.sample(lg, self.step_idx)
        else:
            st = self.lib.dt_argmax_rows(lg.data_ptr(), lg.shape[0], lg.shape[1], lg.stride(0), self.am.data_ptr(),
                                         self.ws_am.data_ptr(), self.ws_am.numel(), self.stream)
            if st != 0:
                raise self.dt.DtError(st, "dt_argmax_rows")
        st = self.lib.dt_accept_path(self.w.num_seqs, self.offs_ptr, self.d_tree[0].data_ptr(),
                                     self.d_tree[1].data_ptr(), self.am.data_ptr(), self.path.data_ptr(),
                                     self.acc.data_ptr(), self.bonus.data_ptr(), self.stream)
        if st != 0:
            raise self.dt.DtError(st, "dt_accept_path")
        if self.do_commit:
            self.commit()

    def advance(self):
        self.step_idx += 1

    def sample(self, lg, offset, temperature=None):
        """Target samples of every node into self.am (the round's offset keys the draws)."""
        T = self.temperature if temperature is None else temperature
        st = self.lib.dt_sample_rows(lg.data_ptr(), lg.shape[0], lg.shape[1], lg.stride(0), T, self.sample_seed,
                                     offset, self.am.data_ptr(), self.ws_am.data_ptr(), self.ws_am.numel(), self.stream)
        if st != 0:
            raise self.dt.DtError(st, "dt_sample_rows")

    def commit(self):
        import ctypes

        a = self.commit_args
        st = self.lib.dt_commit_kv(ctypes.byref(a.desc), a.k_tree, a.v_tree, a.k_cache, a.v_cache,
                                   self.path.data_ptr(), self.acc.data_ptr(), self.stream)
        if st != 0:
            raise self.dt.DtError(st, "dt_commit_kv")

    def attention_flops(self, table):
        """Algorithmic flops of one layer for the trees of `table` (ancestor pairs only)."""
        from oracle.attention import flops

        return flops(self.w.nodes, self.w.prefix_lens, [p for p, _, _, _ in self.trees[table]], self.w.Hq, self.w.d)


def attention_bytes(w):
    """Algorithmic bytes of one call: prefix K and V once, plus per node Q, O,
    tree K and V, and the parent index."""
    kv = sum(2 * P * w.Hkv * w.d * 2 for P in w.prefix_lens)
    per_node = 2 * w.Hq * w.d * 2 + 2 * w.Hkv * w.d * 2 + 4
    return int(kv + w.total_nodes * per_node)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tree_attn_hbm_traffic.json")


def recorded_traffic(w):
    """HBM bytes per dt_tree_attention call measured with the FETCH_SIZE and
    WRITE_SIZE counters (profiles/), valid only for the attention source they
    were taken on and for this workload."""
    import hashlib

    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = os.path.join(ROOT, "draft_tree_verification_dt_amd", "csrc", "attention.hip")
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(w.name)
    if rec.get("attention_source_sha256") != digest or entry is None:
        return None
    return {"bytes_per_launch": entry["bytes_per_launch"], "source": os.path.relpath(TRAFFIC_FILE, ROOT)}


def tree_shape(rnd):
    """Realized shape of the round's trees (the candidate tables cap the depth at
    the number of draft positions; the best-first order decides how deep the
    trees actually grow): node-depth histogram summed over all tables and
    sequences, and the deepest node."""
    hist = {}
    for trees in rnd.trees:
        for _, _, depth, _ in trees:
            for dd, c in zip(*np.unique(depth, return_counts=True)):
                hist[int(dd)] = hist.get(int(dd), 0) + int(c)
    return {"depth_hist": [hist.get(i, 0) for i in range(max(hist) + 1)], "max_depth": max(hist),
            "tables": len(rnd.trees)}


def time_round_graph(rnd, reps=5):
    """The round's GPU calls (36 attention calls, the row scan, the walk, and the
    commit when the step has it) captured in one HIP graph and replayed: the
    device-side time of a round without host launch overhead."""
    torch = rnd.torch
    rnd.device_part(0)
    torch.cuda.synchronize()
    import ctypes

    graph = torch.cuda.CUDAGraph()
    saved = rnd.stream
    with torch.cuda.graph(graph):
        rnd.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # the capturing stream
        rnd.device_part(0)
    rnd.stream = saved
    graph.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def time_on_stream(rnd, fn, reps):
    """Mean GPU time of fn() in ms, from HIP events recorded around it on the
    library's stream. Two attention calls are queued ahead of each start event,
    so the host has enqueued the events and fn's kernels before the GPU reaches
    them: the interval is GPU execution, not host launch latency. One untimed
    call comes first."""
    torch = rnd.torch
    fn(0)  # the first launch of a kernel also loads its code object
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        rnd.attention(0)
        rnd.attention(1 % rnd.w.layers)
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def time_back_to_back(rnd, fn, reps, ahead=2):
    """Mean GPU time of fn() in ms over `reps` consecutive calls bracketed by
    one pair of HIP events on the library's stream (the method of the
    attention calls' launch_us_mean): the kernels' own rate, without the gap
    that an event pair around a single call adds. `ahead` attention calls are
    queued ahead of the start event, so that the host has enqueued every timed
    call before the GPU reaches them (more for calls through the Python
    binding, whose host time exceeds a small kernel's); one untimed call comes
    first."""
    torch = rnd.torch
    fn(0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for l in range(ahead):
        rnd.attention(l % rnd.w.layers)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def argmax_call(rnd):
    def call(i):
        lg = rnd.logits[i % N_TABLES]
        st = rnd.lib.dt_argmax_rows(lg.data_ptr(), lg.shape[0], lg.shape[1], lg.stride(0), rnd.am.data_ptr(),
                                    rnd.ws_am.data_ptr(), rnd.ws_am.numel(), rnd.stream)
        if st != 0:
            raise rnd.dt.DtError(st, "dt_argmax_rows")

    return call


def time_argmax_calls(rnd, reps):
    def call(i):
        lg = rnd.logits[i % N_TABLES]
        st = rnd.lib.dt_argmax_rows(lg.data_ptr(), lg.shape[0], lg.shape[1], lg.stride(0), rnd.am.data_ptr(),
                                    rnd.ws_am.data_ptr(), rnd.ws_am.numel(), rnd.stream)
        if st != 0:
            raise rnd.dt.DtError(st, "dt_argmax_rows")

    return time_on_stream(rnd, call, reps)


def time_sample_calls(rnd, reps, temperature=1.0):
    return time_on_stream(rnd, lambda i: rnd.sample(rnd.logits[i % N_TABLES], 1000 + i, temperature), reps)


def time_commit_calls(rnd, reps):
    """dt_commit_kv over every layer for the accepted paths the last step left on the device."""
    ms = time_on_stream(rnd, lambda i: rnd.commit(), reps)
    acc = rnd.acc.cpu().numpy()
    w = rnd.w
    moved = int(2 * 2 * (acc + 1).sum() * w.Hkv * w.d * 2 * w.layers)  # read + write of K and V rows
    return ms, moved, acc


def time_small_tree(rnd, reps=40, n=16):
    """dt_tree_attention for an n-node chain (parent[i] = i - 1) over the first
    sequence's own prefix, one call per layer cache in turn (so the caches rotate
    through 36 x 34 MB): the small-tree case, bound by streaming the prefix K/V
    from HBM. Mean call time in ms from HIP events on the library's stream, the
    call's algorithmic bytes and flops."""
    import ctypes

    torch, dt, w = rnd.torch, rnd.dt, rnd.w
    from gen import tensors as gten

    P, Hq, Hkv, d = w.prefix_lens[0], w.Hq, w.Hkv, w.d
    sc = 1.0 / np.sqrt(d)
    q = gten.device_randn_bf16((n, Hq, d), w.seed, "chain-q", scale=sc)
    kt = gten.device_randn_bf16((n, Hkv, d), w.seed, "chain-kt", scale=sc)
    vt = gten.device_randn_bf16((n, Hkv, d), w.seed, "chain-vt", scale=sc)
    par = torch.arange(-1, n - 1, dtype=torch.int32, device=rnd.dev)
    out = torch.empty((n, Hq, d), dtype=torch.bfloat16, device=rnd.dev)
    layout = dt.AttnLayout([0, n], [P], [int(rnd.starts[0])])
    desc = dt._attn_geometry(q, kt, rnd.kp[0], layout, None, 0)
    ws_n = dt.dt_tree_attention_workspace_size(q, kt, rnd.kp[0], layout)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=rnd.dev)
    dref = ctypes.byref(desc)

    def call(i):
        l = i % w.layers
        st = rnd.lib.dt_tree_attention(dref, q.data_ptr(), kt.data_ptr(), vt.data_ptr(), rnd.kp[l].data_ptr(),
                                       rnd.vp[l].data_ptr(), par.data_ptr(), out.data_ptr(), ws.data_ptr(),
                                       ws.numel(), rnd.stream)
        if st != 0:
            raise dt.DtError(st, "dt_tree_attention")

    ms = time_on_stream(rnd, call, reps)
    ms_b2b = time_back_to_back(rnd, call, reps)
    nbytes = 2 * P * Hkv * d * 2 + n * (2 * Hq * d * 2 + 2 * Hkv * d * 2 + 4)
    flops = 4.0 * d * Hq * (n * P + n * (n + 1) // 2)
    return ms, ms_b2b, nbytes, flops


def time_stream_floor(rnd, nbytes, tables=10, reps=40):
    """The practical floor of one kernel that streams `nbytes` from HBM: the
    library's arg-max scan over a [256, nbytes / 1024] fp32 table (one
    workgroup per row, nothing but loads and compares), rotating through
    `tables` tables (more bytes than the 256 MB last-level cache holds), timed
    as a single call and back to back like the small-tree call."""
    torch = rnd.torch
    cols = nbytes // (256 * 4) // 4 * 4
    tabs = [torch.randn((256, cols), device=rnd.dev, dtype=torch.float32) for _ in range(tables)]
    out = torch.empty(256, dtype=torch.int32, device=rnd.dev)

    def call(i):
        lg = tabs[i % tables]
        st = rnd.lib.dt_argmax_rows(lg.data_ptr(), 256, cols, cols, out.data_ptr(), None, 0, rnd.stream)
        if st != 0:
            raise rnd.dt.DtError(st, "dt_argmax_rows")

    single = time_on_stream(rnd, call, reps)
    b2b = time_back_to_back(rnd, call, reps)
    del tabs
    return single, b2b, 256 * cols * 4


OTHER_WORKLOADS = (("b128", 40), ("ragged", 6), ("long", 3))  # (workload, rotating layer caches)


def time_attention_workload(rnd, name, layers, reps=3):
    """dt_tree_attention alone on another workload's geometry: its own trees
    (best-first over its candidate tables), operands drawn on the device, and
    `layers` independent KV caches that the calls rotate through so that the
    prefix streams from HBM. Mean call time from one pair of HIP events around
    reps x layers calls on the library's stream (two round calls are queued
    ahead so the host has enqueued the calls before the GPU reaches them); the
    roofline object of that call."""
    import ctypes

    from gen import configs as gconf, draft as gdraft, rng as grng, tensors as gten
    from oracle.attention import flops as att_flops

    torch, dt = rnd.torch, rnd.dt
    w = gconf.get(name)
    w.layers = layers
    N, CR, Hq, Hkv, d = w.total_nodes, w.total_cache_rows, w.Hq, w.Hkv, w.d
    sc = 1.0 / np.sqrt(d)
    parents = []
    for s, n in enumerate(w.nodes):
        r = grng.stream(w.seed, "cand", 0, s)
        lp, tok = gdraft.candidates(r, depths=w.depths, vocab=w.vocab, k=w.cand_k(n))
        parents.append(dt.dt_build_tree(lp, tok, int(r.integers(0, w.vocab)), n, with_score=False)[0])
    par = torch.from_numpy(np.concatenate(parents).astype(np.int32)).to(rnd.dev)
    layout = dt.AttnLayout(w.node_offsets(), w.prefix_lens, w.cache_row_starts())
    kp = [gten.device_randn_bf16((CR, Hkv, d), w.seed, "kp", l, scale=sc) for l in range(layers)]
    vp = [gten.device_randn_bf16((CR, Hkv, d), w.seed, "vp", l, scale=sc) for l in range(layers)]
    q = [gten.device_randn_bf16((N, Hq, d), w.seed, "q", l, scale=sc) for l in range(layers)]
    kt = [gten.device_randn_bf16((N, Hkv, d), w.seed, "kt", l, scale=sc) for l in range(layers)]
    vt = [gten.device_randn_bf16((N, Hkv, d), w.seed, "vt", l, scale=sc) for l in range(layers)]
    out = torch.empty((N, Hq, d), dtype=torch.bfloat16, device=rnd.dev)
    desc = dt._attn_geometry(q[0], kt[0], kp[0], layout, None, 0)
    desc.out_row_stride = out.stride(0)
    ws = torch.empty(max(dt.dt_tree_attention_workspace_size(q[0], kt[0], kp[0], layout), 256), dtype=torch.uint8,
                     device=rnd.dev)
    dref = ctypes.byref(desc)

    def call(l):
        st = rnd.lib.dt_tree_attention(dref, q[l].data_ptr(), kt[l].data_ptr(), vt[l].data_ptr(), kp[l].data_ptr(),
                                       vp[l].data_ptr(), par.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                       rnd.stream)
        if st != 0:
            raise dt.DtError(st, "dt_tree_attention")

    for l in range(layers):
        call(l)  # first touch of every cache, and the code object
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rnd.attention(0)
    rnd.attention(1 % rnd.w.layers)
    a.record()
    for i in range(reps * layers):
        call(i % layers)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * layers)
    fl = float(att_flops(w.nodes, w.prefix_lens, parents, Hq, d))
    nbytes = attention_bytes(w)
    res = {"workload": w.name, "num_seqs": w.num_seqs, "tree_nodes": w.nodes[0] if len(set(w.nodes)) == 1 else w.nodes,
           "prefix_lens": w.prefix_lens, "us": round(ms * 1e3, 2), "calls_timed": reps * layers,
           "layer_caches": layers, "flops_per_launch": fl, "algorithmic_bytes_per_launch": nbytes}
    if fl / nbytes >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        tf = fl / (ms / 1e3) / 1e12
        res.update({"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
    else:
        gbs = nbytes / (ms / 1e3) / 1e9
        res.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)})
    del kp, vp, q, kt, vt
    torch.cuda.empty_cache()
    return res


class DraftBuild:
    """DARTree's construction kernels at the pages' pruned configuration: gamma = 16
    draft positions over the vocabulary, K = 64 candidates, width W = 12, beta =
    -0.2, budget B = 64. The correction head is a trained network outside this
    library; its log q~ inputs here are fixed seeded values of the right shape
    (the kernels' work does not depend on them)."""

    GAMMA, K, W, BETA, B = 16, 64, 12, -0.2, 64

    def __init__(self, w, device):
        import torch

        from gen import tensors as gten

        import draft_tree_verification_dt_amd as dtm

        self.dt, self.torch = dtm, torch
        g, K, W = self.GAMMA, self.K, self.W
        self.base = gten.device_logits(g, w.vocab, w.seed, "draft-base")
        self.ws = torch.empty(max(dtm.dt_topk_rows_workspace_size(g, w.vocab, K), 256), dtype=torch.uint8,
                              device=device)
        self.tok = torch.empty((g, K), dtype=torch.int32, device=device)
        self.lp = torch.empty((g, K), dtype=torch.float32, device=device)
        gen = torch.Generator(device=device)
        gen.manual_seed(w.seed)
        self.logq = torch.log_softmax(torch.randn((g, W, K), generator=gen, device=device) * 2, dim=-1)
        self.root_score = torch.zeros((1, 1), dtype=torch.float32, device=device)
        self.par = torch.full((1, g, W), -1, dtype=torch.int32, device=device)
        self.cand = torch.full((1, g, W), -1, dtype=torch.int32, device=device)
        self.stok = torch.full((1, g, W), -1, dtype=torch.int32, device=device)
        self.ssc = torch.full((1, g, W), float("-inf"), dtype=torch.float32, device=device)
        self.root_tok = torch.zeros(1, dtype=torch.int32, device=device)
        self.tree = [torch.empty((1, self.B + 1), dtype=dt_, device=device)
                     for dt_ in (torch.int32, torch.int32, torch.int32, torch.float32)] + \
                    [torch.empty(1, dtype=torch.int32, device=device)]

    def topk(self):
        self.dt.dt_topk_rows(self.base, self.K, out_token=self.tok, out_logprob=self.lp, workspace=self.ws)

    def expand(self, d):
        prev = self.root_score if d == 0 else self.ssc[:, d - 1]
        lq = self.logq[d:d + 1, :1] if d == 0 else self.logq[d:d + 1]
        self.dt.dt_expand_depth(prev, lq, self.tok[d:d + 1], self.W, self.BETA,
                                out=(self.par[:, d], self.cand[:, d], self.stok[:, d], self.ssc[:, d]))

    def prune(self):
        self.dt.dt_prune_topb(self.par, self.stok, self.ssc, self.root_tok, self.B, out=tuple(self.tree))

    def chain(self):
        self.topk()
        for d in range(self.GAMMA):
            self.expand(d)
        self.prune()


def phase_stamps(rnd, reps=24, rows=8192):
    """Per-workgroup phase stamps (the descriptor's phase_stamps: the GPU's
    100 MHz real-time counter at fixed points of every workgroup of the forward
    and merge kernels) over `reps` consecutive calls that rotate through the
    layer caches. Per call, times are taken from that call's first forward
    workgroup entry: for each forward phase the median over the calls of the
    median, minimum and maximum over workgroups; the merge kernel's first entry
    and last store; and the gaps at the kernel boundaries (last forward store to
    first merge entry, last merge store to the next call's first entry), in µs."""
    import ctypes

    torch, w = rnd.torch, rnd.w
    bufs = torch.zeros((reps, rows, 8), dtype=torch.int64, device=rnd.dev)
    descs = []
    for i in range(reps):
        d = type(rnd.desc).from_buffer_copy(rnd.desc)
        d.phase_stamps = bufs[i].data_ptr()
        d.phase_stamp_rows = rows
        descs.append(d)
    torch.cuda.synchronize()
    for i in range(reps):
        st = rnd.lib.dt_tree_attention(ctypes.byref(descs[i]), *rnd.att_args[i % w.layers], rnd.stream)
        if st != 0:
            raise rnd.dt.DtError(st, "dt_tree_attention")
    torch.cuda.synchronize()
    s = bufs.cpu().numpy()
    names = ["entry", "first_stage_requested", "setup_done", "first_stage_landed", "main_loop_done", "stored"]
    per = {k: {"median": [], "min": [], "max": []} for k in names}
    merge = {"first_entry": [], "last_stored": []}
    gaps = {"forward_to_merge": [], "merge_to_next_call": [], "call_period": []}
    wgs, mbs, spans = [], [], []
    for i in range(reps):
        f = s[i][(s[i][:, 7] == 1) & (s[i][:, 5] != 0)]  # forward workgroups that stored outputs
        m = s[i][(s[i][:, 7] == 2) & (s[i][:, 5] != 0)]  # merge blocks that stored outputs
        wgs.append(len(f))
        mbs.append(len(m))
        t0 = s[i][s[i][:, 7] == 1][:, 0].min()
        for k, name in enumerate(names):
            v = (f[:, k][f[:, k] != 0] - t0) / 100.0
            per[name]["median"].append(np.median(v))
            per[name]["min"].append(v.min())
            per[name]["max"].append(v.max())
        end = f[:, 5].max()
        if len(m):
            merge["first_entry"].append((m[:, 0].min() - t0) / 100.0)
            merge["last_stored"].append((m[:, 5].max() - t0) / 100.0)
            gaps["forward_to_merge"].append((m[:, 0].min() - f[:, 5].max()) / 100.0)
            end = m[:, 5].max()
        if i + 1 < reps:
            t1 = s[i + 1][s[i + 1][:, 7] == 1][:, 0].min()
            gaps["merge_to_next_call"].append((t1 - end) / 100.0)
            gaps["call_period"].append((t1 - t0) / 100.0)
    med = lambda x: round(float(np.median(x)), 2) if len(x) else None
    return {"workload": w.name, "calls": reps, "forward_workgroups": int(np.median(wgs)),
            "merge_blocks": int(np.median(mbs)),
            "clock": "s_memrealtime, 100 MHz; µs after the call's first forward workgroup entry",
            "forward_phases_us": {k: {m_: med(x) for m_, x in v.items()} for k, v in per.items()},
            "merge_us": {k: med(v) for k, v in merge.items()},
            "gaps_us": {k: med(v) for k, v in gaps.items()}}


def time_draft_build(rnd, reps=10):
    db = DraftBuild(rnd.w, rnd.dev)
    topk_ms = time_on_stream(rnd, lambda i: db.topk(), reps)
    topk_b2b = time_back_to_back(rnd, lambda i: db.topk(), 20, ahead=16)
    db.chain()  # every layer filled, so each timed expansion selects from real scores
    exp_ms = time_on_stream(rnd, lambda i: db.expand(1 + i % (db.GAMMA - 1)), reps)
    exp_b2b = time_back_to_back(rnd, lambda i: db.expand(1 + i % (db.GAMMA - 1)), 20, ahead=16)
    prune_ms = time_on_stream(rnd, lambda i: db.prune(), reps)
    prune_b2b = time_back_to_back(rnd, lambda i: db.prune(), 20, ahead=16)
    chain_ms = time_on_stream(rnd, lambda i: db.chain(), reps)
    # the same chain from one HIP graph: no host launch gaps between its 18 kernels
    torch = rnd.torch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        db.chain()
    graph_ms = time_on_stream(rnd, lambda i: graph.replay(), reps)
    n_out = int(db.tree[4].cpu()[0])
    depth = db.tree[2].cpu().numpy()[0, :n_out]
    topk_bytes = db.GAMMA * rnd.w.vocab * 4
    return db, {"config": f"gamma {db.GAMMA}, vocab {rnd.w.vocab}, K {db.K}, W {db.W}, beta {db.BETA}, B {db.B}",
            "timing": "single call between an event pair (topk_us, expand_us, prune_us); consecutive calls "
                      "(*_us_back_to_back); the chain call by call and replayed from one HIP graph",
            "topk_us": topk_ms * 1e3, "topk_GB/s": topk_bytes / (topk_ms / 1e3) / 1e9,
            "topk_us_back_to_back": topk_b2b * 1e3,
            "expand_us": exp_ms * 1e3, "expand_us_back_to_back": exp_b2b * 1e3,
            "prune_us": prune_ms * 1e3, "prune_us_back_to_back": prune_b2b * 1e3,
            "chain_us": chain_ms * 1e3, "chain_graph_us": graph_ms * 1e3, "tree_nodes": n_out,
            "tree_max_depth": int(depth.max())}


def reference_outputs(rnd, t1_offset):
    """One more (untimed) round on candidate table 0 whose outputs the CPU
    baseline leg checks: every layer's attention, the greedy tokens, the walk,
    the T = 1 samples of the same logits, and the commit of the accepted rows."""
    torch = rnd.torch
    rnd.step_idx = (rnd.step_idx // N_TABLES + 1) * N_TABLES  # next step uses table 0
    saved = rnd.temperature, rnd.do_commit
    rnd.temperature, rnd.do_commit = 0.0, False
    rnd.step()
    rnd.temperature, rnd.do_commit = saved
    torch.cuda.synchronize()
    ref = {"am": rnd.am.cpu().numpy(), "acc": rnd.acc.cpu().numpy(), "bonus": rnd.bonus.cpu().numpy(),
           "path": rnd.path.cpu().numpy()}
    rnd.sample(rnd.logits[0], t1_offset, 1.0)
    torch.cuda.synchronize()
    ref["t1"] = rnd.am.cpu().numpy()
    before = (rnd.kp[0].clone(), rnd.vp[0].clone())
    rnd.commit()
    torch.cuda.synchronize()
    ref["commit_layer0"] = (before, (rnd.kp[0], rnd.vp[0]))
    return ref


def draft_oracle(db):
    """The oracle's DARTree construction over the bench's draft inputs (the same
    base logits and stand-in log q~), timed, and compared with the GPU's last
    chain (topk, 16 expansions, prune) node for node."""
    from oracle import dartree as odt

    torch = db.torch
    db.chain()
    torch.cuda.synchronize()
    base = db.base.cpu().numpy()
    logq = db.logq.cpu().numpy()
    t0 = time.perf_counter()
    ctok, _ = odt.topk_logprobs(base, db.K)
    heads = [(lambda d: (lambda paths: logq[d][:len(paths)]))(d) for d in range(db.GAMMA)]
    layers = odt.build_supertree(heads, db.BETA, db.W)
    kept = odt.prune_topb(layers, db.B)
    parent, token, depth, _ = odt.tree_arrays(layers, kept, ctok)
    seconds = time.perf_counter() - t0
    token[0] = int(db.root_tok.cpu()[0])
    n = int(db.tree[4].cpu()[0])
    ok = (np.array_equal(db.tok.cpu().numpy(), ctok) and n == len(kept) and
          np.array_equal(db.tree[0].cpu().numpy()[0, :n], parent) and
          np.array_equal(db.tree[1].cpu().numpy()[0, :n], token) and
          np.array_equal(db.tree[2].cpu().numpy()[0, :n], depth))
    return seconds, bool(ok)


def cpu_baseline(rnd, budget_s, ref, t1_offset, db=None):
    """The oracle, as it is, on this host's cores: a bounded sample of the same
    round (some of the layers' attention, plus argmax, walk and tree build),
    scaled to a full round. Its outputs are compared with the GPU's outputs of
    the same round (`ref`), which gives the parity record."""
    from oracle import argmax as oarg, attention as oatt, build_tree as obt, commit as ocommit, sample as osmp
    from oracle import walk as owalk

    w, torch = rnd.w, rnd.torch
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    f = lambda x: x.float().cpu().numpy()  # noqa: E731
    t = 0
    t0 = time.perf_counter()
    trees = [obt.build_tree_heap(lp, tok, root, n) for lp, tok, root, n in rnd.tables[t]]
    t_build = time.perf_counter() - t0
    build_ok = all(list(a[0]) == list(b[0]) and list(a[1]) == list(b[1]) for a, b in zip(trees, rnd.trees[t]))
    parents = [np.array(x[0]) for x in trees]
    layer_times = []
    spent = 0.0
    worst_abs, worst_rel = 0.0, 0.0
    for l in range(w.layers):
        args = [f(x[l]) for x in (rnd.q, rnd.kt, rnd.vt, rnd.kp, rnd.vp)]
        t0 = time.perf_counter()
        o = oatt.batch_tree_attention(*args, np.concatenate(parents), rnd.offs, w.prefix_lens, rnd.starts)
        layer_times.append(time.perf_counter() - t0)
        spent += layer_times[-1]
        got = rnd.out[l].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - o)
        worst_abs = max(worst_abs, float(err.max()))
        worst_rel = max(worst_rel, float((err.max(-1) / np.maximum(np.abs(o).max(-1), 1e-30)).max()))
        if spent > budget_s and len(layer_times) >= 1:
            break
    lg = rnd.logits[t].cpu().numpy()
    t0 = time.perf_counter()
    am = oarg.argmax_rows(lg)
    t_arg = time.perf_counter() - t0
    t0 = time.perf_counter()
    walks = owalk.batch_accept_path(np.concatenate(parents), np.concatenate([x[1] for x in trees]), am, rnd.offs)
    t_walk = time.perf_counter() - t0
    walk_ok = all(int(ref["acc"][s]) == L and int(ref["bonus"][s]) == bo and
                  list(ref["path"][rnd.offs[s]:rnd.offs[s] + L + 1]) == pth for s, (pth, L, bo) in enumerate(walks))
    # T = 1: the oracle's Gumbel-max over the same logits and stream; a mismatch must be a near tie in fp32
    ids = np.unique(np.linspace(0, lg.shape[0] - 1, min(lg.shape[0], 256)).astype(np.int64))
    t0 = time.perf_counter()
    scores = np.concatenate([osmp.perturbed_scores(lg[ids[i:i + 32]], 1.0, ids[i:i + 32], rnd.sample_seed, t1_offset)
                             for i in range(0, len(ids), 32)])
    smp = np.argmax(scores, axis=1)
    t_smp = time.perf_counter() - t0
    gpu = ref["t1"][ids].astype(np.int64)
    rows = np.arange(len(ids))
    gap = scores[rows, smp] - scores[rows, gpu]
    tol = 2 * 2.0 ** -22 * (np.abs(lg[ids]).max(axis=1) * 1.4426950408889634 + 24.0) / 1.4426950408889634
    sample_ok = bool(((gpu == smp) | (gap <= tol)).all())
    # commit: layer 0's cache after the GPU commit equals the oracle's commit of the cache before it
    (k0, v0), (k1, v1) = ref["commit_layer0"]
    wk, wv = ocommit.commit_kv(f(k0), f(v0), f(rnd.kt[0]), f(rnd.vt[0]), ref["path"], ref["acc"], rnd.offs,
                               w.prefix_lens, rnd.starts)
    commit_ok = bool(np.array_equal(wk, f(k1)) and np.array_equal(wv, f(v1)))
    k0h, v0h, kth, vth = f(k0), f(v0), f(rnd.kt[0]), f(rnd.vt[0])
    t0 = time.perf_counter()
    ocommit.commit_kv(k0h, v0h, kth, vth, ref["path"], ref["acc"], rnd.offs, w.prefix_lens, rnd.starts)
    t_commit = (time.perf_counter() - t0) * w.layers  # one layer timed, scaled to all layers
    t_draft, draft_ok = draft_oracle(db) if db is not None else (None, None)
    round_s = t_build + np.mean(layer_times) * w.layers + t_arg + t_walk
    flops = rnd.attention_flops(t) * w.layers
    parity = {"layers_checked": len(layer_times), "attention_max_abs_err": worst_abs,
              "attention_row_rel_err_max": worst_rel,
              "attention_ok": bool(worst_abs <= 2e-2 and worst_rel <= 1e-2), "build_tree_exact": bool(build_ok),
              "argmax_exact": bool(np.array_equal(ref["am"], am)), "walk_exact": bool(walk_ok),
              "sample_t1_ok": sample_ok, "sample_t1_rows_checked": int(len(ids)),
              "sample_t1_exact_rows": int((gpu == smp).sum()),
              "commit_exact": commit_ok, "draft_tree_exact": draft_ok,
              "mean_accept_len": float(np.mean([L for _, L, _ in walks]))}
    return {
        "value": flops / round_s / 1e12, "unit": "TFLOP/s", "cores": int(min(cores, blas_threads) if blas_threads else cores),
        "kind": "oracle",
        "sample": f"{len(layer_times)} of {w.layers} layers' attention timed (numpy float64, dense ancestor mask), "
                  f"plus tree build, argmax and walk once; scaled to one full round",
        "us_per_round": round_s * 1e6, "host_cores_visible": cores, "blas_threads": blas_threads,
        "seconds": {"build": t_build, "attention_per_layer": float(np.mean(layer_times)), "argmax": t_arg,
                    "walk": t_walk, "sample_t1": t_smp, "commit_all_layers": t_commit,
                    "draft_tree_construction": t_draft},
    }, parity


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the verification path of one round is "
              "single-GPU; sharding by sequence, KV head, vocabulary or prefix is a design note, not code.", file=sys.stderr)
        sys.exit(2)
    import torch

    from gen import configs as gconf

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src_buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        print(f"calibration copy: {nbytes} bytes read, {nbytes} bytes written", file=sys.stderr, flush=True)
        del src_buf, dst_buf
    w = gconf.get(args.workload)
    if args.layers:
        w.layers = args.layers
    rnd = Round(w, dev, temperature=args.temperature, commit=args.commit)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        rnd.step()
    torch.cuda.synchronize()
    if args.phase_stamps:
        print(json.dumps(phase_stamps(rnd)), flush=True)
        return
    # the timed region; HIP events on the kernels' stream bracket each step's attention calls
    att_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        rnd.step(att_events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    att_call_ms = [a.elapsed_time(b) / w.layers for a, b in att_events]  # one dt_tree_attention call

    flops_layer = float(np.mean([rnd.attention_flops(t) for t in range(N_TABLES)]))
    round_flops = flops_layer * w.layers
    value = round_flops / (ms_per_step / 1e3) / 1e12

    att_mean_ms = float(np.mean(att_call_ms))
    arg_ms_single = time_argmax_calls(rnd, reps=10)
    smp_ms_single = time_sample_calls(rnd, reps=10)
    arg_ms = time_back_to_back(rnd, argmax_call(rnd), reps=20)
    smp_ms = time_back_to_back(rnd, lambda i: rnd.sample(rnd.logits[i % N_TABLES], 1000 + i, 1.0), reps=20)
    com_ms, com_bytes, com_acc = time_commit_calls(rnd, reps=10)
    db, draft = time_draft_build(rnd)
    graph_ms = time_round_graph(rnd)
    others = None
    if w.name == gconf.qwen_b256_round().name and not args.no_other_workloads:
        others = {name: time_attention_workload(rnd, name, layers) for name, layers in OTHER_WORKLOADS}
    small = None
    if w.num_seqs == 1:
        ch_ms, ch_b2b_ms, ch_bytes, ch_flops = time_small_tree(rnd)
        sf_ms, sf_b2b_ms, sf_bytes = time_stream_floor(rnd, ch_bytes)
        ch_gbs = ch_bytes / (ch_ms / 1e3) / 1e9
        small = {"workload": f"16-node chain (parent[i] = i - 1) over the same {w.prefix_lens[0]}-token prefix",
                 "bound": "hbm", "us": round(ch_ms * 1e3, 2), "achieved": round(ch_gbs, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(ch_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": ch_bytes,
                 "TFLOP/s": round(ch_flops / (ch_ms / 1e3) / 1e12, 1),
                 "tree_over_chain_time": round(att_mean_ms / ch_ms, 2),
                 "timing": "single call between an event pair (us); consecutive calls (us_back_to_back)",
                 "us_back_to_back": round(ch_b2b_ms * 1e3, 2),
                 "stream_floor": {"kernel": "dt_argmax_rows over a [256, n] fp32 table of the same bytes: one kernel, "
                                            "one workgroup per row, loads and compares only",
                                  "bytes": sf_bytes, "us": round(sf_ms * 1e3, 2),
                                  "us_back_to_back": round(sf_b2b_ms * 1e3, 2),
                                  "GB/s_back_to_back": round(sf_bytes / (sf_b2b_ms / 1e3) / 1e9, 1)}}
    achieved = flops_layer / (att_mean_ms / 1e3) / 1e12
    argmax_bytes = w.total_nodes * w.vocab * 4 + w.total_nodes * 4
    traffic = recorded_traffic(w)
    # the call's bound: matrix cores above the ridge point (peak flops / peak bytes), HBM below it
    att_bytes = attention_bytes(w)
    if flops_layer / att_bytes >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        gbs = att_bytes / (att_mean_ms / 1e3) / 1e9
        bound = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(gbs / PEAK_HBM_GBS, 4), "TFLOP/s": round(achieved, 2)}

    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "prefix_lens": w.prefix_lens if w.num_seqs <= 8 else "ragged",
                   "tree_nodes": w.nodes[0] if len(set(w.nodes)) == 1 else w.nodes, "layers": w.layers,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "vocab": w.vocab, "tree": w.tree},
        "us_per_round": round(ms_per_step * 1e3, 1),
        "us_per_round_device_graph": round(graph_ms * 1e3, 1),
        "roofline": {**bound, "kernel": "dt_tree_attention call (tree_attn_fwd + tree_attn_combine)",
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "flops_per_launch": flops_layer, "launch_us_mean": round(att_mean_ms * 1e3, 2),
                     "launch_us_median": round(float(np.median(att_call_ms)) * 1e3, 2),
                     "algorithmic_bytes_per_launch": att_bytes,
                     "traffic_source": traffic["source"] if traffic else None},
        "argmax": {"ms": arg_ms, "GB/s": argmax_bytes / (arg_ms / 1e3) / 1e9,
                   "frac_hbm": argmax_bytes / (arg_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                   "timing": "mean of 20 back-to-back calls between one event pair",
                   "ms_single_call": arg_ms_single},
        "sample": {"kernel": "dt_sample_rows (Gumbel-max, Philox4x32-10), T = 1", "ms": smp_ms,
                   "GB/s": argmax_bytes / (smp_ms / 1e3) / 1e9,
                   "frac_hbm": argmax_bytes / (smp_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                   "timing": "mean of 20 back-to-back calls between one event pair",
                   "ms_single_call": smp_ms_single},
        "commit": {"kernel": "dt_commit_kv, all layers in one call", "us": com_ms * 1e3, "bytes": com_bytes,
                   "GB/s": com_bytes / (com_ms / 1e3) / 1e9, "accept_len": com_acc.tolist()},
        "small_tree": small,
        "other_workloads": others,
        "draft_tree": dict(draft, kernels="dt_topk_rows, dt_expand_depth (x16 in the chain), dt_prune_topb"),
        "step_variant": {"temperature": args.temperature, "commit": bool(args.commit)},
        "parity": None,
        "trees": tree_shape(rnd),
    }
    if not args.no_cpu_baseline:
        t1_offset = 424242
        ref = reference_outputs(rnd, t1_offset)
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(rnd, args.cpu_budget_s, ref, t1_offset, db)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
