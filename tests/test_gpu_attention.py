"""GPU parity of dt_tree_attention against the oracle (fp64, dense ancestor mask).

Tolerance (attention output, bf16): max |got - ref| <= 2e-2 and, per (node,
head) row, max |got - ref| / max |ref| <= 1e-2. Mask behaviour is also checked
bit-exactly: perturbing the K/V of a node's non-ancestors leaves its output
bits unchanged, and repeated runs give identical bits.
"""

import numpy as np
import pytest

import draft_tree_verification_dt_amd as dt
from _helpers import assert_attention_close, dev_bf16, dev_i32, host_f64, require_gpu, tree, workload_inputs
from gen import configs as gconf, rng as grng, tensors as gten
from oracle import attention as oatt, tree as otree

pytestmark = pytest.mark.gpu


def _run(ops, parents, nodes, plens, Hq, Hkv, d, scale=None, split_keys=0, prefix=None, layout=None):
    """Run dt_tree_attention on packed host operands; returns (out tensor, device inputs)."""
    import torch

    q, kt, vt = dev_bf16(ops["q"]), dev_bf16(ops["k_tree"]), dev_bf16(ops["v_tree"])
    if prefix is None:
        kp = dev_bf16(ops["k_prefix"]) if ops["k_prefix"].shape[0] else None
        vp = dev_bf16(ops["v_prefix"]) if ops["v_prefix"].shape[0] else None
    else:
        kp, vp = prefix
    par = dev_i32(np.concatenate(parents))
    if layout is None:
        layout = dt.AttnLayout(np.concatenate([[0], np.cumsum(nodes)]), plens)
    out = dt.dt_tree_attention(q, kt, vt, kp, vp, par, layout, scale=scale, split_keys=split_keys)
    torch.cuda.synchronize()
    return out, (q, kt, vt, kp, vp, par, layout)


def _oracle(ops, parents, nodes, plens, scale=None):
    offs = np.concatenate([[0], np.cumsum(nodes)])
    starts = np.concatenate([[0], np.cumsum(plens)[:-1]]).astype(np.int64)
    return oatt.batch_tree_attention(ops["q"], ops["k_tree"], ops["v_tree"], ops["k_prefix"], ops["v_prefix"],
                                     np.concatenate(parents), offs, plens, starts, scale)


def _case(nodes, plens, Hq, Hkv, d, shapes, seed, scale=None):
    r = grng.stream(seed, "gpu-att")
    parents = [tree(shapes[i % len(shapes)], n, seed * 31 + i)[0] for i, n in enumerate(nodes)]
    ops = [gten.attention_operands(r, n, P, Hq, Hkv, d, scale=scale) for n, P in zip(nodes, plens)]
    return parents, {k: np.concatenate([o[k] for o in ops]) for k in ops[0]}


def test_tiny_config():
    require_gpu()
    w = gconf.tiny()
    parents, tokens, ops = workload_inputs(w)
    print("tiny: n=16 P=128 d=64 Hq=Hkv=1", flush=True)
    out, _ = _run(ops, parents, w.nodes, w.prefix_lens, w.Hq, w.Hkv, w.d)
    assert_attention_close(host_f64(out), _oracle(ops, parents, w.nodes, w.prefix_lens), what="tiny")


EDGE_N = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 512]


@pytest.mark.parametrize("P", [0, 1, 63, 64, 65])
@pytest.mark.parametrize("n", EDGE_N)
def test_edge_shapes_d128_g4(P, n):
    require_gpu()
    parents, ops = _case([n], [P], 8, 2, 128, ["recursive", "deep", "bfs"], seed=P * 1000 + n)
    print(f"edge d=128 g=4 P={P} n={n}", flush=True)
    out, _ = _run(ops, parents, [n], [P], 8, 2, 128)
    assert_attention_close(host_f64(out), _oracle(ops, parents, [n], [P]), what=f"P={P} n={n}")


@pytest.mark.parametrize("P,n", [(0, 1), (1, 17), (65, 64), (200, 129), (64, 512)])
def test_edge_shapes_d64_g1(P, n):
    require_gpu()
    parents, ops = _case([n], [P], 2, 2, 64, ["deep"], seed=7 + P + n)
    print(f"edge d=64 g=1 P={P} n={n}", flush=True)
    out, _ = _run(ops, parents, [n], [P], 2, 2, 64)
    assert_attention_close(host_f64(out), _oracle(ops, parents, [n], [P]), what=f"d64 P={P} n={n}")


@pytest.mark.parametrize("g", [1, 2, 3, 8])
def test_group_sizes(g):
    require_gpu()
    parents, ops = _case([40], [150], 2 * g, 2, 128, ["recursive"], seed=90 + g)
    print(f"gqa g={g}", flush=True)
    out, _ = _run(ops, parents, [40], [150], 2 * g, 2, 128)
    assert_attention_close(host_f64(out), _oracle(ops, parents, [40], [150]), what=f"g={g}")


def test_sharp_distribution_and_custom_scale():
    require_gpu()
    parents, ops = _case([100], [300], 8, 2, 128, ["deep"], seed=5, scale=1.0)
    print("sharp", flush=True)
    out, _ = _run(ops, parents, [100], [300], 8, 2, 128)
    assert_attention_close(host_f64(out), _oracle(ops, parents, [100], [300]), what="sharp")
    out2, _ = _run(ops, parents, [100], [300], 8, 2, 128, scale=0.05)
    assert_attention_close(host_f64(out2), _oracle(ops, parents, [100], [300], scale=0.05), what="scale")


@pytest.mark.parametrize("seed", range(4))
def test_random_batches(seed):
    """Seeded random batches: sequence counts, tree sizes and shapes, prefix
    lengths (ragged or equal), GQA group sizes, head dims 64 and 128, and now
    and then a forced key split, against the oracle. The planner picks its row
    tiles, splits and launches on its own for each."""
    require_gpu()
    r = grng.stream(seed, "attention-sweep")
    for case in range(4):
        S = int(r.integers(1, 5))
        nodes = [int(r.integers(1, 300)) for _ in range(S)]
        if r.random() < 0.5:
            plens = [int(r.integers(0, 2500)) for _ in range(S)]
        else:
            plens = [int(r.integers(0, 2500))] * S
        Hkv, g = int(r.choice([1, 2, 4])), int(r.choice([1, 2, 3, 4, 8]))
        d = int(r.choice([64, 128]))
        split = int(r.choice([0, 0, 0, 64, 192, 1024]))
        shapes = [str(r.choice(["recursive", "deep", "bfs", "chain", "heap"]))]
        print(f"attention sweep {seed}.{case} S={S} n={nodes} P={plens} Hkv={Hkv} g={g} d={d} split={split} "
              f"shape={shapes[0]}", flush=True)
        parents, ops = _case(nodes, plens, Hkv * g, Hkv, d, shapes, seed=seed * 10 + case)
        out, _ = _run(ops, parents, nodes, plens, Hkv * g, Hkv, d, split_keys=split)
        assert_attention_close(host_f64(out), _oracle(ops, parents, nodes, plens), what=f"sweep {seed}.{case}")


@pytest.mark.parametrize("split", [64, 128, 576, 4096])
def test_forced_key_splits(split):
    require_gpu()
    parents, ops = _case([100], [1000], 8, 2, 128, ["deep"], seed=11, scale=0.5)
    print(f"split_keys={split}", flush=True)
    out, _ = _run(ops, parents, [100], [1000], 8, 2, 128, split_keys=split)
    assert_attention_close(host_f64(out), _oracle(ops, parents, [100], [1000]), what=f"split {split}")


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 6, 3)])
def test_forced_splits_over_several_launches(d, Hq, Hkv):
    """More sequences than one launch carries, every one split into key chunks of
    its own count: each launch's partials (chunk, KV head, packed row) and merge
    rows stay within their sequence's region."""
    require_gpu()
    rng = grng.stream(5, "many-split")
    nodes = [int(x) for x in rng.integers(1, 60, size=40)]
    plens = [int(x) for x in rng.integers(0, 700, size=40)]
    parents, ops = _case(nodes, plens, Hq, Hkv, d, ["recursive", "deep", "bfs"], seed=44)
    print(f"40 sequences, split_keys=128, d={d}", flush=True)
    out, _ = _run(ops, parents, nodes, plens, Hq, Hkv, d, split_keys=128)
    assert_attention_close(host_f64(out), _oracle(ops, parents, nodes, plens), what="many split")


@pytest.mark.parametrize("v_scale", [1e-3, 3e3])
def test_split_partials_keep_precision_at_any_magnitude(v_scale):
    """Split sequences merge per-chunk partials; the merge must be exact up to
    rounding whatever the magnitude of V (the result is linear in V)."""
    require_gpu()
    parents, ops = _case([120], [900], 8, 2, 128, ["deep"], seed=13, scale=0.7)
    ops = dict(ops)
    for key in ("v_tree", "v_prefix"):
        ops[key] = gten.bf16_round(ops[key] * np.float32(v_scale))
    print(f"split partials v_scale={v_scale}", flush=True)
    for split in (64, 320):
        out, _ = _run(ops, parents, [120], [900], 8, 2, 128, split_keys=split)
        assert_attention_close(host_f64(out), _oracle(ops, parents, [120], [900]), atol=2e-2 * max(v_scale, 1.0),
                               what=f"v_scale={v_scale} split={split}")


def test_ragged_batch_strided_cache():
    """Five sequences with different prefixes and trees; the prefix cache is
    head-major [Hkv][rows][d] with gaps between the sequences' rows."""
    import torch

    require_gpu()
    nodes, plens = [1, 33, 100, 256, 17], [0, 17, 500, 1000, 64]
    Hq, Hkv, d = 8, 2, 128
    parents, ops = _case(nodes, plens, Hq, Hkv, d, ["deep", "recursive", "bfs", "heap", "chain"], seed=21, scale=0.6)
    gap = 37
    starts = []
    row = 5
    for P in plens:
        starts.append(row)
        row += P + gap
    cache_rows = row
    kc = torch.zeros((Hkv, cache_rows, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    src = 0
    for P, st in zip(plens, starts):
        kc[:, st:st + P] = dev_bf16(ops["k_prefix"][src:src + P]).transpose(0, 1)
        vc[:, st:st + P] = dev_bf16(ops["v_prefix"][src:src + P]).transpose(0, 1)
        src += P
    kp = kc.transpose(0, 1)  # [rows][Hkv][d] view: row stride d, head stride rows*d
    vp = vc.transpose(0, 1)
    layout = dt.AttnLayout(np.concatenate([[0], np.cumsum(nodes)]), plens, starts)
    print("ragged strided", flush=True)
    out, _ = _run(ops, parents, nodes, plens, Hq, Hkv, d, prefix=(kp, vp), layout=layout)
    assert_attention_close(host_f64(out), _oracle(ops, parents, nodes, plens), what="ragged")


def test_many_sequences_multi_launch():
    """More sequences than one launch carries."""
    require_gpu()
    rng = grng.stream(3, "many")
    nodes = [int(x) for x in rng.integers(1, 40, size=70)]
    plens = [int(x) for x in rng.integers(0, 130, size=70)]
    parents, ops = _case(nodes, plens, 4, 1, 64, ["recursive", "deep"], seed=33)
    print("70 sequences", flush=True)
    out, _ = _run(ops, parents, nodes, plens, 4, 1, 64)
    assert_attention_close(host_f64(out), _oracle(ops, parents, nodes, plens), what="many")


def test_non_ancestor_perturbation_bit_exact_and_determinism():
    import torch

    require_gpu()
    n, P = 200, 300
    parents, ops = _case([n], [P], 8, 2, 128, ["recursive"], seed=41)
    print("perturbation", flush=True)
    base, _ = _run(ops, parents, [n], [P], 8, 2, 128)
    again, _ = _run(ops, parents, [n], [P], 8, 2, 128)
    assert torch.equal(base, again), "two runs differ"
    anc = otree.ancestor_matrix(parents[0])
    rng = grng.stream(42)
    for i in [0, 1, 57, 150, 199]:
        others = ~anc[i]
        ops2 = dict(ops)
        for key in ("k_tree", "v_tree"):
            a = ops[key].copy()
            sign = np.where(rng.random(int(others.sum())) < 0.5, -1.0, 1.0).astype(np.float32)[:, None, None]
            a[others] = gten.bf16_round(a[others] + np.float32(500.0) * sign)
            ops2[key] = a
        pert, _ = _run(ops2, parents, [n], [P], 8, 2, 128)
        assert torch.equal(pert[i], base[i]), f"node {i} saw a non-ancestor"
        if others.any():
            assert not torch.equal(pert, base)


@pytest.mark.parametrize("name", ["b128", "b256", "chain16"])
def test_full_size_single_sequence(name):
    """Qwen3-4B-shaped layers (Hq=32, Hkv=8, d=128) at full size, whole output."""
    require_gpu()
    w = gconf.get(name)
    parents, tokens, ops = workload_inputs(w)
    print(f"full {w.name}", flush=True)
    out, _ = _run(ops, parents, w.nodes, w.prefix_lens, w.Hq, w.Hkv, w.d)
    assert_attention_close(host_f64(out), _oracle(ops, parents, w.nodes, w.prefix_lens), what=w.name)


def test_full_size_ragged_batch():
    require_gpu()
    w = gconf.ragged()
    parents, tokens, ops = workload_inputs(w)
    print(f"full {w.name} P={w.prefix_lens}", flush=True)
    out, _ = _run(ops, parents, w.nodes, w.prefix_lens, w.Hq, w.Hkv, w.d)
    assert_attention_close(host_f64(out), _oracle(ops, parents, w.nodes, w.prefix_lens), what=w.name)


def test_long_context_full_output():
    """4 x (P=32768, n=512), one layer: operands drawn on the device, the whole
    output (4 x 512 nodes x 32 heads) compared with the oracle sequence by
    sequence. No key split happens at this size: 256 workgroups of 256 rows
    each stream all 33280 keys of their sequence."""
    import torch

    require_gpu()
    w = gconf.long_context()
    Hq, Hkv, d = w.Hq, w.Hkv, w.d
    N, PT = w.total_nodes, w.total_prefix
    sc = 1.0 / np.sqrt(d)
    q = gten.device_randn_bf16((N, Hq, d), w.seed, "q", scale=sc)
    kt = gten.device_randn_bf16((N, Hkv, d), w.seed, "kt", scale=sc)
    vt = gten.device_randn_bf16((N, Hkv, d), w.seed, "vt", scale=sc)
    kp = gten.device_randn_bf16((PT, Hkv, d), w.seed, "kp", scale=sc)
    vp = gten.device_randn_bf16((PT, Hkv, d), w.seed, "vp", scale=sc)
    parents = [tree("heap", n, w.seed * 1000 + s)[0] for s, n in enumerate(w.nodes)]
    layout = dt.AttnLayout(w.node_offsets(), w.prefix_lens)
    print(f"long {w.name}", flush=True)
    out = dt.dt_tree_attention(q, kt, vt, kp, vp, dev_i32(np.concatenate(parents)), layout)
    torch.cuda.synchronize()
    hq, hkt, hvt, hout = (host_f64(t) for t in (q, kt, vt, out))
    offs, starts = w.node_offsets(), w.prefix_row_starts()
    for s in range(w.num_seqs):
        a, b, p0, P = offs[s], offs[s + 1], starts[s], w.prefix_lens[s]
        ref = oatt.tree_attention(hq[a:b], hkt[a:b], hvt[a:b], host_f64(kp[p0:p0 + P]), host_f64(vp[p0:p0 + P]),
                                  parents[s])
        print(f"long seq {s} checked", flush=True)
        assert_attention_close(hout[a:b], ref, what=f"long seq {s}")


def test_round_replays_from_a_hip_graph():
    """A verification round (tree attention over four layers, arg-max, walk and
    KV commit) captured once in a HIP graph: the library allocates nothing and
    records no memset, so every call is capturable. Each replay, with new inputs
    written into the same buffers, equals the eager calls on those inputs."""
    import torch

    from _helpers import dev_i32
    from gen import tensors as gten

    require_gpu()
    layers, n, P, Hq, Hkv, d, vocab = 4, 256, 4096, 32, 8, 128, 32000
    dev = "cuda"
    parent, token = tree("heap", n, 31, vocab=vocab)
    par, tok = dev_i32(parent), dev_i32(token)
    layout = dt.AttnLayout([0, n], [P], [0])
    q = [torch.empty((n, Hq, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    kt = [torch.empty((n, Hkv, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    vt = [torch.empty((n, Hkv, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    kc = [torch.empty((P + n, Hkv, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    vc = [torch.empty((P + n, Hkv, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    out = [torch.empty((n, Hq, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    logits = torch.empty((n, vocab), dtype=torch.float32, device=dev)
    ws = torch.empty(max(dt.dt_tree_attention_workspace_size(q[0], kt[0], kc[0], layout), 256), dtype=torch.uint8,
                     device=dev)
    am = torch.empty(n, dtype=torch.int32, device=dev)
    am_ws = torch.empty(max(dt.dt_argmax_rows_workspace_size(n, vocab), 256), dtype=torch.uint8, device=dev)
    path = torch.empty(n, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    bonus = torch.empty(1, dtype=torch.int32, device=dev)
    commit = dt.CommitArgs(layout, [P + n], kt, vt, kc, vc, max_path=17)

    def fill(seed):
        for l in range(layers):
            for t, name in ((q[l], "q"), (kt[l], "kt"), (vt[l], "vt"), (kc[l], "kc"), (vc[l], "vc")):
                t.copy_(gten.device_randn_bf16(tuple(t.shape), seed, name, l, scale=d ** -0.5))
        logits.copy_(gten.device_logits(n, vocab, seed, "lg"))
        gten.device_plant(grng.stream(seed, "plant"), logits, 0, parent, token, p=0.9)

    def round_():
        for l in range(layers):
            dt.dt_tree_attention(q[l], kt[l], vt[l], kc[l], vc[l], par, layout, out=out[l], workspace=ws)
        dt.dt_argmax_rows(logits, out=am, workspace=am_ws)
        dt.dt_accept_path([0, n], par, tok, am, path=path, accept_len=acc, bonus=bonus)
        dt.dt_commit_kv(commit, path, acc)

    def snapshot():
        torch.cuda.synchronize()
        return [x.clone() for x in out + [am, path, acc, bonus] + kc + vc]

    fill(1)
    round_()  # warm-up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_()
    print("verification round captured", flush=True)
    for rep, seed in enumerate((2, 3, 4)):
        fill(seed)
        saved = [x.clone() for x in kc + vc]
        round_()
        eager = snapshot()
        for x, y in zip(kc + vc, saved):
            x.copy_(y)  # the commit wrote into the caches: restore them for the replay
        for x in out + [am, path, acc, bonus]:
            x.fill_(0)
        graph.replay()
        replayed = snapshot()
        for a, b in zip(eager, replayed):
            assert torch.equal(a, b), f"replay {rep}"
        assert int(acc.cpu()[0]) > 0


@pytest.mark.parametrize("g,d", [(1, 128), (4, 128), (1, 64)])
def test_maximum_tree_size(g, d):
    """Trees of DT_MAX_TREE_NODES = 1024 nodes. With one query head per KV head
    the ancestor masks of a 256-row tile do not fit beside the K/V ring, so the
    planner falls back to 128-row tiles; with g = 4 the 256-row tiles stay."""
    require_gpu()
    n, P = 1024, 100
    parents, ops = _case([n], [P], 2 * g, 2, d, ["recursive"], seed=71 + g + d, scale=0.5)
    print(f"maximum tree n={n} P={P} g={g} d={d}", flush=True)
    out, _ = _run(ops, parents, [n], [P], 2 * g, 2, d)
    assert_attention_close(host_f64(out), _oracle(ops, parents, [n], [P]), what=f"n={n} g={g} d={d}")


@pytest.mark.parametrize("n,P", [(48, 300), (300, 700)])
def test_relabelling_permutes_outputs(n, P):
    """A random topological renumbering of the same tree (nodes, their Q/K/V and
    parents permuted together) permutes the outputs: node i's attention depends
    on its ancestors, not on their numbering. The tree keys then arrive in
    another order, so the comparison is at the attention tolerance; both runs
    are also checked against the oracle."""
    require_gpu()
    parents, ops = _case([n], [P], 8, 2, 128, ["recursive"], seed=81 + n, scale=0.8)
    parent = parents[0]
    r = grng.stream(82, "relabel", n)
    placed, order = {0}, [0]
    while len(order) < n:
        ready = [i for i in range(n) if i not in placed and parent[i] in placed]
        i = ready[int(r.integers(0, len(ready)))]
        placed.add(i)
        order.append(i)
    new_of = {old: new for new, old in enumerate(order)}
    parent2 = np.array([-1 if old == 0 else new_of[int(parent[old])] for old in order], np.int32)
    ops2 = dict(ops)
    for key in ("q", "k_tree", "v_tree"):
        ops2[key] = ops[key][order]
    print(f"relabelling n={n} P={P}", flush=True)
    base, _ = _run(ops, [parent], [n], [P], 8, 2, 128)
    got, _ = _run(ops2, [parent2], [n], [P], 8, 2, 128)
    b, g2 = host_f64(base), host_f64(got)
    assert_attention_close(g2, b[order], what=f"relabelled n={n}")
    assert_attention_close(b, _oracle(ops, [parent], [n], [P]), what=f"original n={n}")
    assert_attention_close(g2, _oracle(ops2, [parent2], [n], [P]), what=f"relabelled vs oracle n={n}")


@pytest.mark.parametrize("n,P", [(100, 500), (16, 1200)])
def test_fused_qkv_views_and_strided_output(n, P):
    """Q, K and V as column slices of one fused projection output [N, (Hq + 2 Hkv) d]
    (row strides larger than their own width) and the output written into a
    slice of a wider buffer: the same result as contiguous operands, and the
    columns around the output slice untouched."""
    import torch

    require_gpu()
    Hq, Hkv, d = 8, 2, 128
    parents, ops = _case([n], [P], Hq, Hkv, d, ["recursive"], seed=91 + n, scale=0.6)
    qkv = torch.cat([dev_bf16(ops["q"]).reshape(n, Hq * d), dev_bf16(ops["k_tree"]).reshape(n, Hkv * d),
                     dev_bf16(ops["v_tree"]).reshape(n, Hkv * d)], dim=1).contiguous()
    q = qkv[:, :Hq * d].view(n, Hq, d)
    kt = qkv[:, Hq * d:(Hq + Hkv) * d].view(n, Hkv, d)
    vt = qkv[:, (Hq + Hkv) * d:].view(n, Hkv, d)
    assert q.stride(0) == (Hq + 2 * Hkv) * d and kt.stride() == vt.stride()
    kp, vp = dev_bf16(ops["k_prefix"]), dev_bf16(ops["v_prefix"])
    par = dev_i32(parents[0])
    layout = dt.AttnLayout([0, n], [P])
    wide = torch.full((n, (Hq + 3) * d), 7.0, dtype=torch.bfloat16, device="cuda")
    out = wide[:, d:(Hq + 1) * d].view(n, Hq, d)
    print(f"fused qkv n={n} P={P}", flush=True)
    dt.dt_tree_attention(q, kt, vt, kp, vp, par, layout, out=out)
    ref_dev = dt.dt_tree_attention(q.contiguous(), kt.contiguous(), vt.contiguous(), kp, vp, par, layout)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_dev), "strided operands changed the result"
    assert bool((wide[:, :d] == 7.0).all()) and bool((wide[:, (Hq + 1) * d:] == 7.0).all()), "wrote outside the slice"
    assert_attention_close(host_f64(out), _oracle(ops, parents, [n], [P]), what=f"fused qkv n={n}")


def test_phase_stamps():
    """The optional phase stamps: the output is bit-identical with and without
    them; every forward workgroup that stored outputs has non-decreasing stamps
    for its phases (the first-stage stamp only where it visits keys) and every
    merge block that stored outputs has entry <= stored; each row carries its
    kernel's tag; a workgroup past the last work item stamps only its entry;
    slot 6, rows past the call's workgroups and rows past the buffer are
    untouched; over several launches (more sequences than one launch carries)
    the rows keep counting."""
    import torch

    require_gpu()
    Hq, Hkv, d = 8, 2, 128
    parents, ops = _case([100], [3000], Hq, Hkv, d, ["recursive"], seed=57)
    out, (q, kt, vt, kp, vp, par, layout) = _run(ops, parents, [100], [3000], Hq, Hkv, d)
    buf = torch.full((4096, 8), -1, dtype=torch.int64, device="cuda")
    print("phase stamps n=100 P=3000", flush=True)
    out2 = dt.dt_tree_attention(q, kt, vt, kp, vp, par, layout, phase_stamps=buf)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "phase stamps changed the output"
    s = buf.cpu().numpy()
    entered = s[:, 0] != -1
    n_wg = int(entered.sum())
    assert n_wg > 0 and entered[:n_wg].all() and not entered[n_wg:].any(), "rows past the call were written"
    tag = s[:n_wg, 7]
    assert set(np.unique(tag)) == {1, 2}, "a split call runs both kernels"
    n_fwd = int((tag == 1).sum())
    assert (tag[:n_fwd] == 1).all() and (tag[n_fwd:] == 2).all(), "forward rows first, then the merge's"
    fwd, mrg = s[:n_fwd], s[n_fwd:n_wg]
    stored = fwd[:, 5] != -1
    assert stored.sum() > 0
    ph = fwd[stored][:, :6]
    always = ph[:, [0, 1, 2, 4, 5]]  # a work item with no keys to visit has no first stage (slot 3)
    assert (always > 0).all() and (np.diff(always, axis=1) >= 0).all(), "phase stamps out of order"
    landed = ph[:, 3] != -1
    assert landed.any()
    assert ((ph[landed, 3] >= ph[landed, 2]) & (ph[landed, 3] <= ph[landed, 4])).all()
    assert (fwd[~stored][:, 1:7] == -1).all(), "a workgroup without a work item stamped past its entry"
    mst = mrg[:, 5] != -1
    assert mst.any() and (mrg[mst, 5] >= mrg[mst, 0]).all() and (mrg[:, 1:5] == -1).all()
    assert mrg[mst, 0].min() >= ph[:, 5].max(), "the merge started before the forward kernel's last store"
    assert (s[:, 6] == -1).all()
    assert_attention_close(host_f64(out2), _oracle(ops, parents, [100], [3000]), what="phase stamps")

    # several launches, a buffer shorter than the call's workgroups
    rng = grng.stream(3, "many")
    nodes = [int(x) for x in rng.integers(1, 40, size=70)]
    plens = [int(x) for x in rng.integers(0, 130, size=70)]
    parents, ops = _case(nodes, plens, 4, 1, 64, ["recursive", "deep"], seed=33)
    out, (q, kt, vt, kp, vp, par, layout) = _run(ops, parents, nodes, plens, 4, 1, 64)
    big = torch.full((4096, 8), -1, dtype=torch.int64, device="cuda")
    dt.dt_tree_attention(q, kt, vt, kp, vp, par, layout, phase_stamps=big)
    torch.cuda.synchronize()
    e = (big[:, 0] != -1).cpu().numpy()
    total = int(e.sum())
    print(f"phase stamps over launches: {total} workgroups", flush=True)
    assert e[:total].all() and bool(((big[:total, 7] == 1) | (big[:total, 7] == 2)).all())
    rows = total - 5
    big.fill_(-1)
    out3 = dt.dt_tree_attention(q, kt, vt, kp, vp, par, layout, phase_stamps=big[:rows])
    torch.cuda.synchronize()
    assert torch.equal(out, out3)
    e = (big[:, 0] != -1).cpu().numpy()
    assert e[:rows].all() and not e[rows:].any(), "rows past phase_stamp_rows were written"


@pytest.mark.parametrize("n,P,Hq,Hkv,d", [(16, 2500, 8, 2, 128), (40, 900, 8, 2, 128), (200, 3000, 8, 2, 128),
                                          (300, 1500, 4, 1, 64), (12, 4000, 2, 2, 64)])
def test_phase_stamps_builds_match_plain_ones(n, P, Hq, Hkv, d):
    """The stamping instantiations of both kernels compute the same bits as the
    plain ones for every tile shape (64-, 128- and 256-row tiles, d = 64 and
    128, split and unsplit), and every forward workgroup that stored outputs
    stamped its entry before its store."""
    import torch

    require_gpu()
    parents, ops = _case([n], [P], Hq, Hkv, d, ["recursive"], seed=71 + n)
    out, (q, kt, vt, kp, vp, par, layout) = _run(ops, parents, [n], [P], Hq, Hkv, d)
    buf = torch.zeros((4096, 8), dtype=torch.int64, device="cuda")
    print(f"phase-stamp build n={n} P={P} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    out2 = dt.dt_tree_attention(q, kt, vt, kp, vp, par, layout, phase_stamps=buf)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "the stamping build changed the output"
    s = buf.cpu().numpy()
    fwd = s[(s[:, 7] == 1) & (s[:, 5] != 0)]
    assert len(fwd) > 0 and (fwd[:, 5] >= fwd[:, 0]).all()


def test_binding_rejects_mistyped_or_short_tensors():
    """The binding checks what the C library cannot see (dtypes, devices,
    extents, output shapes) and raises ValueError before anything is enqueued;
    the caller's output buffers stay untouched."""
    import torch

    require_gpu()
    Hq, Hkv, d, n, P = 4, 2, 64, 10, 100
    parents, ops = _case([n], [P], Hq, Hkv, d, ["recursive"], seed=3)
    q, kt, vt = dev_bf16(ops["q"]), dev_bf16(ops["k_tree"]), dev_bf16(ops["v_tree"])
    kp, vp = dev_bf16(ops["k_prefix"]), dev_bf16(ops["v_prefix"])
    par = dev_i32(parents[0])
    layout = dt.AttnLayout([0, n], [P])
    out = torch.full((n, Hq, d), 3.0, dtype=torch.bfloat16, device="cuda")
    bad = [
        dict(q=q.half()),                                  # operand dtype
        dict(k_prefix=kp.float()),
        dict(parent=par.long()),                           # int64 parent
        dict(parent=par[: n - 1]),                         # too short
        dict(q=q.cpu()),                                   # host tensor
        dict(out=torch.empty((n, Hq, d), dtype=torch.float16, device="cuda")),
        dict(out=torch.empty((n - 1, Hq, d), dtype=torch.bfloat16, device="cuda")),
        dict(phase_stamps=torch.zeros((8, 4), dtype=torch.int64, device="cuda")),
        dict(phase_stamps=torch.zeros((8, 8), dtype=torch.int32, device="cuda")),
    ]
    for kw in bad:
        args = dict(q=q, k_tree=kt, v_tree=vt, k_prefix=kp, v_prefix=vp, parent=par, out=out)
        args.update(kw)
        with pytest.raises(ValueError):
            dt.dt_tree_attention(args["q"], args["k_tree"], args["v_tree"], args["k_prefix"], args["v_prefix"],
                                 args["parent"], layout, out=args["out"],
                                 **({"phase_stamps": kw["phase_stamps"]} if "phase_stamps" in kw else {}))
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a rejected call wrote its output"
    # the walk: int32 inputs of at least N entries, outputs of the right type and size
    offs = [0, n]
    tok = dev_i32(np.arange(n))
    am = dev_i32(np.zeros(n))
    for kw in [dict(parent=par.long()), dict(token=tok[: n - 2]), dict(argmax_idx=am.float()),
               dict(path=torch.empty(n - 1, dtype=torch.int32, device="cuda")),
               dict(accept_len=torch.empty(1, dtype=torch.int64, device="cuda"))]:
        args = dict(parent=par, token=tok, argmax_idx=am)
        args.update(kw)
        with pytest.raises(ValueError):
            dt.dt_accept_path(offs, args["parent"], args["token"], args["argmax_idx"], path=args.get("path"),
                              accept_len=args.get("accept_len"))
