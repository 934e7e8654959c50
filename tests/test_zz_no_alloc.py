"""dt_tree_attention_noalloc (the entry point for callers that cannot allocate)
against dt_tree_attention, through the C ABI, on two calls in a row: the
first at the 256-node round geometry (the plan splits the keys, so the static
buffer holds the partials), the second smaller (a 40-node tree over 700 keys,
also split) -- the buffer keeps the first call's contents, which the second
must not see. Both are also checked against the oracle, and a call whose
default plan needs more partials than the buffer holds (a ragged batch) runs
with larger key chunks and still meets the attention tolerance.
"""

import numpy as np
import pytest

import draft_tree_verification_dt_amd as dt
from _helpers import assert_attention_close, dev_bf16, dev_i32, host_f64, require_gpu, tree
from gen import rng as grng, tensors as gten
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


def _inputs(nodes, plens, Hq, Hkv, d, seed):
    r = grng.stream(seed, "noalloc")
    parents = [tree("heap", n, seed * 7 + i)[0] for i, n in enumerate(nodes)]
    ops = [gten.attention_operands(r, n, P, Hq, Hkv, d) for n, P in zip(nodes, plens)]
    ops = {k: np.concatenate([o[k] for o in ops]) for k in ops[0]}
    dev = {k: dev_bf16(v) for k, v in ops.items()}
    return parents, ops, dev


def _both(nodes, plens, Hq, Hkv, d, seed, split_keys=0):
    import torch

    parents, ops, t = _inputs(nodes, plens, Hq, Hkv, d, seed)
    par = dev_i32(np.concatenate(parents))
    layout = dt.AttnLayout(np.concatenate([[0], np.cumsum(nodes)]), plens)
    ref = dt.dt_tree_attention(t["q"], t["k_tree"], t["v_tree"], t["k_prefix"], t["v_prefix"], par, layout,
                               split_keys=split_keys)
    out = torch.full_like(t["q"], float("nan"))
    dt.dt_tree_attention_noalloc(t["q"], t["k_tree"], t["v_tree"], t["k_prefix"], t["v_prefix"], par, layout, out,
                                 split_keys=split_keys)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(nodes)])
    starts = np.concatenate([[0], np.cumsum(plens)[:-1]]).astype(np.int64)
    oracle = oatt.batch_tree_attention(ops["q"], ops["k_tree"], ops["v_tree"], ops["k_prefix"], ops["v_prefix"],
                                       np.concatenate(parents), offs, plens, starts)
    return ref, out, oracle, layout, t


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    import torch

    require_gpu()
    print("noalloc call 1: n=256 P=8192 Hq=32 Hkv=8 d=128", flush=True)
    ref, out, oracle, layout, t = _both([256], [8192], 32, 8, 128, seed=1)
    need = dt.dt_tree_attention_workspace_size(t["q"], t["k_tree"], t["k_prefix"], layout)
    assert 0 < need <= (32 << 20), "the round geometry splits and fits the static buffer"
    assert torch.equal(out, ref), "same plan, same kernels: bit-identical to the workspace entry point"
    assert_attention_close(host_f64(out), oracle, what="noalloc call 1")

    print("noalloc call 2: n=40 P=700 Hq=8 Hkv=2 d=128, keys split in 128", flush=True)
    ref2, out2, oracle2, _, _ = _both([40], [700], 8, 2, 128, seed=2, split_keys=128)
    assert torch.equal(out2, ref2), "second, smaller call: bit-identical, untouched by the first call's partials"
    assert_attention_close(host_f64(out2), oracle2, what="noalloc call 2")


def test_noalloc_larger_chunks_when_partials_exceed_the_buffer():
    require_gpu()
    nodes, plens = [256] * 8, [16252, 1703, 15484, 11106, 15151, 8079, 11853, 3256]
    print("noalloc ragged batch (8 x 256 nodes, P 1.7k-16k)", flush=True)
    ref, out, oracle, layout, t = _both(nodes, plens, 32, 8, 128, seed=3)
    need = dt.dt_tree_attention_workspace_size(t["q"], t["k_tree"], t["k_prefix"], layout)
    assert need > (32 << 20), "this batch's default plan needs more than the static buffer"
    assert_attention_close(host_f64(out), oracle, what="noalloc ragged")
    assert_attention_close(host_f64(out), host_f64(ref), what="noalloc vs workspace entry point")


def test_noalloc_rejects_a_forced_split_beyond_the_buffer():
    require_gpu()
    import torch

    plens = [60000]
    q = torch.zeros((1024, 32, 128), dtype=torch.bfloat16, device="cuda")
    kt = torch.zeros((1024, 8, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((60000, 8, 128), dtype=torch.bfloat16, device="cuda")
    par = dev_i32(np.arange(-1, 1023))
    layout = dt.AttnLayout(np.array([0, 1024]), plens)
    out = torch.empty_like(q)
    with pytest.raises(dt.DtError) as e:
        dt.dt_tree_attention_noalloc(q, kt, kt, kp, kp, par, layout, out, split_keys=64)
    assert e.value.status == -6  # DT_ERR_WORKSPACE, nothing launched
