"""GPU parity of dt_sample_rows (exact target-sample matching at T > 0) against
the oracle, and of the sampled verification round (dt_sample_rows followed by
dt_accept_path).

The kernel ranks the vocabulary by an fp32 rescaling of the oracle's float64
Gumbel score (log2 units instead of natural ones), so its pick equals the
oracle's except where two candidates' exact scores lie within fp32 rounding of
each other. The tolerance for such a near tie is derived from the kernel's
arithmetic: one fused multiply-add and two hardware base-2 logarithms
(1-ulp class) per candidate, i.e. a relative 2^-22 of |l| log2(e) / T + 24 (the
largest magnitude of the log2-domain score) per candidate, doubled for the
two candidates compared and converted back to natural-log units. Every
mismatch must be such a near tie; a wrong generator word, counter, uniform map
or temperature scaling shifts scores by far more and fails.
"""

import numpy as np
import pytest
from scipy import stats

import draft_tree_verification_dt_amd as dt
from _helpers import dev_i32, require_gpu, tree
from gen import rng as grng, tensors as gten
from oracle import argmax as oarg, sample as osmp, walk as owalk

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _tol(logits_rows, T):
    lmax = np.abs(np.asarray(logits_rows, np.float64)).max(axis=1)
    return 2 * 2.0 ** -22 * (lmax * LOG2E / T + 24.0) / LOG2E


def check_samples(got, logits_host, T, seed, offset, row_ids=None):
    """Every GPU pick is the oracle's, or within the near-tie tolerance of its score.
    Returns the number of near-tie mismatches."""
    lg = np.asarray(logits_host)
    rows = lg.shape[0]
    ids = np.arange(rows) if row_ids is None else np.asarray(row_ids)
    got = np.asarray(got, np.int64)
    assert got.shape == (rows,)
    assert ((got >= 0) & (got < lg.shape[1])).all()
    tol = _tol(lg, T)
    mism = 0
    for r0 in range(0, rows, 32):
        r1 = min(rows, r0 + 32)
        s = osmp.perturbed_scores(lg[r0:r1], T, ids[r0:r1], seed, offset)
        best = np.argmax(s, axis=1)
        for k in range(r1 - r0):
            g = got[r0 + k]
            if g != best[k]:
                gap = s[k, best[k]] - s[k, g]
                assert gap <= tol[r0 + k], (f"row {ids[r0 + k]}: gpu {g} oracle {best[k]} score gap {gap:.3e} "
                                            f"> near-tie tolerance {tol[r0 + k]:.3e}")
                mism += 1
    assert mism <= max(2, rows // 100), f"{mism} near ties in {rows} rows is implausibly many"
    return mism


def _sample_dev(x_host, T, seed, offset, stride_pad=0):
    import torch

    rows, vocab = x_host.shape
    buf = torch.full((rows, vocab + stride_pad), float("inf"), dtype=torch.float32, device="cuda")
    buf[:, :vocab] = torch.from_numpy(x_host).cuda()
    out = dt.dt_sample_rows(buf[:, :vocab], T, seed, offset)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("rows,vocab", [(1, 1), (3, 7), (16, 1024), (5, 4097), (300, 1000), (16, 151936),
                                        (1, 262144), (2, 10 ** 6)])
@pytest.mark.parametrize("T", [0.6, 1.0])
def test_sample_matches_oracle(rows, vocab, T):
    require_gpu()
    r = grng.stream(rows, vocab, "smp")
    x = (r.standard_normal((rows, vocab), dtype=np.float32) * np.float32(2.0))
    seed, offset = int(r.integers(0, 1 << 63)), int(r.integers(0, 1 << 63))
    print(f"sample rows={rows} vocab={vocab} T={T}", flush=True)
    check_samples(_sample_dev(x, T, seed, offset), x, T, seed, offset)


@pytest.mark.parametrize("seed", range(2))
def test_sample_random_shapes(seed):
    """Seeded random row counts (chunked, one 512-thread workgroup per row, and
    256-thread workgroups from eight rows per CU on), vocabulary sizes, row
    strides and temperatures against the oracle's perturbed scores."""
    require_gpu()
    r = grng.stream(seed, "sample-sweep")
    for case in range(5):
        rows = int(r.choice([1, 9, 255, 256, 700, 2100]))
        vocab = int(r.integers(1, max(2, min(120000, 2_000_000 // rows))))
        pad = int(r.integers(0, 5))
        T = float(r.choice([0.3, 1.0, 1.7]))
        x = (r.standard_normal((rows, vocab), dtype=np.float32) * np.float32(2.0))
        seed_, offset = int(r.integers(0, 1 << 63)), int(r.integers(0, 1 << 63))
        print(f"sample sweep {seed}.{case} rows={rows} vocab={vocab} pad={pad} T={T}", flush=True)
        check_samples(_sample_dev(x, T, seed_, offset, stride_pad=pad), x, T, seed_, offset)


@pytest.mark.parametrize("pad", [1, 3, 4])
def test_sample_strided_rows(pad):
    """Row strides that are not a multiple of four take the scalar path; same draws."""
    require_gpu()
    x = grng.stream(pad, "smp-stride").standard_normal((37, 5003), dtype=np.float32)
    print(f"sample stride pad={pad}", flush=True)
    check_samples(_sample_dev(x, 1.0, 99, 5, stride_pad=pad), x, 1.0, 99, 5)


def test_sample_full_size_round():
    """256 rows x 151936 (the B=256 round), every row against the oracle."""
    import torch

    require_gpu()
    x = gten.device_logits(256, 151936, 23, "smp-full")
    print("sample 256 x 151936", flush=True)
    out = dt.dt_sample_rows(x, 1.0, 0xDEADBEEF12345, 3)
    torch.cuda.synchronize()
    check_samples(out.cpu().numpy(), x.cpu().numpy(), 1.0, 0xDEADBEEF12345, 3)


def test_sample_full_size_batch_all_rows():
    """2048 rows x 151936 (ragged and long-context batches), every row against the oracle."""
    import torch

    require_gpu()
    x = gten.device_logits(2048, 151936, 29, "smp-batch")
    print("sample 2048 x 151936", flush=True)
    out = dt.dt_sample_rows(x, 1.0, 77, 1 << 40)
    torch.cuda.synchronize()
    check_samples(out.cpu().numpy(), x.cpu().numpy(), 1.0, 77, 1 << 40)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_sample_law(T):
    """Frequencies of the GPU's picks over many rows of the same logits match
    softmax(l / T) (chi-square): the kernel's draw law, independent of the oracle."""
    import torch

    require_gpu()
    lg = (grng.stream(3, "law").standard_normal(12) * 1.5).astype(np.float32)
    rows = 30000
    x = torch.from_numpy(np.tile(lg, (rows, 1))).cuda()
    print(f"sample law T={T}", flush=True)
    picks = dt.dt_sample_rows(x, T, 1234, 17).cpu().numpy()
    counts = np.bincount(picks, minlength=lg.size)
    p = osmp.target_distribution(lg, T)
    assert stats.chisquare(counts, rows * p).pvalue > 1e-6


def test_sample_cold_temperature_is_greedy():
    require_gpu()
    r = grng.stream(8, "cold-gpu")
    x = r.standard_normal((64, 151936)).astype(np.float32)
    for i in range(64):
        x[i, r.integers(0, 151936)] = x[i].max() + np.float32(0.05)
    print("sample cold", flush=True)
    np.testing.assert_array_equal(_sample_dev(x, 1e-4, 5, 6), oarg.argmax_rows(x))


def test_sample_streams_change_with_offset_and_seed():
    import torch

    require_gpu()
    x = torch.zeros((64, 4096), dtype=torch.float32, device="cuda")
    a = dt.dt_sample_rows(x, 1.0, 1, 0).cpu().numpy()
    b = dt.dt_sample_rows(x, 1.0, 1, 0).cpu().numpy()
    c = dt.dt_sample_rows(x, 1.0, 1, 1).cpu().numpy()
    d = dt.dt_sample_rows(x, 1.0, 2, 0).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    assert (a != c).mean() > 0.9 and (a != d).mean() > 0.9
    check_samples(a, x.cpu().numpy(), 1.0, 1, 0)


@pytest.mark.parametrize("seed", range(4))
def test_sampled_verification_round(seed):
    """T = 1 round on a ragged batch of trees: GPU samples (checked against the
    oracle) feed the GPU walk, which must equal the oracle walk over the same
    samples bit for bit."""
    import torch

    require_gpu()
    r = grng.stream(seed, "t1-round")
    vocab = 96
    nodes = [int(r.integers(1, 80)) for _ in range(5)]
    offs = np.concatenate([[0], np.cumsum(nodes)]).astype(np.int32)
    parents, tokens, lgs = [], [], []
    for s, n in enumerate(nodes):
        p, t = tree(["recursive", "deep", "chain"][s % 3], n, 50 + seed * 10 + s, vocab=vocab)
        lg = gten.logits(r, n, vocab)
        for u in gten.plant(r, lg, p, t, p=0.9, pick="random"):
            row = lg[u]
            row[np.argmax(row)] += np.float32(5.0)  # the planted token is now well ahead: accepted with high probability
        parents.append(p)
        tokens.append(t)
        lgs.append(lg)
    parent = np.concatenate(parents).astype(np.int32)
    token = np.concatenate(tokens).astype(np.int32)
    logits = np.concatenate(lgs).astype(np.float32)
    T, rseed, roff = 1.0, 1000 + seed, 7
    print(f"sampled round seed={seed} nodes={nodes}", flush=True)
    smp = dt.dt_sample_rows(torch.from_numpy(logits).cuda(), T, rseed, roff)
    path, L, bonus = dt.dt_accept_path(offs, dev_i32(parent), dev_i32(token), smp)
    torch.cuda.synchronize()
    smp_h = smp.cpu().numpy()
    check_samples(smp_h, logits, T, rseed, roff)
    want = owalk.batch_accept_path(parent, token, smp_h, offs)
    path_h, L_h, b_h = path.cpu().numpy(), L.cpu().numpy(), bonus.cpu().numpy()
    accepted = 0
    for s, (wp, wl, wb) in enumerate(want):
        a = offs[s]
        assert L_h[s] == wl and b_h[s] == wb, s
        assert list(path_h[a:a + wl + 1]) == wp, s
        assert (path_h[a + wl + 1:offs[s + 1]] == -1).all()
        accepted += wl
    assert accepted > 0
