"""Softmax over the selected scores (GPU) against the oracle's selection_softmax.

The kernel's input is the top-k score output itself, so the oracle runs on exactly the
same fp32 values (widened to fp64). Tolerance, derived from the fp32 arithmetic: for
entry j with d_j = s_j - m, the subtraction (relative 2^-24 of |d_j|, i.e. a factor
exp(|d_j| 2^-24)), expf (within 2 ulp), a per-lane sequential sum of topk/64 terms plus a
6-step tree, and one division give |p_gpu - p| <= (16 + topk/64 + |d_j|) 2^-23 p, plus an
absolute 1e-37 where the exponential falls into fp32 subnormals. Padding must be exactly 0
and two calls must agree bit for bit.
"""

import numpy as np
import pytest

from oracle import oracle as orc
import gen
import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_attention_indexer_dsa_amd as dsa
    dsa.load()


def _check_rows(scores, probs):
    T, topk = scores.shape
    for t in range(T):
        s = scores[t].astype(np.float64)
        want = orc.selection_softmax(s)
        got = probs[t].astype(np.float64)
        pad = ~(s > -np.inf)
        assert np.all(got[pad] == 0.0), t
        if not (~pad).any():
            assert np.all(got == 0.0), t
            continue
        d = np.abs(s - np.max(s[~pad]))
        tol = (16 + topk / 64 + np.where(pad, 0, d)) * 2.0 ** -23 * want + 1e-37
        ok = np.abs(got - want) <= tol          # false for a NaN
        assert ok.all(), (t, np.flatnonzero(~ok)[:5], got[~ok][:5], want[~ok][:5])


def _crafted(T, topk, rng):
    rows = np.full((T, topk), -np.inf, np.float32)
    for t in range(T):
        kind = t % 8
        n = int(rng.integers(0, topk + 1)) if kind != 7 else topk
        if kind == 0:
            v = rng.standard_normal(n) * 3
        elif kind == 1:
            v = np.full(n, 2.5)                                  # equal scores: uniform
        elif kind == 2:
            v = rng.standard_normal(n) * 60                      # wide range: most weights underflow
        elif kind == 3:
            v = rng.standard_normal(n) * 1e-3 + 1e4              # large offset, small spread
        elif kind == 4:
            n = 0                                                # nothing selected
            v = np.zeros(0)
        elif kind == 5:
            n = min(n, 1)                                        # one entry: weight 1
            v = rng.standard_normal(n)
        elif kind == 6:
            v = -np.abs(rng.standard_normal(n)) * 1e30          # huge magnitudes
        else:
            v = rng.standard_normal(n)                           # full row
        rows[t, :n] = np.sort(v.astype(np.float32))[::-1]
    return rows


@pytest.mark.parametrize("T, topk", [(64, 1), (200, 7), (128, 64), (96, 512), (40, 2048), (9, 4096)])
def test_crafted_rows(T, topk):
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    rng = np.random.default_rng(T * 31 + topk)
    rows = _crafted(T, topk, rng)
    s = torch.from_numpy(rows).cuda()
    p1 = dsa.selection_softmax(s)
    p2 = dsa.selection_softmax(s)
    torch.cuda.synchronize()
    a, b = p1.cpu().numpy(), p2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))          # deterministic
    _check_rows(rows, a)
    # in place gives the same bits
    s2 = s.clone()
    dsa.selection_softmax(s2, out=s2)
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), a.view(np.uint32))


@pytest.mark.parametrize("kp", [1, 4])
def test_after_selection(kp):
    # the softmax of a real selection (scores from the scoring and top-k kernels)
    import sparse_attention_indexer_dsa_amd as dsa
    cfg = dict(precision="fp8", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True, kpool=kp,
               kpool_tail=True)
    inp = gen.small(41 + kp, [37, 100, 5, 0, 130], 64, 128, layernorm=True, rope_dim=64, kpool=kp)
    inp["H"], inp["D"] = 64, 128
    g = parity.gpu_pipeline(inp, cfg, 24, keep_device=True)
    p = dsa.selection_softmax(g["scores"]).cpu().numpy()
    sc = g["scores"].cpu().numpy()
    _check_rows(sc, p)
    n = np.sum(sc > -np.inf, axis=1)
    assert np.all(np.abs(np.sum(p, axis=1)[n > 0] - 1.0) < 1e-5)


def test_full_size_rows():
    # the batch2x4096 selection shape (8192 rows of 512) and the THD one (rows of 2048), sampled
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    for T, topk in ((8192, 512), (32768, 2048)):
        g = torch.Generator(device="cuda").manual_seed(T)
        s = torch.randn((T, topk), generator=g, device="cuda") * 4
        s, _ = torch.sort(s, dim=1, descending=True)
        lens = torch.randint(0, topk + 1, (T,), generator=g, device="cuda")
        s[torch.arange(topk, device="cuda")[None, :] >= lens[:, None]] = -float("inf")
        p = dsa.selection_softmax(s)
        torch.cuda.synchronize()
        rows = np.random.default_rng(T).choice(T, size=64, replace=False)
        ri = torch.as_tensor(rows, device="cuda")
        _check_rows(s.index_select(0, ri).cpu().numpy(), p.index_select(0, ri).cpu().numpy())
