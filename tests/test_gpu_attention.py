"""Sparse absorbed-MLA attention (GPU) against the oracle's sparse_attention.

Inputs are bf16, so the oracle runs on exactly the same values (widened to fp64). Tolerance,
derived from the kernel's arithmetic. For head h of row t, with A_j = sum_i |q_i kv_ji| and
c = |sm_scale| log2(e): every base-2 score x_j carries an absolute error of at most
d = c * 576 * 2^-24 * max_j A_j (fp32 accumulation of exact bf16 products, then one scaling),
so every weight exp2(x_j - m) is off by a relative e = 2 ln2 d + 2^-21 at most. The value
product takes the weights rounded to bf16 (8 significant bits: unit roundoff 2^-8) and
accumulates in fp32; the normaliser sums the fp32 weights; the output is rounded to bf16
(2^-8). Hence per element
    |out - ref| <= 2^-8 |ref| + (2^-8 + 2e + 2^-20) * sum_j w_j |kv_jc| + 1e-30
with w the exact weights, and |lse - ref| <= ln2 (2 d) + 2 e + 2^-18 + 2^-22 |ref|.
Empty rows must be exactly zero with lse -inf; two calls must agree bit for bit.
"""

import numpy as np
import pytest

from oracle import oracle as orc
import gen
import parity

pytestmark = pytest.mark.gpu

DK, DV = 576, 512


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_attention_indexer_dsa_amd as dsa
    dsa.load()


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _check(q, kv, idx, lens, sm, out, lse, rows):
    """q [T,H,DK], kv [S,DK] (fp64 of the bf16 inputs), idx [T,K]; out/lse from the GPU."""
    T, H, _ = q.shape
    S = kv.shape[0]
    K = idx.shape[1]
    c = abs(sm) * np.log2(np.e)
    for t in rows:
        n = K if lens is None else max(0, min(int(lens[t]), K))
        sl = idx[t, :n]
        sel = sl[(sl >= 0) & (sl < S)]
        want, wlse = orc.sparse_attention(q[t:t + 1], kv, idx[t:t + 1], sm, dv=DV,
                                          lengths=None if lens is None else lens[t:t + 1])
        got = out[t].astype(np.float64)
        if sel.size == 0:
            assert np.all(got == 0.0), t
            assert np.all(np.isneginf(lse[t])), t
            continue
        ent = kv[sel]
        s = sm * (q[t] @ ent.T)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        A = np.abs(q[t]) @ np.abs(ent).T
        d = c * DK * 2.0 ** -24 * A.max(axis=1)
        e = 2 * np.log(2) * d + 2.0 ** -21
        B = w @ np.abs(ent[:, :DV])
        tol = 2.0 ** -8 * np.abs(want[0]) + (2.0 ** -8 + 2 * e + 2.0 ** -20)[:, None] * B + 1e-30
        ok = np.abs(got - want[0]) <= tol       # false for a NaN
        assert ok.all(), (t, np.argwhere(~ok)[:4], got[~ok][:4], want[0][~ok][:4])
        ltol = np.log(2) * 2 * d + 2 * e + 2.0 ** -18 + 2.0 ** -22 * np.abs(wlse[0])
        assert np.all(np.abs(lse[t].astype(np.float64) - wlse[0]) <= ltol), (t, lse[t][:4], wlse[0][:4])


def _case(T, H, S, topk, seed, lengths=False, bad_slots=True, scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((T, H, DK)) * scale).astype(np.float32)
    kv = rng.standard_normal((S, DK)).astype(np.float32)
    idx = np.full((T, topk), -1, np.int32)
    for t in range(T):
        k = int(rng.integers(0, topk + 1)) if t % 5 else topk
        if S > 0 and k > 0:
            idx[t, :k] = rng.choice(S, size=k, replace=k > S)
        if bad_slots and t % 3 == 1 and topk > 2:
            pos = rng.choice(topk, size=2, replace=False)
            idx[t, pos] = [S + int(rng.integers(0, 5)), -7]          # out of range: empty slots
        idx[t] = idx[t, rng.permutation(topk)]                         # empty slots anywhere
    lens = rng.integers(0, topk + 1, T).astype(np.int32) if lengths else None
    return q, kv, idx, lens


def _run(q, kv, idx, lens, sm):
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    qd, kvd = _bf16(q).cuda(), _bf16(kv).cuda()
    idd = torch.from_numpy(idx).cuda()
    ld = torch.from_numpy(lens).cuda() if lens is not None else None
    out, lse = dsa.sparse_attention(qd, kvd, idd, sm_scale=sm, lengths=ld)
    out2, lse2 = dsa.sparse_attention(qd, kvd, idd, sm_scale=sm, lengths=ld)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)   # deterministic
    return (qd.float().cpu().numpy().astype(np.float64), kvd.float().cpu().numpy().astype(np.float64),
            out.float().cpu().numpy(), lse.cpu().numpy())


@pytest.mark.parametrize("T, H, S, topk, lengths", [
    (9, 16, 40, 32, False),        # one tile; three of four waves idle (H = 16)
    (13, 64, 300, 100, True),      # ragged last tile, supplied lengths
    (17, 80, 500, 33, False),      # heads past 64: a second workgroup per token with one wave
    (21, 48, 700, 96, True),       # the second wave pair half past the heads (its other wave idle)
    (8, 128, 1000, 7, True),
    (11, 64, 64, 1, False),        # one slot
    (5, 32, 2000, 512, True),      # many tiles
    (3, 64, 6000, 2048, False),    # 64 tiles: the two gather buffers alternate 32 times
])
def test_random_selections(T, H, S, topk, lengths):
    sm = 1.0 / np.sqrt(DK)
    q, kv, idx, lens = _case(T, H, S, topk, T * 1000 + H + topk, lengths=lengths)
    qd, kvd, out, lse = _run(q, kv, idx, lens, sm)
    _check(qd, kvd, idx, lens, sm, out, lse, range(T))


def test_token_groups_across_xcds():
    # 1000 tokens: 16 groups of 64 consecutive tokens dealt to the XCDs in turn, the last one
    # ragged (40 tokens), with 128 heads (two workgroups per token); rows sampled from every group
    sm = 1.0 / np.sqrt(DK)
    T = 1000
    q, kv, idx, lens = _case(T, 128, 3000, 64, 4242, lengths=True)
    qd, kvd, out, lse = _run(q, kv, idx, lens, sm)
    _check(qd, kvd, idx, lens, sm, out, lse, sorted(set(range(0, T, 7)) | {63, 64, 959, 960, T - 1}))


def test_edge_rows():
    # every slot empty, all lengths 0, S = 0, and a large score range (weights far below the max)
    sm = 0.05
    q, kv, idx, _ = _case(6, 16, 50, 40, 7)
    idx[0] = -1
    idx[1] = 50 + np.arange(40)
    qd, kvd, out, lse = _run(q, kv, idx, np.zeros(6, np.int32), sm)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))
    qd, kvd, out, lse = _run(q, kv, idx, None, sm)
    _check(qd, kvd, idx, None, sm, out, lse, range(6))
    q0, kv0, idx0, _ = _case(4, 16, 0, 8, 8)
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    out0, lse0 = dsa.sparse_attention(_bf16(q0).cuda(), torch.empty((0, DK), dtype=torch.bfloat16, device="cuda"),
                                      torch.from_numpy(idx0).cuda(), sm_scale=sm)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0) and torch.all(torch.isneginf(lse0))
    q, kv, idx, _ = _case(7, 32, 400, 64, 9, scale=12.0)
    qd, kvd, out, lse = _run(q, kv, idx, None, 0.2)
    _check(qd, kvd, idx, None, 0.2, out, lse, range(7))


def test_after_selection():
    # attention over a real selection: the indexer's top-k indices and lengths (two packed
    # documents, KPool 4 with its tail), queries and latent entries drawn beside them
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    cfg = dict(precision="fp8", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True, kpool=4,
               kpool_tail=True)
    inp = gen.small(52, [150, 90], 64, 128, layernorm=True, rope_dim=64, kpool=4)
    inp["H"], inp["D"] = 64, 128
    g = parity.gpu_pipeline(inp, cfg, 24, keep_device=True)
    idx, lens = g["indices"], g["lengths"]
    T = idx.shape[0]
    rng = np.random.default_rng(53)
    q = rng.standard_normal((T, 64, DK)).astype(np.float32)
    kv = rng.standard_normal((T, DK)).astype(np.float32)
    sm = 1.0 / np.sqrt(DK)
    qd, kvd, out, lse = _run(q, kv, idx.cpu().numpy(), lens.cpu().numpy(), sm)
    _check(qd, kvd, idx.cpu().numpy(), lens.cpu().numpy(), sm, out, lse, range(T))


def test_full_size_sampled():
    # 2 x 4096 tokens, 64 heads, top-512 causal selections of each document; 48 rows sampled
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    L, B, H, topk = 4096, 2, 64, 512
    T = L * B
    g = torch.Generator(device="cuda").manual_seed(61)
    q = torch.randn((T, H, DK), generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn((T, DK), generator=g, device="cuda").to(torch.bfloat16)
    # causal selections: for token u of document b, min(topk, u+1) distinct earlier tokens
    pos = torch.arange(T, device="cuda") % L
    start = torch.arange(T, device="cuda") - pos
    r = torch.rand((T, topk), generator=g, device="cuda")
    cand = (r * (pos[:, None] + 1).float()).long().clamp(max=L - 1)
    idx = (start[:, None] + torch.minimum(cand, pos[:, None])).to(torch.int32)
    lens = torch.clamp(pos + 1, max=topk).to(torch.int32)
    out, lse = dsa.sparse_attention(q, kv, idx, sm_scale=1.0 / np.sqrt(DK), lengths=lens)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(62).choice(T, 40, replace=False).tolist()) | {0, 1, L - 1, L, T - 1})
    ri = torch.as_tensor(rows, device="cuda")
    qs = q.index_select(0, ri).float().cpu().numpy().astype(np.float64)
    idxs = idx.index_select(0, ri).cpu().numpy()
    _check(qs, kv.float().cpu().numpy().astype(np.float64), idxs, lens.index_select(0, ri).cpu().numpy(),
           1.0 / np.sqrt(DK), out.index_select(0, ri).float().cpu().numpy(), lse.index_select(0, ri).cpu().numpy(),
           range(len(rows)))
