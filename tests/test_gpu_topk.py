"""Selection kernel on crafted score rows (GPU), against the oracle's row selection.

The workspace rows are written directly, so every row's scores are exact fp32 values and
the selection must match the oracle exactly: the same local indices in the same order
(score descending, index ascending; -0 counts as +0), the scores themselves, -1 / -inf
padding and the lengths. Row patterns reach every branch of the kernel: smooth rows (bin
ordering), ties at the threshold with fewer taken than exist, a bin above the threshold
holding more than its ordering limit, a clustered threshold bin (radix select), an outlier
that crushes the linear bins, constant rows, small integers (ties everywhere), signed
zeros, negative rows and magnitudes from subnormal to 1e30. Document lengths select each
of the launch shapes (up to 1024, 2048, 4096, 8192, 16384 and 32768 candidates per row), and
rows of one call fall in several launch size classes, over more than 64 documents.
"""

import numpy as np
import pytest

from oracle import oracle as orc

pytestmark = pytest.mark.gpu

NPAT = 10


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_attention_indexer_dsa_amd as dsa
    dsa.load()


def _row(p, cand, topk, rng):
    """Scores of one row with pattern p (fp32)."""
    v = (rng.standard_normal(cand) * 3.0).astype(np.float32)
    k = min(topk, cand)
    desc = np.sort(v)[::-1]
    if p == 1:      # ties straddling the threshold: fewer taken than equal
        v[rng.choice(cand, size=min(cand, 20), replace=False)] = desc[k - 1]
    elif p == 2:    # one bin above the threshold holding many equal keys
        v[rng.choice(cand, size=min(cand, 100), replace=False)] = desc[k // 4]
    elif p == 3:    # a clustered threshold
        v[rng.choice(cand, size=min(cand, 300), replace=False)] = desc[k - 1]
    elif p == 4:    # one outlier
        v[rng.integers(cand)] = np.float32(1e30)
    elif p == 5:    # constant
        v[:] = np.float32(1.25)
    elif p == 6:    # small integers
        v = rng.integers(0, 8, cand).astype(np.float32)
    elif p == 7:    # signed zeros with a few nonzero scores
        v = np.where(rng.random(cand) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        m = rng.random(cand) < 0.1
        v[m] = rng.standard_normal(int(m.sum())).astype(np.float32)
    elif p == 8:    # all negative
        v = -np.abs(v) - np.float32(1.0)
    elif p == 9:    # magnitudes from subnormal to 1e30
        v = (rng.standard_normal(cand) * 10.0 ** rng.integers(-44, 31, cand)).astype(np.float32)
    return v


def _sample_rows(docs, topk, rng):
    cu = np.concatenate([[0], np.cumsum(docs)])
    rows = set()
    for b, n in enumerate(docs):
        lo = int(cu[b])
        rows |= {lo + u for u in range(max(0, n - 6), n)}
        rows |= {lo + u for u in (0, 1, 63, 64, topk - 1, topk, 4095, 4096, 8191, 8192) if 0 <= u < n}
    T = int(cu[-1])
    rows |= set(int(x) for x in rng.choice(T, size=min(T, 40), replace=False))
    return sorted(rows)


def _run(docs, topk, kp, tail, seed):
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    rng = np.random.default_rng(seed)
    docs = [int(n) for n in docs]
    cu_h = np.concatenate([[0], np.cumsum(docs)]).astype(np.int64)
    T, L = int(cu_h[-1]), max(docs)
    doc_of = np.repeat(np.arange(len(docs)), docs)
    pos = np.arange(T) - cu_h[doc_of]
    max_cand = L if kp == 1 else L // kp
    stride = (max(1, max_cand) + 63) // 64 * 64
    gen_t = torch.Generator(device="cuda").manual_seed(seed)
    flat = torch.randn(T * stride + 64, generator=gen_t, device="cuda", dtype=torch.float32) * 3.0
    ws = flat[:T * stride].view(T, stride)     # the library asks for 256 bytes beyond the rows
    rows = _sample_rows(docs, topk, rng)
    want = {}
    for i, t in enumerate(rows):
        cand = (int(pos[t]) + 1) // kp
        if cand == 0:
            continue
        v = _row(i % NPAT, cand, topk, rng)
        ws[t, :cand] = torch.from_numpy(v).cuda()
        want[t] = v
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    cu_pools = (torch.tensor(np.concatenate([[0], np.cumsum([n // kp for n in docs])]), dtype=torch.int32,
                             device="cuda") if kp > 1 else None)
    out = dsa.topk(flat, T, cu, L, topk, kpool=kp, cu_pools=cu_pools, kpool_tail=tail)
    torch.cuda.synchronize()
    host = {n: out[n].cpu().numpy() for n in out}
    # every row was handled: its length is fixed by its position alone
    cand_all = (pos + 1) // kp
    nsel_all = np.minimum(topk, cand_all)
    if kp == 1:
        assert np.array_equal(host["lengths"], nsel_all)
    else:
        tails = ((pos + 1) % kp) if tail else 0
        assert np.array_equal(host["lengths"], nsel_all * kp + tails)
    # rows left random are checked too: read back after the call
    extra = [int(x) for x in rng.choice(T, size=min(T, 16), replace=False)]
    pbase = np.concatenate([[0], np.cumsum([n // kp for n in docs])])
    for t in sorted(set(want) | set(extra)):
        b, u = int(doc_of[t]), int(pos[t])
        cand = (u + 1) // kp
        v = want[t] if t in want else ws[t, :cand].cpu().numpy()
        sel, s = orc.topk_row(v.astype(np.float64), topk)
        n = sel.size
        sc = host["scores"][t]
        assert np.array_equal(sc[:n].astype(np.float64), s), (t, sc[:8], s[:8])
        assert np.all(np.isneginf(sc[n:])), t
        if kp == 1:
            idx = host["indices"][t].astype(np.int64)
            assert np.array_equal(idx[:n] - cu_h[b], sel), (t, idx[:8], sel[:8])
            assert np.all(idx[n:] == -1), t
        else:
            pidx = host["pool_indices"][t].astype(np.int64)
            assert np.array_equal(pidx[:n] - pbase[b], sel), (t, pidx[:8], sel[:8])
            assert np.all(pidx[n:] == -1), t
            toks = orc.expand(sel, u, kp, int(cu_h[b]), tail)
            tok = host["indices"][t].astype(np.int64)
            assert np.array_equal(tok[:toks.size], toks), t
            assert np.all(tok[toks.size:] == -1), t


@pytest.mark.parametrize("L, topk", [(1000, 64), (2000, 256), (3000, 7), (4000, 512), (8000, 2048),
                                     (16000, 2048), (32768, 2048), (1500, 2048), (9000, 6000)])
def test_selection_patterns(L, topk):
    # (9000, 6000): the 8192- and 16384-candidate shapes and the fallback launch each need
    # more than 64 KB of LDS, so each raises its own limit
    _run([L], topk, 1, True, L + topk)


@pytest.mark.parametrize("tail", [True, False])
def test_selection_patterns_kpool(tail):
    _run([8000], 512, 4, tail, 11 + tail)


@pytest.mark.parametrize("kp", [1, 4])
def test_selection_many_documents(kp):
    # more than 64 documents (the row map takes them 64 at a time), empty ones, and long
    # ones whose rows fall in several launch size classes
    rng = np.random.default_rng(70 + kp)
    docs = rng.integers(0, 1500, 70)
    docs[[3, 17, 40]] = 0
    docs[[5, 66]] = [9000, 5000] if kp == 1 else [20000, 36000]
    _run(docs, 256, kp, True, 80 + kp)


@pytest.mark.parametrize("L, topk, big", [(4096, 512, 3000.0), (4096, 512, 1e30), (6000, 2048, 1e4),
                                          (1500, 2048, 1e6)])
def test_selection_outlier_rows(L, topk, big):
    # every row has one outlying score (an attention-sink-like key), some also a low one:
    # the linear bins over [min, max] crowd the rest into a few bins, and the kernel bins the
    # selected region again
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    rng = np.random.default_rng(int(L + topk + np.log10(big)))
    stride = (L + 63) // 64 * 64
    gen_t = torch.Generator(device="cuda").manual_seed(L + topk)
    flat = torch.randn(L * stride + 64, generator=gen_t, device="cuda", dtype=torch.float32) * 3.0
    ws = flat[:L * stride].view(L, stride)
    t_idx = torch.arange(L, device="cuda")
    pos = torch.as_tensor(rng.integers(0, 1 << 30, L), device="cuda") % (t_idx + 1)
    ws[t_idx, pos] = big
    low = t_idx[t_idx % 5 == 0]
    ws[low, low // 3] = -big
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    out = dsa.topk(flat, L, cu, L, topk)
    torch.cuda.synchronize()
    host = {n: out[n].cpu().numpy() for n in out}
    cand = np.arange(L) + 1
    assert np.array_equal(host["lengths"], np.minimum(topk, cand))
    rows = sorted(set(int(x) for x in rng.choice(L, size=60, replace=False)) | set(range(L - 5, L)))
    for t in rows:
        v = ws[t, :t + 1].cpu().numpy().astype(np.float64)
        sel, s = orc.topk_row(v, topk)
        n = sel.size
        assert np.array_equal(host["indices"][t][:n].astype(np.int64), sel), t
        assert np.array_equal(host["scores"][t][:n].astype(np.float64), s), t


def test_lds_limit_kept_for_captured_launch():
    # A top-k call whose 16384-candidate launch needs ~140 KB of dynamic LDS is captured into
    # a graph (one stream); then an eager call needing ~74 KB in the same kernels runs; the
    # graph is replayed (twice, with eager work between). The kernels' LDS limit must still
    # cover the captured launch: every replay equals the eager result of the captured call,
    # byte for byte. The smaller call's selection is the prefix of the larger one's (both
    # are ordered by score descending, then index ascending).
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    L, big, small = 9000, 8500, 6000
    stride = (L + 63) // 64 * 64
    gen_t = torch.Generator(device="cuda").manual_seed(123)
    flat = torch.randn(L * stride + 64, generator=gen_t, device="cuda", dtype=torch.float32) * 3.0
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    ref = dsa.topk(flat, L, cu, L, big)
    torch.cuda.synchronize()
    out = dsa._alloc_outputs(None, L, big, 1, "cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dsa.topk(flat, L, cu, L, big, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dsa.topk(flat, L, cu, L, big, out=out)
    for rep in range(2):
        for n in out:
            out[n].fill_(7)
        sm = dsa.topk(flat, L, cu, L, small)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in ("indices", "scores", "lengths"):
            assert torch.equal(out[n].view(torch.int32), ref[n].view(torch.int32)), (rep, n)
        assert torch.equal(sm["indices"], ref["indices"][:, :small]), rep
        assert torch.equal(sm["scores"].view(torch.int32), ref["scores"][:, :small].view(torch.int32)), rep
    # the captured call's rows against the oracle on a few rows
    host_i, host_s = ref["indices"].cpu().numpy(), ref["scores"].cpu().numpy()
    for t in (0, 4000, 8191, 8192, 8600, L - 1):
        v = flat[t * stride:t * stride + t + 1].cpu().numpy().astype(np.float64)
        sel, s = orc.topk_row(v, big)
        assert np.array_equal(host_i[t][:sel.size].astype(np.int64), sel), t
        assert np.array_equal(host_s[t][:sel.size].astype(np.float64), s), t
