"""The oracle's scoring, selection and expansion against exact brute force (CPU).

``oracle.exact.brute_force`` enumerates candidates and heads with exact
rationals and sorts exactly; ``oracle.oracle.index_topk`` works in float64 with
numpy. They share no code. Hundreds of seeded tiny cases cover several
documents (including empty ones and ones shorter than the pool), kpool 1..4,
tail on and off, negative weights, zero scores and the three precisions.
"""

import numpy as np
import pytest

from oracle import exact
from oracle import formats as fm
from oracle import oracle as orc


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    n_docs = int(rng.integers(1, 4))
    docs = [int(v) for v in rng.integers(0, 9, n_docs)]
    if sum(docs) == 0:
        docs[0] = 3
    T = sum(docs)
    H = int(rng.integers(1, 5))
    precision = ["bf16", "fp8", "mxfp8"][seed % 3]
    D = 32 if precision == "mxfp8" else int(rng.choice([1, 2, 4, 8]))
    kp = int(rng.integers(1, 5))
    topk = int(rng.choice([1, 2, 3, 5, 100]))
    tail = bool(rng.integers(0, 2))
    sm_scale = float(rng.choice([1.0, 0.5, 0.125, 3.0]))
    cu = np.concatenate([[0], np.cumsum(docs)]).astype(np.int64)
    qc = rng.standard_normal((T, H, D)).astype(np.float32)
    kc = rng.standard_normal((T, D)).astype(np.float32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    if seed % 7 == 0:
        w[:, 0] = 0.0                      # a zero weight
    qo, qs = orc.quantize(qc, precision)
    q = orc.dequantize(qo, qs, precision)
    if kp == 1:
        ko, ks = orc.quantize(kc, precision)
        k = orc.dequantize(ko, ks, precision)
        cu_pools = None
    else:
        gate = fm.bf16_bits(rng.standard_normal(T).astype(np.float32))
        bias = (0.14 * rng.standard_normal(kp)).astype(np.float32)
        pooled, cu_pools = orc.kpool(kc, cu, gate, bias, kp)
        ko, ks = orc.quantize(pooled, precision)
        k = orc.dequantize(ko, ks, precision) if pooled.shape[0] else np.zeros((0, D))
    return dict(q=q, k=k, w=w.astype(np.float64), cu=cu, topk=topk, sm=sm_scale, kp=kp,
                cu_pools=cu_pools, tail=tail, T=T)


@pytest.mark.parametrize("seed", range(240))
def test_oracle_matches_brute_force(seed):
    c = _case(seed)
    got = orc.index_topk(c["q"], c["k"], c["w"], c["cu"], c["topk"], c["sm"], c["kp"],
                         c["cu_pools"], c["tail"])
    want = exact.brute_force(c["q"], c["k"], c["w"], c["cu"], c["topk"], c["sm"], c["kp"], c["tail"])
    assert len(got) == c["T"] == len(want)
    for t in range(c["T"]):
        g, e = got[t], want[t]
        Ie = np.array([float(v) for v in e["I"]])
        assert g["I"].shape == Ie.shape
        assert np.all(np.abs(g["I"] - Ie) <= 1e-12 * g["M"] + 1e-300)
        assert list(g["sel"]) == list(e["sel"]), (t, g["sel"], e["sel"])
        assert list(g["indices"]) == list(e["indices"])
        assert g["length"] == e["length"]
        if c["kp"] > 1:
            assert list(g["tokens"]) == list(e["tokens"])


def test_dense_outputs_padding():
    c = _case(5)
    res = orc.index_topk(c["q"], c["k"], c["w"], c["cu"], c["topk"], c["sm"], c["kp"],
                         c["cu_pools"], c["tail"])
    idx, scr, lng, tok = orc.dense_outputs(res, c["T"], c["topk"], c["kp"])
    for t in range(c["T"]):
        n = res[t]["sel"].size
        assert np.all(idx[t, n:] == -1) and np.all(np.isneginf(scr[t, n:]))
        assert lng[t] == res[t]["length"]
