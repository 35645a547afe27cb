"""The parity checker itself (CPU): results built from the oracle pass it, and planted faults
(a NaN in any compared value, a wrong score, a swapped index, a wrong length) fail it.

The fake "GPU" outputs are the oracle's own scores rounded to fp32 and re-ordered by
(fp32 score descending, index ascending), the order the library writes.
"""

import numpy as np
import pytest

from oracle import oracle as orc
import gen
import parity


def _fake_gpu(seed, kp=1, topk=6):
    docs = [37, 0, 20, 9]
    H, D = 16, 64
    inp = gen.small(seed, docs, H, D, kpool=kp)
    inp["H"], inp["D"] = H, D
    cfg = dict(precision="bf16", preprocess=False, kpool=kp, kpool_tail=True)
    o = parity.oracle_operands(inp, cfg)
    res = orc.index_topk(o["q_deq"], o["k_deq"], inp["w"].astype(np.float64), inp["cu_seqlens"], topk,
                         1.0, kp, o.get("cu_pools"), True)
    T = inp["q"].shape[0]
    cu = np.asarray(inp["cu_seqlens"], np.int64)
    doc, pos = orc.geometry(cu, T)
    base = cu if kp == 1 else np.asarray(o["cu_pools"], np.int64)
    width = topk if kp == 1 else topk * kp + kp - 1
    g = {"ws": {}, "scores": np.full((T, topk), -np.inf, np.float32), "indices": np.full((T, width), -1, np.int32),
         "lengths": np.zeros(T, np.int32)}
    if kp > 1:
        g["pool_indices"] = np.full((T, topk), -1, np.int32)
        g["cu_pools"] = o["cu_pools"]
    for t, r in res.items():
        ws = r["I"].astype(np.float32)
        g["ws"][t] = ws
        # the fp32 top-k of the fp32 row, in (score desc, index asc) order
        order = np.lexsort((np.arange(ws.size), -ws.astype(np.float64)))[:min(topk, ws.size)]
        n = order.size
        g["scores"][t, :n] = ws[order]
        b = doc[t]
        if kp == 1:
            g["indices"][t, :n] = base[b] + order
            g["lengths"][t] = n
        else:
            g["pool_indices"][t, :n] = base[b] + order
            toks = orc.expand(order, int(pos[t]), kp, int(cu[b]), True)
            g["indices"][t, :toks.size] = toks
            g["lengths"][t] = toks.size
    return inp, cfg, res, g, topk


@pytest.mark.parametrize("kp", [1, 3])
def test_oracle_built_results_pass(kp):
    inp, cfg, res, g, topk = _fake_gpu(1, kp)
    parity.compare_rows(g, res, inp, cfg, topk, range(inp["q"].shape[0]))
    parity.check_invariants(g, inp, cfg, topk)


def _row_with_unselected(res, topk):
    for t, r in res.items():
        if r["I"].size > topk + 2:
            return t
    raise AssertionError("no row with unselected candidates")


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_nan_in_unselected_workspace_slot_fails(sign):
    inp, cfg, res, g, topk = _fake_gpu(2)
    t = _row_with_unselected(res, topk)
    unsel = np.setdiff1d(np.arange(res[t]["I"].size), res[t]["sel"])
    g["ws"][t] = g["ws"][t].copy()
    g["ws"][t][unsel[0]] = np.float32(sign * np.nan)
    with pytest.raises(AssertionError):
        parity.compare_rows(g, res, inp, cfg, topk, [t])


def test_nan_in_selected_score_fails():
    inp, cfg, res, g, topk = _fake_gpu(3)
    t = _row_with_unselected(res, topk)
    g["scores"][t, 0] = np.nan
    with pytest.raises(AssertionError):
        parity.check_invariants(g, inp, cfg, topk)


def test_score_outside_tolerance_fails():
    inp, cfg, res, g, topk = _fake_gpu(4)
    t = _row_with_unselected(res, topk)
    r = res[t]
    c = int(np.setdiff1d(np.arange(r["I"].size), r["sel"])[0])
    g["ws"][t] = g["ws"][t].copy()
    g["ws"][t][c] += np.float32(1e-3 * r["M"][c] + 1e-6)     # 100x the bf16 tolerance
    with pytest.raises(AssertionError):
        parity.compare_rows(g, res, inp, cfg, topk, [t])


def test_wrong_selection_fails():
    inp, cfg, res, g, topk = _fake_gpu(5)
    t = _row_with_unselected(res, topk)
    r = res[t]
    # replace the best selected candidate by the worst candidate of the row
    worst = int(np.argmin(r["I"]))
    g["indices"][t, 0] = int(r["indices"][0] - r["sel"][0]) + worst
    g["scores"][t, 0] = g["ws"][t][worst]
    with pytest.raises(AssertionError):
        parity.compare_rows(g, res, inp, cfg, topk, [t])


def test_wrong_length_fails():
    inp, cfg, res, g, topk = _fake_gpu(6)
    t = _row_with_unselected(res, topk)
    g["lengths"][t] -= 1
    with pytest.raises(AssertionError):
        parity.compare_rows(g, res, inp, cfg, topk, [t])
