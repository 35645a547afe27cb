"""The five indexer workloads at full size, in the launch configuration bench.py times (GPU).

Inputs come from tests/gen.py (seed = workload id). Every row is checked against the size,
padding, causality and order invariants; sampled rows (document starts and ends, the rows
where the candidate count crosses topk, random rows) are checked against the oracle row by
row; key operands / pooled keys are compared in full and query operands on the sampled rows.
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


@pytest.mark.parametrize("wid, w_bf16", [(1, False), (2, False), (3, False), (4, False), (5, False), (3, True)])
def test_workload(wid, w_bf16):
    import torch
    inp = gen.workload(wid)
    if w_bf16:      # the same workload with the per-head weights passed as bf16
        parity.bf16_weights(inp)
    cfg = parity.config_of(inp)
    topk, kp = inp["topk"], inp["kpool"]
    T = inp["q"].shape[0]
    print(f"workload {wid} {inp['name']} T={T}", flush=True)
    gd = parity.gpu_pipeline(inp, cfg, topk, keep_device=True)
    rows = parity.sample_rows(inp, topk, kp)
    o = parity.oracle_operands_rows(inp, cfg, rows)
    # operands
    if cfg["preprocess"]:
        r = torch.as_tensor(np.asarray(rows, np.int64), device="cuda")
        gq = parity.host(gd["q_op"].index_select(0, r))
        assert np.array_equal(gq.view(np.uint8), o["q_op"].view(np.uint8)), "q operands differ"
        if cfg["precision"] != "bf16":
            assert np.array_equal(parity.host(gd["q_scale"].index_select(0, r)), o["q_scale"])
        if kp == 1:
            assert np.array_equal(parity.host(gd["k_op"]).view(np.uint8), o["k_op"].view(np.uint8))
            if cfg["precision"] != "bf16":
                assert np.array_equal(parity.host(gd["k_scale"]), o["k_scale"])
    if kp > 1:
        P = int(o["cu_pools"][-1])
        assert np.array_equal(parity.host(gd["cu_pools"]), o["cu_pools"])
        assert np.array_equal(parity.host(gd["pooled"])[:P].view(np.uint8), o["pooled"].view(np.uint8))
    # sampled rows against the oracle
    g = parity.fetch_rows(gd, rows, T, inp["max_seqlen"], kp)
    ores = orc.index_topk(o["q_deq"], o["k_deq"], inp["w"].astype(np.float64), inp["cu_seqlens"], topk, 1.0, kp,
                          o.get("cu_pools"), True, rows=rows)
    parity.compare_rows(g, ores, inp, cfg, topk, rows)
    # invariants on every row
    full = {n: parity.host(gd[n]) for n in ("scores", "indices", "lengths")}
    parity.check_invariants(full, inp, cfg, topk)
