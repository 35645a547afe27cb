"""dsa_index_score_topk_noalloc against dsa_index_score_topk (GPU).

The entry point that allocates nothing keeps its score rows in the library's fixed device
scratch instead of a caller workspace; everything else is the same kernels. Its outputs must
be byte-identical to dsa_index_score_topk's on the same inputs, over two calls in a row (the
second on a smaller problem, so the scratch holds the first call's rows when it starts), and
the second call is also checked against the oracle. A problem whose score rows exceed the
scratch is rejected before anything runs.
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


def _operands(inp, cfg, d):
    import sparse_attention_indexer_dsa_amd as dsa
    prec, kp = cfg["precision"], cfg.get("kpool", 1)
    if cfg.get("preprocess"):
        ops = dsa.preprocess(d["q"], d["k"], d["cu"], ln_gamma=d.get("gamma") if cfg.get("layernorm") else None,
                             ln_beta=d.get("beta") if cfg.get("layernorm") else None, ln_eps=gen.LN_EPS,
                             rope_cos=d.get("cos"), rope_sin=d.get("sin"), rope_dim=cfg.get("rope_dim", 0),
                             rope_fp32=cfg.get("rope_fp32", False), precision=prec, return_fp32=kp > 1)
        q_op, q_sc, k_op, k_sc = ops["q_op"], ops.get("q_scale"), ops["k_op"], ops.get("k_scale")
        k_src = ops.get("k_f32")
    else:
        q_op, q_sc, k_op, k_sc = d["q"], None, d["k"], None
        k_src = d["k"]
    cu_pools = None
    if kp > 1:     # pooled from the keys' fp32 carrier (or the raw bf16 keys)
        k_op, k_sc, cu_pools = dsa.kpool(k_src, d["cu"], d["gate"], d["bias"], kp, precision=prec)
    return q_op, q_sc, k_op, k_sc, cu_pools


def _both(inp, cfg, topk):
    """(workspace path outputs, no-alloc outputs) as host arrays."""
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    prec, kp = cfg["precision"], cfg.get("kpool", 1)
    d = parity.gpu_inputs(inp)
    q_op, q_sc, k_op, k_sc, cu_pools = _operands(inp, cfg, d)
    kw = dict(q_scale=q_sc, k_scale=k_sc, precision=prec, kpool=kp, cu_pools=cu_pools, kpool_tail=True)
    ref = dsa.score_topk(q_op, k_op, d["w"], d["cu"], inp["max_seqlen"], topk, **kw)
    T = inp["q"].shape[0]
    out = dsa._alloc_outputs(None, T, topk, kp, "cuda")
    for t in out.values():
        t.fill_(-7)
    torch.cuda.synchronize()
    print(f"noalloc call T={T} max_seqlen={inp['max_seqlen']} topk={topk} {prec} kpool={kp}", flush=True)
    dsa.score_topk_noalloc(q_op, k_op, d["w"], d["cu"], inp["max_seqlen"], topk, out=out, **kw)
    torch.cuda.synchronize()
    names = ["indices", "scores", "lengths"] + (["pool_indices"] if kp > 1 else [])
    return {n: parity.host(ref[n]) for n in names}, {n: parity.host(out[n]) for n in names}


def _same(a, b):
    for n in a:
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n


def test_noalloc_matches_workspace_path_two_calls():
    # first call: the 2 x 4096, H=64, fp8 workload (score rows 8192 x 4096 floats fill the
    # scratch); second call: a small problem, whose rows are then checked against the oracle
    big = gen.workload(3)
    ref, got = _both(big, parity.config_of(big), big["topk"])
    _same(ref, got)
    cfg = dict(precision="fp8", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True)
    small = gen.small(17, [37, 100, 5, 0, 130], 64, 128, layernorm=True, rope_dim=64)
    small["H"], small["D"] = 64, 128
    ref2, got2 = _both(small, cfg, 16)
    _same(ref2, got2)
    o = parity.oracle_operands(small, cfg)
    ores = orc.index_topk(o["q_deq"], o["k_deq"], small["w"].astype(np.float64), small["cu_seqlens"], 16)
    T = small["q"].shape[0]
    # the no-alloc call exposes no workspace: its selected scores stand for the rows
    g = dict(got2)
    g["ws"] = {t: _ws_from_selection(got2, ores, t) for t in range(T)}
    parity.compare_rows(g, ores, small, cfg, 16, range(T))
    parity.check_invariants(got2, small, cfg, 16)


def _ws_from_selection(g, ores, t):
    """A stand-in workspace row for compare_rows: the oracle's scores, with the GPU's selected
    scores at the candidates the GPU selected (those are what the no-alloc call outputs)."""
    I = ores[t]["I"].astype(np.float32)
    n = int(g["lengths"][t])
    cu0 = int(ores[t]["indices"][0] - ores[t]["sel"][0]) if ores[t]["sel"].size else 0
    ws = I.copy()
    if n:
        ws[g["indices"][t][:n].astype(np.int64) - cu0] = g["scores"][t][:n]
    return ws


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_noalloc_kpool_and_bf16(precision):
    cfg = dict(precision=precision, preprocess=precision != "bf16", layernorm=False, rope_dim=0, kpool=4,
               kpool_tail=True)
    inp = gen.small(23, [300, 2, 0, 517], 32, 128, kpool=4)
    inp["H"], inp["D"] = 32, 128
    ref, got = _both(inp, cfg, 20)
    _same(ref, got)
    raw = dict(precision="bf16", preprocess=False)
    inp2 = gen.small(24, [90, 7], 16, 64)
    inp2["H"], inp2["D"] = 16, 64
    ref2, got2 = _both(inp2, raw, 8)
    _same(ref2, got2)


def test_noalloc_rejects_problem_beyond_scratch():
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    T, H, D, L = 8192, 64, 128, 8192          # 8192 rows x 8192 floats > 128 MiB + 4 KiB
    need = dsa.workspace_size(T, L, 64, 1, H, D, 1, "bf16")
    assert need > dsa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    out = dsa._alloc_outputs(None, T, 64, 1, "cuda")
    with pytest.raises(ValueError, match="scratch"):
        dsa.score_topk_noalloc(q, k, w, cu, L, 64, out=out)
