"""HIP library vs CPU oracle on seeded small problems (GPU).

Sizes span several query and key tiles and ragged tails: documents of 37, 100, 5, 0 and
130 tokens (the workgroup tiles are 4-16 query tokens and 64 keys). Operands, scales and
pooled keys must be byte-identical; scores and selections follow the rules in parity.py.
"""

import json
import os

import numpy as np
import pytest

from oracle import oracle as orc
import gen
import parity

pytestmark = pytest.mark.gpu

DOCS = [37, 100, 5, 0, 130]
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_attention_indexer_dsa_amd as dsa
    dsa.load()


def _problem(seed, H, D, cfg, docs=DOCS):
    inp = gen.small(seed, docs, H, D, layernorm=cfg.get("layernorm", False), rope_dim=cfg.get("rope_dim", 0),
                    kpool=cfg.get("kpool", 1))
    inp["H"], inp["D"] = H, D
    return inp


def _run_and_compare(seed, H, D, cfg, topk, docs=DOCS, sm_scale=1.0, w_bf16=False):
    inp = _problem(seed, H, D, cfg, docs)
    if w_bf16:
        parity.bf16_weights(inp)
    g = parity.gpu_pipeline(inp, cfg, topk, sm_scale=sm_scale)
    o = parity.oracle_operands(inp, cfg)
    kp = cfg.get("kpool", 1)
    # operands byte for byte
    if cfg.get("preprocess"):
        assert np.array_equal(g["q_op"].view(np.uint8), o["q_op"].view(np.uint8)), "q operands differ"
        if cfg["precision"] != "bf16":
            assert np.array_equal(g["q_scale"], o["q_scale"]), "q scales differ"
        if kp == 1:
            assert np.array_equal(g["k_op"].view(np.uint8), o["k_op"].view(np.uint8)), "k operands differ"
            if cfg["precision"] != "bf16":
                assert np.array_equal(g["k_scale"], o["k_scale"]), "k scales differ"
    if kp > 1:
        P = int(o["cu_pools"][-1])
        assert np.array_equal(g["cu_pools"], o["cu_pools"])
        assert np.array_equal(g["pooled"][:P].view(np.uint8), o["pooled"].view(np.uint8)), "pooled keys differ"
        if cfg["precision"] != "bf16":
            assert np.array_equal(g["pooled_scale"][:P], o["pooled_scale"])
    ores = orc.index_topk(o["q_deq"], o["k_deq"], inp["w"].astype(np.float64), inp["cu_seqlens"], topk,
                          sm_scale, kp, o.get("cu_pools"), cfg.get("kpool_tail", True))
    parity.compare_rows(g, ores, inp, cfg, topk, range(inp["q"].shape[0]), sm_scale)
    parity.check_invariants(g, inp, cfg, topk)
    return g, ores


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("topk", [1, 8, 64])
def test_bf16_raw_operands(H, D, topk):
    cfg = dict(precision="bf16", preprocess=False)
    _run_and_compare(100 + H + D + topk, H, D, cfg, topk)


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("rope_fp32", [False, True])
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("HD", [(64, 128), (32, 64), (16, 128)])
def test_preprocess_and_score(precision, rope_fp32, interleaved, HD):
    H, D = HD
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=64 if D == 128 else 32,
               rope_fp32=rope_fp32, interleaved=interleaved)
    _run_and_compare(7 + H + D + rope_fp32 + 2 * interleaved, H, D, cfg, 16)


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("rope_fp32", [False, True])
@pytest.mark.parametrize("interleaved", [False, True])
def test_preprocess_fp32_inputs(precision, rope_fp32, interleaved):
    # fp32 inputs that bf16 cannot hold: the bf16 carrier rounding (rope_fp32 off) is visible
    H, D = 64, 128
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=64, rope_fp32=rope_fp32,
               interleaved=interleaved)
    inp = gen.small(61 + rope_fp32 + 2 * interleaved, [40, 0, 77], H, D, layernorm=True, rope_dim=64)
    rng = np.random.default_rng(5)
    inp["q"] = (rng.standard_normal(inp["q"].shape) * 3.0).astype(np.float32)
    inp["k"] = (rng.standard_normal(inp["k"].shape) * 0.5 + 0.25).astype(np.float32)
    g = parity.gpu_pipeline(inp, cfg, 16)
    o = parity.oracle_operands(inp, cfg)
    assert np.array_equal(g["q_op"].view(np.uint8), np.asarray(o["q_op"]).view(np.uint8))
    assert np.array_equal(g["k_op"].view(np.uint8), np.asarray(o["k_op"]).view(np.uint8))
    if precision != "bf16":
        assert np.array_equal(g["q_scale"], o["q_scale"]) and np.array_equal(g["k_scale"], o["k_scale"])


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
def test_quantize_only(precision):
    # no LayerNorm, no RoPE: bf16 inputs quantised for scoring
    cfg = dict(precision=precision, preprocess=True, layernorm=False, rope_dim=0)
    _run_and_compare(31, 64, 128, cfg, 32)


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_weights(precision, H, D):
    # per-head weights passed as bf16 (PR 8403, codex review finding 3: the weights stay BF16),
    # widened exactly by the scoring kernel
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=64 if D == 128 else 32,
               rope_fp32=True)
    _run_and_compare(400 + H + D, H, D, cfg, 16, w_bf16=True)


@pytest.mark.parametrize("H", [16, 64])
def test_bf16_weights_raw_bf16_and_kpool(H):
    _run_and_compare(430 + H, H, 128, dict(precision="bf16", preprocess=False), 8, w_bf16=True)
    _run_and_compare(440 + H, H, 128, dict(precision="bf16", preprocess=False, kpool=4, kpool_tail=True), 5,
                     docs=[37, 100, 5, 0, 130, 2, 3], w_bf16=True)


@pytest.mark.parametrize("kp", [2, 3, 4])
@pytest.mark.parametrize("tail", [True, False])
@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
def test_kpool(kp, tail, precision):
    cfg = dict(precision=precision, preprocess=precision != "bf16", layernorm=False, rope_dim=0, kpool=kp,
               kpool_tail=tail)
    _run_and_compare(50 + kp + 2 * tail, 64, 128, cfg, 6, docs=[37, 100, 5, 0, 130, 2, 3])


@pytest.mark.parametrize("ndocs", [63, 64, 70])
@pytest.mark.parametrize("kp", [2, 4, 5])
@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_kpool_many_documents(ndocs, kp, precision):
    # Pooling takes one launch when the documents fit a wave's lanes (fewer than 64) and
    # kpool is 2, 3 or 4, and a pool-offset launch plus a generic kernel otherwise: both
    # sides of each bound, with empty, one-token and incomplete-pool documents.
    rng = np.random.default_rng(600 + ndocs + kp)
    docs = [int(x) for x in rng.integers(0, 24, ndocs)]
    docs[3], docs[10], docs[-1] = 0, 1, kp - 1
    cfg = dict(precision=precision, preprocess=precision != "bf16", layernorm=False, rope_dim=0, kpool=kp,
               kpool_tail=True)
    _run_and_compare(60 + ndocs + kp, 16, 64, cfg, 4, docs=docs)


def test_kpool_after_preprocess():
    cfg = dict(precision="bf16", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True, kpool=4,
               kpool_tail=True)
    _run_and_compare(77, 32, 128, cfg, 5)


def test_sm_scale_and_topk_above_candidates():
    cfg = dict(precision="bf16", preprocess=False)
    _run_and_compare(5, 64, 128, cfg, 300, sm_scale=0.125)


def test_single_token_documents_and_empty_docs():
    cfg = dict(precision="fp8", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=False)
    _run_and_compare(9, 64, 128, cfg, 4, docs=[1, 0, 1, 1, 0, 2, 65])


def test_ties_go_to_lowest_index():
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    T, H, D = 70, 16, 64
    rng = np.random.default_rng(0)
    k1 = np.abs(rng.standard_normal(D)).astype(np.float32)
    k = np.tile(gen.to_bf16_bits(k1), (T, 1))
    q = gen.to_bf16_bits(np.abs(rng.standard_normal((T, H, D))).astype(np.float32))
    w = np.ones((T, H), np.float32)
    cu = np.array([0, T], np.int32)
    res = dsa.score_topk(parity.dev_bf16(q), parity.dev_bf16(k), parity.dev(w), parity.dev(cu), T, 5)
    idx = parity.host(res["indices"])
    for t in range(T):
        n = min(5, t + 1)
        assert list(idx[t, :n]) == list(range(n)) and np.all(idx[t, n:] == -1)


def test_all_negative_weights_zero_ties():
    # w < 0 makes every score <= 0; candidates whose logits are all negative score 0 and
    # tie; the selection must still be exact (zeros tie by index, -0 counts as +0)
    cfg = dict(precision="bf16", preprocess=False)
    inp = _problem(11, 64, 128, cfg)
    inp["w"] = -np.abs(inp["w"])
    g = parity.gpu_pipeline(inp, cfg, 16)
    o = parity.oracle_operands(inp, cfg)
    ores = orc.index_topk(o["q_deq"], o["k_deq"], inp["w"].astype(np.float64), inp["cu_seqlens"], 16)
    parity.compare_rows(g, ores, inp, cfg, 16, range(inp["q"].shape[0]))


def test_golden_bf16_boundary_worked_example():
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    gd = json.load(open(os.path.join(GOLD, "bf16_boundary_worked_example.json")))
    H, D = 16, 64                          # one live head and dimension, the rest zero
    q = np.zeros((1, H, D), np.float32); q[0, 0, 0] = gd["q"]
    k = np.zeros((1, D), np.float32); k[0, 0] = gd["k"]
    w = np.zeros((1, H), np.float32); w[0, 0] = gd["w"]
    cu = parity.dev(np.array([0, 1], np.int32))
    ops = dsa.preprocess(parity.dev(q), parity.dev(k), cu, rope_fp32=True, precision="bf16", return_fp32=True)
    assert parity.host(ops["q_f32"])[0, 0, 0] == np.float32(gd["q"])
    res = dsa.score_topk(ops["q_op"], ops["k_op"], parity.dev(w), cu, 1, 1, sm_scale=gd["sm_scale"])
    assert parity.host(res["scores"])[0, 0] == gd["expected_bf16_score"]
    assert parity.host(res["indices"])[0, 0] == 0 and parity.host(res["lengths"])[0] == 1


def test_golden_repeated_ends():
    import sparse_attention_indexer_dsa_amd as dsa
    gd = json.load(open(os.path.join(GOLD, "repeated_ends_topk.json")))
    H, D = 16, 64
    k = np.zeros((4, D), np.float32)
    k[:, 0] = np.array(gd["keys"] * 2)[:, 0]
    q = np.zeros((4, H, D), np.float32)
    w = np.zeros((4, H), np.float32)
    for r, t in enumerate((1, 3)):
        q[t, 0, 0] = gd["queries"][r][0][0]
        w[t, 0] = gd["weights"][r][0]
    cu = parity.dev(np.array([0, 2, 4], np.int32))
    res = dsa.score_topk(parity.dev_bf16(gen.to_bf16_bits(q)), parity.dev_bf16(gen.to_bf16_bits(k)),
                         parity.dev(w), cu, 2, gd["topk"])
    idx, sc, ln = (parity.host(res[n]) for n in ("indices", "scores", "lengths"))
    starts = {1: 0, 3: 2}
    assert [list(idx[t] - starts[t]) for t in (1, 3)] == gd["expected_indices"]
    assert [int(ln[t]) for t in (1, 3)] == gd["expected_lengths"]
    assert [list(sc[t].astype(float)) for t in (1, 3)] == gd["expected_scores"]
