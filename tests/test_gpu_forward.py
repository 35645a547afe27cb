"""The one-call hot path (dsa_index_forward) against the oracle and the two-call path (GPU).

dsa_index_forward builds the query operands inside the scoring kernel. Its query operands
(returned on request) must be byte-identical to the oracle's, and its outputs identical to
dsa_index_preprocess + dsa_index_score_topk on the same inputs, which the parity tests tie to
the oracle; the selections are also checked against the oracle directly.
"""

import numpy as np
import pytest

from oracle import oracle as orc
import gen
import parity

pytestmark = pytest.mark.gpu

DOCS = [37, 100, 5, 0, 130]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def _forward(inp, cfg, topk, d=None):
    import sparse_attention_indexer_dsa_amd as dsa
    d = parity.gpu_inputs(inp) if d is None else d
    res = dsa.forward(d["q"], d["k"], d["w"], d["cu"], inp["max_seqlen"], topk,
                      ln_gamma=d.get("gamma") if cfg.get("layernorm") else None,
                      ln_beta=d.get("beta") if cfg.get("layernorm") else None, ln_eps=gen.LN_EPS,
                      rope_cos=d.get("cos"), rope_sin=d.get("sin"), rope_dim=cfg.get("rope_dim", 0),
                      rope_interleaved=cfg.get("interleaved", False), rope_fp32=cfg.get("rope_fp32", False),
                      precision=cfg["precision"], return_operands=True)
    out = {k: parity.host(v) for k, v in res.items() if k != "workspace"}
    out["ws"] = parity.workspace_scores(parity.host(res["workspace"]), inp["q"].shape[0], inp["max_seqlen"], 1)
    return out


def _check(inp, cfg, topk):
    f = _forward(inp, cfg, topk)
    two = parity.gpu_pipeline(inp, cfg, topk)
    o = parity.oracle_operands(inp, cfg)
    assert np.array_equal(f["q_op"].view(np.uint8), np.asarray(o["q_op"]).view(np.uint8)), "q operands differ"
    if cfg["precision"] != "bf16":
        assert np.array_equal(f["q_scale"], o["q_scale"]), "q scales differ"
    for k in ("indices", "scores", "lengths"):
        assert np.array_equal(f[k].view(np.uint8), two[k].view(np.uint8)), k
    T = inp["q"].shape[0]
    ores = orc.index_topk(o["q_deq"], o["k_deq"], inp["w"].astype(np.float64), inp["cu_seqlens"], topk)
    parity.compare_rows(f, ores, inp, cfg, topk, range(T))


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("HD", [(64, 128), (32, 64), (16, 128)])
@pytest.mark.parametrize("rope", ["half64_fp32", "half64_bf16", "interleaved", "none"])
def test_forward_matches(precision, HD, rope):
    H, D = HD
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=0 if rope == "none" else 64,
               rope_fp32=rope != "half64_bf16", interleaved=rope == "interleaved")
    inp = gen.small(200 + H + D + len(rope), DOCS, H, D, layernorm=True, rope_dim=cfg["rope_dim"])
    inp["H"], inp["D"] = H, D
    _check(inp, cfg, 16)


@pytest.mark.parametrize("R", [32, 96, 128])
def test_forward_bf16_rope_dims(R):
    # bf16 operands keep every rotate-half pair in one lane for rope_dim % 32 == 0
    cfg = dict(precision="bf16", preprocess=True, layernorm=False, rope_dim=R, rope_fp32=False)
    inp = gen.small(300 + R, DOCS, 64, 128, rope_dim=R)
    inp["H"], inp["D"] = 64, 128
    _check(inp, cfg, 16)


@pytest.mark.parametrize("precision", ["fp8", "mxfp8"])
def test_forward_fp8_rope128(precision):
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=128, rope_fp32=True)
    inp = gen.small(310, DOCS, 64, 128, layernorm=True, rope_dim=128)
    inp["H"], inp["D"] = 64, 128
    _check(inp, cfg, 16)


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
def test_forward_fp32_inputs(precision):
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=64, rope_fp32=False)
    inp = gen.small(320, [40, 0, 77], 64, 128, layernorm=True, rope_dim=64)
    inp["H"], inp["D"] = 64, 128
    rng = np.random.default_rng(9)
    inp["q"] = (rng.standard_normal(inp["q"].shape) * 3.0).astype(np.float32)
    inp["k"] = (rng.standard_normal(inp["k"].shape) * 0.5 + 0.25).astype(np.float32)
    _check(inp, cfg, 16)


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("H", [16, 32, 64])
def test_forward_bf16_weights(precision, H):
    # bf16 per-head weights through the fused path (query preprocessing in the scoring kernel)
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True)
    inp = gen.small(330 + H, DOCS, H, 128, layernorm=True, rope_dim=64)
    inp["H"], inp["D"] = H, 128
    parity.bf16_weights(inp)
    _check(inp, cfg, 16)


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("w_bf16", [False, True])
def test_score_fused_direct(precision, w_bf16):
    # dsa_index_score_fused on its own: the score rows it writes are those of
    # dsa_index_preprocess + dsa_index_score (byte for byte) and within tolerance of the oracle,
    # and the query operands it returns are the oracle's
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    H, D = 64, 128
    cfg = dict(precision=precision, preprocess=True, layernorm=True, rope_dim=64, rope_fp32=False)
    inp = gen.small(340 + w_bf16, DOCS, H, D, layernorm=True, rope_dim=64)
    inp["H"], inp["D"] = H, D
    if w_bf16:
        parity.bf16_weights(inp)
    d = parity.gpu_inputs(inp)
    T, ms = inp["q"].shape[0], inp["max_seqlen"]
    ops = dsa.preprocess(d["q"], d["k"], d["cu"], ln_gamma=d["gamma"], ln_beta=d["beta"], ln_eps=gen.LN_EPS,
                         rope_cos=d["cos"], rope_sin=d["sin"], rope_dim=64, rope_fp32=False, precision=precision)
    n = dsa.workspace_size(T, ms, 1, 1, H, D, len(inp["docs"]), precision)
    ws_two = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ws_one = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dsa.score(ops["q_op"], ops["k_op"], d["w"], d["cu"], ms, ws_two, q_scale=ops.get("q_scale"),
              k_scale=ops.get("k_scale"), precision=precision)
    got_ops = {"q_op": torch.empty_like(ops["q_op"])}
    if precision != "bf16":
        got_ops["q_scale"] = torch.empty_like(ops["q_scale"])
    dsa.score_fused(d["q"], ops["k_op"], d["w"], d["cu"], ms, ws_one, k_scale=ops.get("k_scale"),
                    rope_cos=d["cos"], rope_sin=d["sin"], rope_dim=64, rope_fp32=False, precision=precision,
                    out_operands=got_ops)
    torch.cuda.synchronize()
    assert torch.equal(ws_one, ws_two), "fused score rows differ from the two-call path"
    o = parity.oracle_operands(inp, cfg)
    assert np.array_equal(parity.host(got_ops["q_op"]).view(np.uint8), np.asarray(o["q_op"]).view(np.uint8))
    if precision != "bf16":
        assert np.array_equal(parity.host(got_ops["q_scale"]), o["q_scale"])
    ws = parity.workspace_scores(parity.host(ws_one), T, ms, 1)
    ores = orc.score_rows(o["q_deq"], o["k_deq"], inp["w"].astype(np.float64), inp["cu_seqlens"])
    tau = parity.TAU[precision]
    for t, (I, M) in ores.items():
        g = ws[t, :I.size].astype(np.float64)
        assert np.all(np.abs(g - I) <= tau * M + 1e-30), t      # false for a NaN


def test_forward_full_workload():
    # the 2 x 4096, H=64, D=128, fp8 workload: one call against the two-call path, all rows
    inp = gen.workload(3)
    cfg = parity.config_of(inp)
    f = _forward(inp, cfg, inp["topk"])
    two = parity.gpu_pipeline(inp, cfg, inp["topk"])
    for k in ("indices", "scores", "lengths"):
        assert np.array_equal(f[k].view(np.uint8), two[k].view(np.uint8)), k
    assert np.array_equal(f["q_op"].view(np.uint8), two["q_op"].view(np.uint8))
    assert np.array_equal(f["q_scale"], two["q_scale"])
