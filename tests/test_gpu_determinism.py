"""Bit-exact replays and graph capture (GPU), for the indexer step and the two kernels after the
selection (softmax over the selection, sparse attention).

Three runs of the same inputs, the second with a concurrent contention stream, must give
byte-identical operands and outputs (Megatron-LM PR 8403, codex review finding 3: replays
must be byte-identical, with contention). cu_seqlens is read on the device on every call,
so a captured graph replayed with different document boundaries of the same shape must
match eager runs on those boundaries (PR 5992, review: boundaries may change between
capture and replay while shapes and maxima stay fixed).
"""

import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


CASES = {
    "fp8_ln_rope": dict(precision="fp8", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True),
    "mxfp8": dict(precision="mxfp8", preprocess=True, layernorm=False, rope_dim=0),
    "bf16_kpool": dict(precision="bf16", preprocess=False, kpool=4, kpool_tail=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_replays_bit_exact(name):
    import torch
    cfg = CASES[name]
    inp = gen.small(3, [700, 300, 1024], 64, 128, layernorm=cfg.get("layernorm", False),
                    rope_dim=cfg.get("rope_dim", 0), kpool=cfg.get("kpool", 1))
    inp["H"], inp["D"] = 64, 128
    d = parity.gpu_inputs(inp)
    keys = ("q_op", "q_scale", "k_op", "k_scale", "pooled", "pooled_scale", "cu_pools", "indices", "scores",
            "lengths", "pool_indices")
    runs = []
    for rep in range(3):
        if rep == 1:       # contention: a matmul stream running alongside
            side = torch.cuda.Stream()
            a = torch.randn(4096, 4096, device="cuda")
            with torch.cuda.stream(side):
                for _ in range(4):
                    a = a @ a
                    a = a / a.abs().max()
        g = parity.gpu_pipeline(inp, cfg, 64, d=d)
        runs.append({k: g[k] for k in keys if g.get(k) is not None})
        torch.cuda.synchronize()
    for k in runs[0]:
        for r in runs[1:]:
            assert np.array_equal(runs[0][k].view(np.uint8), r[k].view(np.uint8)), k


def test_graph_replay_with_new_boundaries():
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    H, D, topk, T, max_seqlen = 64, 128, 32, 1200, 700
    layouts = [[700, 300, 200], [100, 400, 700], [600, 600, 0], [1, 499, 700]]
    inp = gen.small(4, layouts[0], H, D, layernorm=True, rope_dim=64)
    inp["H"], inp["D"], inp["max_seqlen"] = H, D, max_seqlen
    cos, sin = gen.rope_table(max_seqlen, 64)
    d = parity.gpu_inputs(inp)
    d["cos"], d["sin"] = parity.dev(cos), parity.dev(sin)
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    prec = "fp8"
    bufs = {
        "q_op": torch.empty((T, H, D), dtype=torch.uint8, device="cuda"),
        "q_scale": torch.empty((T, H), dtype=torch.uint8, device="cuda"),
        "k_op": torch.empty((T, D), dtype=torch.uint8, device="cuda"),
        "k_scale": torch.empty((T,), dtype=torch.uint8, device="cuda"),
    }
    outs = {
        "indices": torch.empty((T, topk), dtype=torch.int32, device="cuda"),
        "scores": torch.empty((T, topk), dtype=torch.float32, device="cuda"),
        "lengths": torch.empty((T,), dtype=torch.int32, device="cuda"),
    }
    ws = torch.empty(dsa.workspace_size(T, max_seqlen, topk, 1, H, D, 3, prec), dtype=torch.uint8, device="cuda")

    def step():
        dsa.preprocess(d["q"], d["k"], cu, ln_gamma=d["gamma"], ln_beta=d["beta"], ln_eps=gen.LN_EPS,
                       rope_cos=d["cos"], rope_sin=d["sin"], rope_dim=64, rope_fp32=True, precision=prec, out=bufs)
        dsa.score_topk(bufs["q_op"], bufs["k_op"], d["w"], cu, max_seqlen, topk, q_scale=bufs["q_scale"],
                       k_scale=bufs["k_scale"], precision=prec, workspace=ws, out=outs)

    def eager(layout):
        cu.copy_(torch.tensor(gen.cu_from_lengths(layout), device="cuda"))
        step()
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in outs.items()}

    want = [eager(l) for l in layouts]
    cu.copy_(torch.tensor(gen.cu_from_lengths(layouts[0]), device="cuda"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(2):
        for i, l in enumerate(layouts):
            cu.copy_(torch.tensor(gen.cu_from_lengths(l), device="cuda"))
            graph.replay()
            torch.cuda.synchronize()
            for k in outs:
                assert torch.equal(outs[k], want[i][k]), (rep, i, k)
            _ = torch.randn(1000, device="cuda").sum().item()    # eager work between replays


def _after_selection_inputs(seed):
    """A small selection (two documents, fp8 indexer with LN + RoPE, top-64), its softmax
    input, and attention operands drawn beside it (64 heads, 576-wide latent entries)."""
    import torch
    inp = gen.small(seed, [300, 212], 64, 128, layernorm=True, rope_dim=64)
    inp["H"], inp["D"] = 64, 128
    cfg = dict(precision="fp8", preprocess=True, layernorm=True, rope_dim=64, rope_fp32=True)
    g = parity.gpu_pipeline(inp, cfg, 64, keep_device=True)
    T = g["indices"].shape[0]
    gen_t = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((T, 64, 576), generator=gen_t, device="cuda").to(torch.bfloat16)
    kv = torch.randn((T, 576), generator=gen_t, device="cuda").to(torch.bfloat16)
    return g, q, kv


def test_softmax_and_attention_bit_exact():
    # the two kernels after the selection: three runs, the second beside a contention stream,
    # byte-identical (fixed reduction orders, no floating-point atomics)
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    g, q, kv = _after_selection_inputs(11)
    runs = []
    for rep in range(3):
        if rep == 1:
            side = torch.cuda.Stream()
            a = torch.randn(4096, 4096, device="cuda")
            with torch.cuda.stream(side):
                for _ in range(4):
                    a = a @ a
                    a = a / a.abs().max()
        p = dsa.selection_softmax(g["scores"])
        out, lse = dsa.sparse_attention(q, kv, g["indices"], sm_scale=576 ** -0.5, lengths=g["lengths"])
        torch.cuda.synchronize()
        runs.append((p.clone(), out.clone(), lse.clone()))
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_softmax_and_attention_graph_replays():
    # captured once, replayed with eager work and synchronisation between replays; every
    # replay equals the eager result
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    g, q, kv = _after_selection_inputs(12)
    T = q.shape[0]
    p_out = torch.empty_like(g["scores"])
    o_out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device="cuda")
    l_out = torch.empty((T, 64), dtype=torch.float32, device="cuda")

    def step():
        dsa.selection_softmax(g["scores"], out=p_out)
        dsa.sparse_attention(q, kv, g["indices"], sm_scale=576 ** -0.5, lengths=g["lengths"], out=o_out, lse=l_out)

    step()
    torch.cuda.synchronize()
    want = (p_out.clone(), o_out.clone(), l_out.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (p_out, l_out):
            t.fill_(float("nan"))
        o_out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip((p_out, o_out, l_out), want):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), rep
        _ = torch.randn(1000, device="cuda").sum().item()    # eager work between replays
