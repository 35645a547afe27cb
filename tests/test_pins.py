"""Pins of the oracle against the pages' worked values, closed forms and invariants (CPU)."""

import json
import os

import numpy as np
import pytest

from oracle import formats as fm
from oracle import oracle as orc
import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------ values printed on the pages

def test_bf16_boundary_worked_example():
    g = json.load(open(os.path.join(GOLD, "bf16_boundary_worked_example.json")))
    q_car, k_car = orc.preprocess(np.full((1, 1, 1), g["q"], np.float32),
                                  np.full((1, 1), g["k"], np.float32), [0, 1], rope_fp32=True)
    assert q_car[0, 0, 0] == np.float32(g["q"])          # the fp32 carrier is kept
    qo, _ = orc.quantize(q_car, "bf16")
    ko, _ = orc.quantize(k_car, "bf16")
    w = np.array([[g["w"]]])
    res = orc.index_topk(orc.dequantize(qo, None, "bf16"), orc.dequantize(ko, None, "bf16"), w,
                         [0, 1], topk=1, sm_scale=g["sm_scale"])
    assert res[0]["scores"][0] == g["expected_bf16_score"]
    res32 = orc.index_topk(q_car.astype(np.float64), k_car.astype(np.float64), w, [0, 1], topk=1)
    assert abs(res32[0]["scores"][0] - g["expected_fp32_score_approx"]) < 1e-6


def test_repeated_ends_outputs():
    g = json.load(open(os.path.join(GOLD, "repeated_ends_topk.json")))
    # two documents of two tokens: the last row of each sees exactly the two keys of its document
    keys = np.array(g["keys"] * 2)
    q = np.zeros((4, 1, 1))
    w = np.zeros((4, 1))
    for r, t in enumerate((1, 3)):
        q[t] = g["queries"][r]
        w[t] = g["weights"][r]
    res = orc.index_topk(q, keys, w, [0, 2, 4], topk=g["topk"])
    assert [list(res[t]["sel"]) for t in (1, 3)] == g["expected_indices"]
    assert [res[t]["length"] for t in (1, 3)] == g["expected_lengths"]
    assert [list(res[t]["scores"]) for t in (1, 3)] == g["expected_scores"]
    # global indices of the second document are offset by its start
    assert list(res[3]["indices"]) == [2 + i for i in g["expected_indices"][1]]


# ------------------------------------------------ LayerNorm

def test_layernorm_constant_vector_gives_beta():
    rng = np.random.default_rng(0)
    beta = rng.standard_normal(128).astype(np.float32)
    gamma = rng.standard_normal(128).astype(np.float32)
    x = np.full((3, 128), 1.7, np.float32)
    y = orc.key_layernorm(x, gamma, beta, 1e-6)
    assert np.array_equal(y, np.broadcast_to(beta, y.shape))


def test_tree_sum_order_is_pinned():
    # Pairwise halving: (1 + -1) + (2^-24 + 2^-24) = 2^-23; a left-to-right sum gives
    # (1 + 2^-24) -> 1 (tie to even), then 0, then 2^-24.
    x = np.array([1.0, 2.0 ** -24, -1.0, 2.0 ** -24], np.float32)
    assert orc.tree_sum32(x) == np.float32(2.0 ** -23)
    x8 = np.array([1, 0, 0, 0, -1, 0, 0, 0], np.float32)
    x8[1] = x8[5] = 2.0 ** -24
    assert orc.tree_sum32(x8) == np.float32(2.0 ** -23)


@pytest.mark.parametrize("scale", [1.0, 1e-3, 30.0])
def test_layernorm_matches_float64_library_form(scale):
    rng = np.random.default_rng(1)
    D = 128
    x = (scale * rng.standard_normal((64, D)) + 0.3).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(D)).astype(np.float32)
    eps = 1e-6
    y = orc.key_layernorm(x, gamma, beta, eps).astype(np.float64)
    x64 = x.astype(np.float64)
    ref = (x64 - x64.mean(-1, keepdims=True)) / np.sqrt(x64.var(-1, keepdims=True) + eps) * gamma + beta
    rstd = 1 / np.sqrt(x64.var(-1, keepdims=True) + eps)
    mag = np.abs((x64 - x64.mean(-1, keepdims=True)) * rstd * gamma) + np.abs(beta)
    # fp32 rounding bound: a few ulps of the output, plus the error of the tree-summed
    # mean (log2(D) levels, each within one ulp of the partial sums) scaled by rstd*gamma
    u = 2.0 ** -24
    mean_err = 2 * np.log2(D) * u * np.abs(x64).mean(-1, keepdims=True)
    tol = 4e-6 * mag.max(-1, keepdims=True) + mean_err * rstd * np.abs(gamma)
    assert np.all(np.abs(y - ref) <= tol)


# ------------------------------------------------ RoPE

def _rope_complex(x, pos, cos, sin, R, interleaved):
    """Rotary embedding as a complex product (x1 + i x2) * (cos + i sin), float64."""
    x = x.astype(np.float64).copy()
    D = x.shape[-1]
    if interleaved:
        z = x[..., D - R::2] + 1j * x[..., D - R + 1::2]
    else:
        z = x[..., D - R:D - R // 2] + 1j * x[..., D - R // 2:]
    z = z * (cos[pos].astype(np.float64) + 1j * sin[pos].astype(np.float64))
    if interleaved:
        x[..., D - R::2], x[..., D - R + 1::2] = z.real, z.imag
    else:
        x[..., D - R:D - R // 2], x[..., D - R // 2:] = z.real, z.imag
    return x


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_is_a_complex_rotation(interleaved):
    rng = np.random.default_rng(2)
    D, R, P = 128, 64, 300
    cos, sin = gen.rope_table(P, R)
    x = rng.standard_normal((P, D)).astype(np.float32)
    pos = np.arange(P)
    y = orc.rope(x, pos, cos, sin, R, interleaved)
    ref = _rope_complex(x, pos, cos, sin, R, interleaved)
    assert np.allclose(y, ref, rtol=0, atol=4e-6 * np.abs(x).max())
    assert np.array_equal(y[:, :D - R], x[:, :D - R])            # NoPE dims untouched


def test_rope_position_zero_and_nope_are_identity():
    rng = np.random.default_rng(3)
    cos, sin = gen.rope_table(8, 64)
    x = rng.standard_normal((5, 128)).astype(np.float32)
    assert np.array_equal(orc.rope(x, np.zeros(5, int), cos, sin, 64), x)
    assert np.array_equal(orc.rope(x, np.arange(5), cos, sin, 0), x)


def test_rope_relative_position_property():
    rng = np.random.default_rng(4)
    cos, sin = gen.rope_table(400, 64)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)
    def dot(u, v):
        return float(orc.rope(q, u, cos, sin, 64).astype(np.float64) @ orc.rope(k, v, cos, sin, 64))
    base = dot(10, 3)
    for shift in (1, 57, 300):
        assert abs(dot(10 + shift, 3 + shift) - base) < 1e-3
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-2         # direction matters


# ------------------------------------------------ bf16 default vs fp32-RoPE (PR 8403)

def test_rope_fp32_invariants():
    d = gen.small(5, [40, 24], 4, 128, layernorm=True, rope_dim=64)
    q = gen.bf16_bits_to_f32(d["q"])
    k = gen.bf16_bits_to_f32(d["k"])
    cu = d["cu_seqlens"]
    args = dict(gamma=d["gamma"], beta=d["beta"], eps=1e-6, cos=d["cos"], sin=d["sin"], rope_dim=64)
    q0, k0 = orc.preprocess(q, k, cu, rope_fp32=False, **args)
    q1, k1 = orc.preprocess(q, k, cu, rope_fp32=True, **args)
    _, pos = orc.geometry(cu, q.shape[0])
    ln = orc.key_layernorm(k, d["gamma"], d["beta"], 1e-6)
    # 1. default k = bf16(RoPE(bf16(LN(k))))
    assert np.array_equal(k0, fm.bf16_round(orc.rope(fm.bf16_round(ln), pos, d["cos"], d["sin"], 64)))
    # 2. fp32 mode, bf16 scoring: bf16(RoPE(LN(k)))
    assert np.array_equal(orc.quantize(k1, "bf16")[0], fm.bf16_bits(orc.rope(ln, pos, d["cos"], d["sin"], 64)))
    # 3. bf16 q inputs: identical q operands in both modes
    assert np.array_equal(orc.quantize(q0, "bf16")[0], orc.quantize(q1, "bf16")[0])
    # 4. NoPE dims of k: same in both modes once rounded for scoring
    assert np.array_equal(orc.quantize(k0, "bf16")[0][:, :64], orc.quantize(k1, "bf16")[0][:, :64])
    # the round-trip is really gone in fp32 mode: carriers differ somewhere
    assert not np.array_equal(k0, k1)


# ------------------------------------------------ KPool

def test_kpool_one_is_token_mode():
    d = gen.small(6, [7, 5], 2, 64, kpool=1)
    k = gen.bf16_bits_to_f32(d["k"])
    gate = fm.bf16_bits(np.random.default_rng(0).standard_normal(12).astype(np.float32))
    pooled, cu_pools = orc.kpool(k, d["cu_seqlens"], gate, np.array([0.3], np.float32), 1)
    assert np.array_equal(pooled, k) and list(cu_pools) == list(d["cu_seqlens"])


def test_kpool_equal_logits_is_exact_mean():
    rng = np.random.default_rng(7)
    k = rng.integers(-8, 9, (12, 64)).astype(np.float32)
    gate = fm.bf16_bits(np.full(12, 0.7, np.float32))
    pooled, cu_pools = orc.kpool(k, [0, 12], gate, np.zeros(4, np.float32), 4)
    assert np.array_equal(pooled, k.reshape(3, 4, 64).mean(1))


def test_kpool_matches_float64_softmax():
    rng = np.random.default_rng(8)
    docs = [9, 3, 0, 13]
    cu = np.concatenate([[0], np.cumsum(docs)])
    T = cu[-1]
    k = rng.standard_normal((T, 128)).astype(np.float32)
    gate = fm.bf16_bits(rng.standard_normal(T).astype(np.float32))
    bias = (0.3 * rng.standard_normal(4)).astype(np.float32)
    pooled, cu_pools = orc.kpool(k, cu, gate, bias, 4)
    assert list(cu_pools) == [0, 2, 2, 2, 5]
    g = fm.bf16_to_f32(gate).astype(np.float64)
    rows = []
    for b in range(len(docs)):
        for p in range(docs[b] // 4):
            s = cu[b] + 4 * p
            z = g[s:s + 4] + bias.astype(np.float64)
            a = np.exp(z - z.max()); a /= a.sum()
            rows.append(a @ k[s:s + 4].astype(np.float64))
    ref = np.array(rows)
    assert np.all(np.abs(pooled - ref) <= 1e-6 * np.abs(k).max())


# ------------------------------------------------ selection invariants

def test_identical_keys_tie_to_lowest_indices():
    rng = np.random.default_rng(9)
    q = np.abs(rng.standard_normal((20, 2, 8)))
    k = np.tile(np.abs(rng.standard_normal(8)), (20, 1))
    w = np.ones((20, 2))
    res = orc.index_topk(q, k, w, [0, 20], topk=5)
    for t in range(20):
        assert list(res[t]["sel"]) == list(range(min(5, t + 1)))


def test_causality_and_lengths():
    d = gen.small(10, [11, 0, 29, 6], 4, 64, kpool=4)
    cu = d["cu_seqlens"]
    T = d["T"]
    k = gen.bf16_bits_to_f32(d["k"])
    pooled, cu_pools = orc.kpool(k, cu, d["gate"], d["bias"], 4)
    q = gen.bf16_bits_to_f32(d["q"]).astype(np.float64)
    doc, pos = orc.geometry(cu, T)
    for kp, kk, cp in ((1, k, None), (4, pooled, cu_pools)):
        for tail in (True, False):
            res = orc.index_topk(q, kk.astype(np.float64), d["w"].astype(np.float64), cu, 3, 1.0, kp, cp, tail)
            for t in range(T):
                r = res[t]
                lo, hi = cu[doc[t]], t
                cand = (pos[t] + 1) // kp
                nsel = min(3, cand)
                if kp == 1:
                    assert r["length"] == nsel
                    assert np.all((r["indices"] >= lo) & (r["indices"] <= hi))
                else:
                    tl = (pos[t] + 1) % 4 if tail else 0
                    assert r["length"] == nsel * 4 + tl
                    toks = r["tokens"]
                    assert np.all((toks >= lo) & (toks <= hi)) and len(set(toks)) == toks.size
                    chosen = set()
                    for p in r["sel"]:
                        chosen |= set(range(lo + 4 * p, lo + 4 * p + 4))
                    assert set(toks[:nsel * 4]) == chosen


def test_fp8_changes_selection():
    # Qualitative check: identical inputs, fp8 vs bf16 operands, some rows select differently.
    d = gen.small(11, [256], 64, 128, layernorm=True, rope_dim=64)
    q = gen.bf16_bits_to_f32(d["q"])
    k = gen.bf16_bits_to_f32(d["k"])
    qc, kc = orc.preprocess(q, k, d["cu_seqlens"], d["gamma"], d["beta"], 1e-6, d["cos"], d["sin"], 64,
                            rope_fp32=True)
    sel = {}
    for p in ("bf16", "fp8"):
        qo, qs = orc.quantize(qc, p)
        ko, ks = orc.quantize(kc, p)
        res = orc.index_topk(orc.dequantize(qo, qs, p), orc.dequantize(ko, ks, p), d["w"], d["cu_seqlens"], 32)
        sel[p] = [frozenset(res[t]["sel"]) for t in range(256)]
    diff = sum(a != b for a, b in zip(sel["bf16"], sel["fp8"]))
    assert 0 < diff < 256


# ---------------------------------------------------------------- selection softmax

def test_selection_softmax_worked_values():
    # scores 0, ln 2, ln 3: the exponentials are 1, 2, 3, so the softmax is 1/6, 2/6, 3/6
    p = orc.selection_softmax([np.log(3.0), np.log(2.0), 0.0, -np.inf])
    np.testing.assert_allclose(p, [0.5, 1 / 3, 1 / 6, 0.0], rtol=1e-14, atol=0)
    assert p[3] == 0.0


def test_selection_softmax_equal_scores_are_uniform():
    for n in (1, 2, 4, 64, 2048):
        p = orc.selection_softmax(np.full(n, 3.25))
        assert np.all(p == 1.0 / n)          # exact: every exponential is 1


def test_selection_softmax_two_scores_are_logistic():
    rng = np.random.default_rng(5)
    for a, b in rng.standard_normal((20, 2)) * 10:
        p = orc.selection_softmax([a, b])
        # the logistic function of the difference, written through tanh
        assert abs(p[0] - 0.5 * (1.0 + np.tanh((a - b) / 2.0))) <= 1e-15


def test_selection_softmax_invariants():
    rng = np.random.default_rng(6)
    s = np.sort(rng.standard_normal(300) * 4)[::-1]
    s = np.concatenate([s, np.full(212, -np.inf)])
    p = orc.selection_softmax(s)
    assert abs(np.sum(p) - 1.0) <= 1e-13
    assert np.all(p[300:] == 0.0) and np.all(p[:300] > 0.0)
    assert np.all(np.diff(p[:300]) <= 0)                 # descending scores, descending weights
    np.testing.assert_allclose(orc.selection_softmax(s + 7.5), p, rtol=1e-12)   # shift invariance
    # ratio of two weights is the exponential of the score difference
    assert abs(p[0] / p[1] - np.exp(s[0] - s[1])) <= 1e-12 * np.exp(s[0] - s[1])


def test_selection_softmax_empty_row():
    assert np.all(orc.selection_softmax(np.full(16, -np.inf)) == 0.0)
    assert orc.selection_softmax(np.zeros(0)).size == 0


# ---------------------------------------------------------------- sparse attention

def _mla_case(rng, T, H, dk=40, dv=32, scale=3.0):
    q = rng.standard_normal((T, H, dk)) * scale
    kv = rng.standard_normal((T, dk))
    return q, kv, dv


def test_sparse_attention_full_selection_is_causal_sdpa():
    # every causal key selected: dense causal attention, here torch's scaled_dot_product_attention
    # (float64, CPU) with the shared entry expanded to every head and the value its first dv
    # elements; two packed documents through a block-diagonal causal mask
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(21)
    docs = [13, 7]
    T, H = sum(docs), 4
    q, kv, dv = _mla_case(rng, T, H)
    cu = np.concatenate([[0], np.cumsum(docs)])
    K = max(docs)
    idx = np.full((T, K), -1, np.int64)
    allowed = np.zeros((T, T), bool)
    for b in range(len(docs)):
        for u in range(docs[b]):
            t = cu[b] + u
            idx[t, :u + 1] = np.arange(cu[b], t + 1)[::-1]          # any slot order
            allowed[t, cu[b]:t + 1] = True
    sm = 0.3
    out, lse = orc.sparse_attention(q, kv, idx, sm, dv=dv)
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [H, T, dk]
    kt = torch.from_numpy(kv)[None].expand(H, T, -1)
    vt = torch.from_numpy(kv[:, :dv])[None].expand(H, T, -1)
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(allowed), scale=sm)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_sparse_attention_single_and_identical_entries():
    rng = np.random.default_rng(22)
    q, kv, dv = _mla_case(rng, 6, 3)
    sm = 0.7
    for t in range(6):
        j = (3 * t + 1) % 6
        idx = np.full((6, 5), -1)
        idx[t, 2] = j                                                 # one entry, any slot
        out, lse = orc.sparse_attention(q, kv, idx, sm, dv=dv)
        assert np.array_equal(out[t], np.broadcast_to(kv[j, :dv], (3, dv)))    # weight exactly 1
        np.testing.assert_allclose(lse[t], sm * (q[t] @ kv[j]), rtol=1e-14)
    # n equal entries: the value itself, log-sum-exp raised by log n
    kv2 = np.tile(kv[:1], (6, 1))
    idx = np.tile(np.arange(6), (6, 1))
    out, lse = orc.sparse_attention(q, kv2, idx, sm, dv=dv)
    np.testing.assert_allclose(out, np.broadcast_to(kv[0, :dv], out.shape), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, sm * (q @ kv[0]) + np.log(6.0), rtol=1e-13)


def test_sparse_attention_two_entries_are_logistic():
    rng = np.random.default_rng(23)
    q, kv, dv = _mla_case(rng, 4, 2, scale=0.5)
    idx = np.tile([1, 3], (4, 1))
    out, _ = orc.sparse_attention(q, kv, idx, 1.0, dv=dv)
    for t in range(4):
        for h in range(2):
            d = q[t, h] @ kv[1] - q[t, h] @ kv[3]
            w = 0.5 * (1.0 + np.tanh(d / 2.0))                       # logistic function of the difference
            np.testing.assert_allclose(out[t, h], w * kv[1, :dv] + (1 - w) * kv[3, :dv], rtol=1e-12, atol=1e-13)


def test_sparse_attention_slots_padding_lengths():
    rng = np.random.default_rng(24)
    T, S = 5, 30
    q = rng.standard_normal((T, 4, 40))
    kv = rng.standard_normal((S, 40))
    idx = np.stack([rng.choice(S, 12, replace=False) for _ in range(T)])
    out, lse = orc.sparse_attention(q, kv, idx, 0.25, dv=32)
    # slot order does not matter; empty slots (-1) and out-of-range indices are ignored
    perm = idx[:, rng.permutation(12)]
    padded = np.concatenate([perm, np.full((T, 3), -1), np.full((T, 2), S + 4)], axis=1)
    out2, lse2 = orc.sparse_attention(q, kv, padded[:, rng.permutation(17)], 0.25, dv=32)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # supplied lengths cut the slot list
    lens = np.array([0, 1, 5, 12, 40])
    out3, lse3 = orc.sparse_attention(q, kv, idx, 0.25, dv=32, lengths=lens)
    assert np.all(out3[0] == 0.0) and np.all(np.isneginf(lse3[0]))           # nothing selected
    for t in range(1, T):
        o, l = orc.sparse_attention(q[t:t + 1], kv, idx[t:t + 1, :min(lens[t], 12)], 0.25, dv=32)
        np.testing.assert_allclose(out3[t], o[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse3[t], l[0], rtol=1e-13)
    # a slot listed twice counts twice: like one entry whose score is raised by log 2
    dup = np.concatenate([idx[:, :1], idx[:, :4]], axis=1)
    o_dup, l_dup = orc.sparse_attention(q, kv, dup, 0.25, dv=32)
    s = 0.25 * np.einsum("thd,tjd->thj", q, kv[idx[:, :4]])
    s[:, :, 0] += np.log(2.0)
    e = np.exp(s - s.max(axis=2, keepdims=True))
    w = e / e.sum(axis=2, keepdims=True)
    np.testing.assert_allclose(o_dup, np.einsum("thj,tjc->thc", w, kv[idx[:, :4], :32]), rtol=1e-12, atol=1e-13)


def test_sparse_attention_splits_merge():
    # attention over a union of two disjoint selections is the log-sum-exp weighted merge of
    # the two partial attentions (the identity split-KV kernels rely on)
    rng = np.random.default_rng(25)
    T, S = 6, 50
    q = rng.standard_normal((T, 3, 40)) * 2
    kv = rng.standard_normal((S, 40))
    idx = np.stack([rng.choice(S, 20, replace=False) for _ in range(T)])
    o, l = orc.sparse_attention(q, kv, idx, 0.5, dv=32)
    oa, la = orc.sparse_attention(q, kv, idx[:, :7], 0.5, dv=32)
    ob, lb = orc.sparse_attention(q, kv, idx[:, 7:], 0.5, dv=32)
    lm = np.logaddexp(la, lb)
    np.testing.assert_allclose(l, lm, rtol=1e-13)
    merged = np.exp(la - lm)[..., None] * oa + np.exp(lb - lm)[..., None] * ob
    np.testing.assert_allclose(o, merged, rtol=1e-11, atol=1e-12)
