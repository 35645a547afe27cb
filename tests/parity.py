"""Shared test helpers: run the same seeded inputs through the HIP library (via the Python
binding) and through the CPU oracle, and compare them under the parity rules.

Parity rules (scores and selections; operands are compared byte for byte elsewhere):

* scores: |I_gpu - I_oracle| <= tau * M, M = |sm_scale| sum_h |w| sum_i |q k| (the forward
  error scale of the dot products), tau = 1e-5 for bf16 operands and 1e-3 for fp8/mxfp8;
* selections: lengths and padding equal; with theta the oracle's k-th best score of the row,
  every GPU-selected candidate c has I_or[c] >= theta - tau (M[c] + M_theta) and every
  oracle-selected candidate the GPU left out has I_or[c] <= theta + tau (M[c] + M_theta),
  i.e. only near-ties may swap; the GPU's own order is (its score descending, index
  ascending) and its scores equal its workspace scores;
* KPool: the GPU's token list equals the expansion of the GPU's own chosen pools plus the tail.
"""

import numpy as np

from oracle import formats as fm
from oracle import oracle as orc
import gen

TAU = {"bf16": 1e-5, "fp8": 1e-3, "mxfp8": 1e-3}


# ----------------------------------------------------------------- GPU side

def _torch():
    import torch
    return torch


def dev_bf16(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch = _torch()
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dev_in(a):
    """Device tensor of an input held as bf16 bits (uint16) or as float32 values."""
    return dev(a) if a.dtype == np.float32 else dev_bf16(a)


def in_f32(a):
    """fp32 values of an input held as bf16 bits (uint16) or as float32 values."""
    return np.asarray(a, np.float32) if a.dtype == np.float32 else gen.bf16_bits_to_f32(a)


def bf16_weights(inp):
    """Switch a problem to bf16 per-head weights: the values are rounded to nearest-even bf16
    (the oracle widens them exactly) and the library receives them as torch.bfloat16."""
    inp["w"] = gen.bf16_bits_to_f32(gen.to_bf16_bits(inp["w"]))
    inp["w_bf16"] = True
    return inp


def gpu_inputs(inp):
    """Device tensors of a generated problem."""
    w = dev_bf16(gen.to_bf16_bits(inp["w"])) if inp.get("w_bf16") else dev(inp["w"])
    d = dict(q=dev_in(inp["q"]), k=dev_in(inp["k"]), w=w, cu=dev(inp["cu_seqlens"]))
    for name in ("gamma", "beta", "cos", "sin", "bias"):
        if name in inp:
            d[name] = dev(inp[name])
    if "gate" in inp:
        d["gate"] = dev_bf16(inp["gate"])
    return d


def gpu_pipeline(inp, cfg, topk, d=None, keep_device=False, sm_scale=1.0):
    """Run preprocess (if cfg['preprocess']), kpool (if kpool > 1) and score_topk."""
    import sparse_attention_indexer_dsa_amd as dsa
    torch = _torch()
    d = gpu_inputs(inp) if d is None else d
    prec, kp = cfg["precision"], cfg.get("kpool", 1)
    out = {}
    if cfg.get("preprocess"):
        ops = dsa.preprocess(d["q"], d["k"], d["cu"], ln_gamma=d.get("gamma") if cfg.get("layernorm") else None,
                             ln_beta=d.get("beta") if cfg.get("layernorm") else None, ln_eps=gen.LN_EPS,
                             rope_cos=d.get("cos"), rope_sin=d.get("sin"), rope_dim=cfg.get("rope_dim", 0),
                             rope_interleaved=cfg.get("interleaved", False), rope_fp32=cfg.get("rope_fp32", False),
                             precision=prec, return_fp32=kp > 1)
        q_op, q_sc, k_op, k_sc = ops["q_op"], ops.get("q_scale"), ops["k_op"], ops.get("k_scale")
        k_src = ops.get("k_f32")
        out.update(q_op=q_op, q_scale=q_sc, k_op=k_op, k_scale=k_sc)
    else:
        assert prec == "bf16"
        q_op, q_sc, k_op, k_sc = d["q"], None, d["k"], None
        k_src = d["k"]
    cu_pools = None
    if kp > 1:
        k_op, k_sc, cu_pools = dsa.kpool(k_src, d["cu"], d["gate"], d["bias"], kp, precision=prec)
        out.update(pooled=k_op, pooled_scale=k_sc, cu_pools=cu_pools)
    T = inp["q"].shape[0]
    ws = torch.empty(max(dsa.workspace_size(T, inp["max_seqlen"], topk, kp, inp["H"], inp["D"],
                                            len(inp["docs"]), prec), 256), dtype=torch.uint8, device="cuda")
    res = dsa.score_topk(q_op, k_op, d["w"], d["cu"], inp["max_seqlen"], topk, q_scale=q_sc, k_scale=k_sc,
                         precision=prec, sm_scale=sm_scale, kpool=kp, cu_pools=cu_pools,
                         kpool_tail=cfg.get("kpool_tail", True), workspace=ws)
    out.update(res)
    out["workspace"] = ws
    torch.cuda.synchronize()
    if keep_device:
        return out
    h = {k: host(v) for k, v in out.items()}
    h["ws"] = workspace_scores(h["workspace"], T, inp["max_seqlen"], kp)
    return h


def ws_stride(max_seqlen, kp):
    max_cand = max_seqlen if kp == 1 else max_seqlen // kp
    return (max(max_cand, 1) + 63) // 64 * 64


def workspace_scores(ws_bytes, T, max_seqlen, kp):
    stride = ws_stride(max_seqlen, kp)
    return ws_bytes[:T * stride * 4].view(np.float32).reshape(T, stride)


def fetch_rows(gd, rows, T, max_seqlen, kp):
    """Host copies of the given rows of device outputs (for full-size problems)."""
    torch = _torch()
    stride = ws_stride(max_seqlen, kp)
    ws = gd["workspace"][:T * stride * 4].view(torch.float32).view(T, stride)
    r = torch.as_tensor(np.asarray(rows, np.int64), device=ws.device)
    out = {"ws": dict(zip(rows, host(ws.index_select(0, r))))}
    for name in ("scores", "indices", "lengths", "pool_indices"):
        if gd.get(name) is not None:
            out[name] = dict(zip(rows, host(gd[name].index_select(0, r))))
    if gd.get("cu_pools") is not None:
        out["cu_pools"] = host(gd["cu_pools"])
    return out


# ----------------------------------------------------------------- oracle side

def oracle_operands(inp, cfg):
    """Scoring operands (and pooled keys) computed by the oracle from the same inputs."""
    prec, kp = cfg["precision"], cfg.get("kpool", 1)
    q32 = in_f32(inp["q"])
    k32 = in_f32(inp["k"])
    if cfg.get("preprocess"):
        qc, kc = orc.preprocess(q32, k32, inp["cu_seqlens"],
                                gamma=inp.get("gamma") if cfg.get("layernorm") else None,
                                beta=inp.get("beta") if cfg.get("layernorm") else None, eps=gen.LN_EPS,
                                cos=inp.get("cos"), sin=inp.get("sin"), rope_dim=cfg.get("rope_dim", 0),
                                interleaved=cfg.get("interleaved", False), rope_fp32=cfg.get("rope_fp32", False))
    else:
        qc, kc = q32, k32
    o = {}
    o["q_op"], o["q_scale"] = orc.quantize(qc, prec)
    if kp > 1:
        pooled, cu_pools = orc.kpool(kc, inp["cu_seqlens"], inp["gate"], inp["bias"], kp)
        o["pooled"], o["pooled_scale"] = orc.quantize(pooled, prec)
        o["cu_pools"] = cu_pools
        o["k_deq"] = orc.dequantize(o["pooled"], o["pooled_scale"], prec)
    else:
        o["k_op"], o["k_scale"] = orc.quantize(kc, prec)
        o["k_deq"] = orc.dequantize(o["k_op"], o["k_scale"], prec)
    o["q_deq"] = orc.dequantize(o["q_op"], o["q_scale"], prec)
    return o


# ----------------------------------------------------------------- comparisons

def compare_rows(g, ores, inp, cfg, topk, rows, sm_scale=1.0):
    """Check the GPU outputs of the given rows against oracle results ``ores`` (index_topk)."""
    prec, kp = cfg["precision"], cfg.get("kpool", 1)
    tau = TAU[prec]
    T = inp["q"].shape[0]
    cu = np.asarray(inp["cu_seqlens"], np.int64)
    doc, pos = orc.geometry(cu, T)
    base = cu if kp == 1 else np.asarray(g["cu_pools"], np.int64)
    for t in rows:
        r = ores[int(t)]
        I, M = r["I"], r["M"]
        cand = I.size
        nsel = min(topk, cand)
        b = doc[t]
        # all candidate scores from the workspace
        gs = np.asarray(g["ws"][t][:cand], dtype=np.float64)
        # written as "within tolerance" so that a NaN (which compares false) fails
        ok = np.abs(gs - I) <= tau * M + 1e-30
        assert np.all(np.isfinite(gs)) and ok.all(), (t, np.flatnonzero(~ok)[:5], gs[~ok][:5], I[~ok][:5], M[~ok][:5])
        # selection
        gsc = g["scores"][t]
        assert np.all(np.isneginf(gsc[nsel:])), t
        if kp == 1:
            gi = g["indices"][t].astype(np.int64)
            assert g["lengths"][t] == nsel, (t, g["lengths"][t], nsel)
            assert np.all(gi[nsel:] == -1), t
            loc = gi[:nsel] - base[b]
        else:
            gp = g["pool_indices"][t].astype(np.int64)
            assert np.all(gp[nsel:] == -1), t
            loc = gp[:nsel] - base[b]
        assert np.all((loc >= 0) & (loc < cand)), (t, loc)
        assert np.unique(loc).size == nsel, t
        # GPU scores are its workspace scores, in (score desc, index asc) order
        assert np.array_equal(gsc[:nsel].astype(np.float64), gs[loc]), t
        order = np.lexsort((loc, -gsc[:nsel].astype(np.float64)))
        assert np.array_equal(order, np.arange(nsel)), t
        if nsel < cand:
            theta = r["scores"][-1]
            m_theta = M[r["sel"][-1]]
            assert np.all(I[loc] >= theta - tau * (M[loc] + m_theta)), t
            missing = np.setdiff1d(r["sel"], loc)
            assert np.all(I[missing] <= theta + tau * (M[missing] + m_theta)), t
        else:
            assert set(loc.tolist()) == set(range(cand)), t
        if kp > 1:
            toks = orc.expand(loc, int(pos[t]), kp, int(cu[b]), cfg.get("kpool_tail", True))
            gt = g["indices"][t].astype(np.int64)
            assert g["lengths"][t] == toks.size, (t, g["lengths"][t], toks.size)
            assert np.array_equal(gt[:toks.size], toks), t
            assert np.all(gt[toks.size:] == -1), t


def check_invariants(g, inp, cfg, topk, chunk=4096):
    """Size, padding, causality and order invariants on every row (vectorised in row chunks)."""
    kp = cfg.get("kpool", 1)
    T = inp["q"].shape[0]
    cu = np.asarray(inp["cu_seqlens"], np.int64)
    doc, pos = orc.geometry(cu, T)
    cand = orc.candidate_count(pos, kp)
    nsel_all = np.minimum(topk, cand)
    tail_all = np.where(cfg.get("kpool_tail", True), (pos + 1) % kp, 0) if kp > 1 else 0 * pos
    for r0 in range(0, T, chunk):
        r1 = min(T, r0 + chunk)
        nsel = nsel_all[r0:r1]
        j = np.arange(topk)[None, :]
        valid = j < nsel[:, None]
        sc = np.asarray(g["scores"][r0:r1])
        assert np.all(np.isneginf(sc[~valid])) and np.all(np.isfinite(sc[valid]))
        s64 = sc.astype(np.float64)
        d = s64[:, 1:] - np.where(valid[:, 1:], s64[:, :-1], 0.0)
        assert np.all(d[valid[:, 1:]] <= 0)
        lng = np.asarray(g["lengths"][r0:r1])
        lo = cu[doc[r0:r1]][:, None]
        t = np.arange(r0, r1)[:, None]
        idx = np.asarray(g["indices"][r0:r1]).astype(np.int64)
        if kp == 1:
            assert np.array_equal(lng, nsel)
            assert np.all(idx[~valid] == -1)
            assert np.all(((idx >= lo) & (idx <= t))[valid])
        else:
            assert np.array_equal(lng, nsel * kp + tail_all[r0:r1])
            tv = np.arange(idx.shape[1])[None, :] < lng[:, None]
            assert np.all(idx[~tv] == -1)
            assert np.all(((idx >= lo) & (idx <= t))[tv])


def config_of(inp):
    """Pipeline settings of a named workload from tests/gen.py."""
    return dict(precision=inp["precision"], preprocess=inp["preprocess"], layernorm=inp["layernorm"],
                rope_dim=inp["rope_dim"], rope_fp32=inp["rope_fp32"], interleaved=False,
                kpool=inp["kpool"], kpool_tail=True)


def sample_rows(inp, topk, kp, n_random=16, seed=0):
    """Rows worth checking: document starts and ends, the rows where the candidate count
    crosses topk, and a few random rows."""
    cu = np.asarray(inp["cu_seqlens"], np.int64)
    T = int(cu[-1])
    rows = set()
    for b in range(cu.size - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        for u in (0, 1, hi - lo - 2, hi - lo - 1, topk * kp - 2, topk * kp - 1, topk * kp, topk * kp + kp):
            if 0 <= u < hi - lo:
                rows.add(lo + u)
    rng = np.random.default_rng(seed)
    rows |= set(int(v) for v in rng.integers(0, T, n_random))
    return sorted(rows)


def oracle_operands_rows(inp, cfg, rows, keys=True):
    """Oracle operands of the sampled query rows (dict t -> values) and, if ``keys``, of all keys."""
    prec, kp = cfg["precision"], cfg.get("kpool", 1)
    rows = np.asarray(rows, np.int64)
    q32 = in_f32(inp["q"][rows])
    k32 = in_f32(inp["k"]) if keys else None
    if cfg.get("preprocess"):
        qc, kc = orc.preprocess(q32, k32, inp["cu_seqlens"],
                                gamma=inp.get("gamma") if cfg.get("layernorm") else None,
                                beta=inp.get("beta") if cfg.get("layernorm") else None, eps=gen.LN_EPS,
                                cos=inp.get("cos"), sin=inp.get("sin"), rope_dim=cfg.get("rope_dim", 0),
                                interleaved=cfg.get("interleaved", False), rope_fp32=cfg.get("rope_fp32", False),
                                q_rows=rows)
    else:
        qc, kc = q32, k32
    o = {"rows": rows}
    o["q_op"], o["q_scale"] = orc.quantize(qc, prec)
    qd = orc.dequantize(o["q_op"], o["q_scale"], prec)
    o["q_deq"] = {int(t): qd[i] for i, t in enumerate(rows)}
    if not keys:
        return o
    if kp > 1:
        pooled, cu_pools = orc.kpool(kc, inp["cu_seqlens"], inp["gate"], inp["bias"], kp)
        o["pooled"], o["pooled_scale"] = orc.quantize(pooled, prec)
        o["cu_pools"] = cu_pools
        o["k_deq"] = orc.dequantize(o["pooled"], o["pooled_scale"], prec)
    else:
        o["k_op"], o["k_scale"] = orc.quantize(kc, prec)
        o["k_deq"] = orc.dequantize(o["k_op"], o["k_scale"], prec)
    return o
