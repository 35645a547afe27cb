"""Seeded synthetic inputs for the indexer workloads (shared by tests, smoke and bench).

This module creates input data only; it holds none of the indexer's arithmetic.
Values drawn here are handed unchanged to both the HIP library and the CPU
oracle. numpy's PCG64 generator (``numpy.random.default_rng(seed)``) draws
every value, in a fixed order per workload.

Recipe (the pages run their checks on mock data and random weights, and name no
dataset; these shapes and distributions are the workloads):

* "bf16 ~N(0,1)": fp32 standard normal draws rounded to nearest-even bf16.
* w [T,H]: fp32 normal with standard deviation 1/sqrt(H).
* LayerNorm gamma = 1 + 0.1*N(0,1), beta = 0.1*N(0,1), fp32.
* KPool gate: bf16 N(0,1) logits; per-slot bias fp32 normal with variance 0.02.
* Draw order: (document lengths,) q, k, w, gamma, beta, gate, bias.
* RoPE angle table: cos/sin of u * base**(-2j/R) computed in float64 and rounded
  to fp32, one row per position. The library receives the table as data, like
  gamma and beta.
"""

import numpy as np

# workload id -> definition
WORKLOADS = {
    1: dict(name="single-seq-512-h16-d64-nope-bf16", docs=[512], H=16, D=64, topk=64,
            precision="bf16", rope_dim=0, layernorm=False, rope_fp32=False, kpool=1,
            preprocess=False),
    2: dict(name="batch4x2048-h32-d128-ln-rope64-fp32-bf16", docs=[2048] * 4, H=32, D=128,
            topk=256, precision="bf16", rope_dim=64, layernorm=True, rope_fp32=True, kpool=1,
            preprocess=True),
    3: dict(name="batch2x4096-h64-d128-ln-rope64-fp32-fp8", docs=[4096] * 2, H=64, D=128,
            topk=512, precision="fp8", rope_dim=64, layernorm=True, rope_fp32=True, kpool=1,
            preprocess=True),
    4: dict(name="thd-32768-12docs-h64-d128-mxfp8", docs=None, H=64, D=128, topk=2048,
            precision="mxfp8", rope_dim=0, layernorm=False, rope_fp32=False, kpool=1,
            preprocess=True),
    5: dict(name="kpool4-seq65536-h64-d128-bf16", docs=[65536], H=64, D=128, topk=2048,
            precision="bf16", rope_dim=0, layernorm=False, rope_fp32=False, kpool=4,
            preprocess=False),
}

ROPE_BASE = 10000.0
LN_EPS = 1e-6


def to_bf16_bits(x):
    """Round fp32 draws to bf16 bit patterns (nearest, ties to even). Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def thd_lengths(rng, total=32768, n_docs=12, lo=512, hi=6144):
    """Document lengths by rejection sampling: n-1 uniform draws, the last takes the rest."""
    while True:
        a = rng.integers(lo, hi + 1, n_docs - 1)
        last = total - int(a.sum())
        if lo <= last <= hi:
            return [int(v) for v in a] + [last]


def rope_table(max_pos, rope_dim, base=ROPE_BASE):
    """cos/sin [max_pos, rope_dim/2] fp32 of angle u * base**(-2j/rope_dim)."""
    if rope_dim == 0:
        return np.zeros((max(max_pos, 1), 1), np.float32), np.zeros((max(max_pos, 1), 1), np.float32)
    j = np.arange(rope_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def cu_from_lengths(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def draw(seed, docs, H, D, layernorm=False, rope_dim=0, kpool=1, rng=None):
    """Inputs for one problem: dict of numpy arrays (bf16 as uint16 bits)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    T = int(sum(docs))
    q = to_bf16_bits(rng.standard_normal((T, H, D), dtype=np.float32))
    k = to_bf16_bits(rng.standard_normal((T, D), dtype=np.float32))
    w = (rng.standard_normal((T, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))).astype(np.float32)
    out = dict(q=q, k=k, w=w, cu_seqlens=cu_from_lengths(docs), T=T, H=H, D=D,
               max_seqlen=int(max(docs)) if docs else 0, docs=list(docs))
    if layernorm:
        out["gamma"] = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
        out["beta"] = (0.1 * rng.standard_normal(D)).astype(np.float32)
    if kpool > 1:
        out["gate"] = to_bf16_bits(rng.standard_normal(T, dtype=np.float32))
        out["bias"] = (np.sqrt(0.02) * rng.standard_normal(kpool)).astype(np.float32)
    if rope_dim:
        out["cos"], out["sin"] = rope_table(out["max_seqlen"], rope_dim)
    return out


def workload(wid):
    """Inputs of a named workload (seed = workload id) plus its settings."""
    cfg = dict(WORKLOADS[wid])
    rng = np.random.default_rng(wid)
    docs = thd_lengths(rng) if cfg["docs"] is None else cfg["docs"]
    cfg["docs"] = docs
    inp = draw(wid, docs, cfg["H"], cfg["D"], cfg["layernorm"], cfg["rope_dim"], cfg["kpool"], rng=rng)
    inp.update(cfg)
    return inp


def small(seed, docs, H, D, **kw):
    """A seeded small problem with the same recipe (for parity tests)."""
    return draw(seed, docs, H, D, **kw)
