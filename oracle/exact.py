"""Exact-rational brute force used to pin the oracle (test infrastructure).

Every operand of the scoring step is a binary fraction (bf16, or E4M3 times a
power of two), so scores can be computed exactly with ``fractions.Fraction``
and sorted exactly. This module re-derives the score, the causal candidate sets,
the top-k order and the pool expansion by direct enumeration over (t, c, h, i),
sharing no code with ``oracle.oracle``. It is only practical for tiny inputs.

It also holds an exact round-to-nearest-even of a rational to fp32, which pins
``formats.fma32``.
"""

from fractions import Fraction

import numpy as np


def frac(x):
    return Fraction(float(x))


def rn32(q):
    """Nearest fp32 value (ties to even) of an exact rational, with subnormals; as a Fraction."""
    if q == 0:
        return Fraction(0)
    sgn = -1 if q < 0 else 1
    a = abs(q)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** E > a:
        E -= 1
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    E = max(E, -126)
    quantum = Fraction(2) ** (E - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** 128:
        raise OverflowError
    return sgn * v


def fma32_exact(a, b, c):
    """fl32(a*b + c) by exact rational arithmetic (a, b, c fp32)."""
    return float(rn32(frac(a) * frac(b) + frac(c)))


def brute_force(q, k, w, cu_seqlens, topk, sm_scale=1.0, kp=1, kpool_tail=True):
    """Exact scores, selection and expansion for every query row.

    q [T,H,D], k [Sk,D] (tokens, or the pooled keys in pool order), w [T,H]
    hold exact binary values. Returns a list over rows t of dicts with 'I'
    (list of Fractions over candidates), 'sel' (document-local ids),
    'indices', 'length' and, for kp > 1, 'tokens'.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, H, D = q.shape
    cu = [int(v) for v in cu_seqlens]
    sm = frac(sm_scale)
    # documents and pools by enumeration
    doc_of, pos_of, pool_base = [], [], []
    pools_before = 0
    for b in range(len(cu) - 1):
        pool_base.append(pools_before)
        pools_before += (cu[b + 1] - cu[b]) // kp
        for t in range(cu[b], cu[b + 1]):
            doc_of.append(b)
            pos_of.append(t - cu[b])
    out = []
    for t in range(T):
        b, u = doc_of[t], pos_of[t]
        if kp == 1:
            cands = [c for c in range(u + 1)]          # keys cu[b] .. t
            krow = [cu[b] + c for c in cands]
        else:
            cands = [p for p in range((u + 1) // kp)]  # pools wholly at or before u
            krow = [pool_base[b] + p for p in cands]
        scores = []
        for c, r in zip(cands, krow):
            tot = Fraction(0)
            for h in range(H):
                dot = sum((frac(q[t, h, i]) * frac(k[r, i]) for i in range(D)), Fraction(0))
                if dot > 0:
                    tot += frac(w[t, h]) * dot
            scores.append(sm * tot)
        ranked = sorted(range(len(cands)), key=lambda j: (-scores[j], cands[j]))
        sel = [cands[j] for j in ranked[:topk]]
        rec = {"I": scores, "sel": sel}
        if kp == 1:
            rec["indices"] = [cu[b] + c for c in sel]
            rec["length"] = len(sel)
        else:
            rec["indices"] = [pool_base[b] + p for p in sel]
            toks = []
            for p in sel:
                toks += [cu[b] + p * kp + r for r in range(kp)]
            if kpool_tail:
                start = (u // kp) * kp
                if start + kp - 1 > u:               # the pool holding u is incomplete
                    toks += [cu[b] + s for s in range(start, u + 1)]
            rec["tokens"] = toks
            rec["length"] = len(toks)
        out.append(rec)
    return out
