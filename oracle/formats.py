"""Number formats of the indexer's scoring operands (CPU oracle, test infrastructure).

Sources on the pages:

* bf16 scoring rounds fp32 carriers to bf16 at the scoring boundary
  (PR 8403, codex review finding 2: an fp32 carrier of 1.001 must score as 1.0).
* FP8 scoring uses E4M3 operands with UE8M0 per-vector scales
  (PR 8403, "What does this PR do?").
* MXFP8 uses E4M3 data with block scale factors (PR 5992, "Key changes":
  BF16-to-MXFP8 quantization); the block is 32 elements.

Readings where the pages are silent (each is listed in the design doc):

* E4M3 is the OCP "E4M3FN" encoding: bias 7, no infinities, the single NaN
  pattern S.1111.111, largest finite 448.
* UE8M0 is an unsigned biased exponent, value 2**(code - 127); code 255 (NaN)
  is never produced.
* The scale exponent of a vector (or block) is the smallest integer e with
  amax <= 448 * 2**e, so the payload never saturates; an all-zero vector
  gets e = 0. e is clamped to [-127, 127].
* ``pexp``: the exponential of the KPool softmax is pinned to one definition
  (Cody-Waite two-constant reduction, degree-7 Taylor polynomial evaluated with
  fused multiply-adds, exact scaling by 2**n) so that host and device agree
  bit for bit.
"""

import math
from fractions import Fraction

import numpy as np

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_bits(x):
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    NaN maps to a quiet NaN with the same sign; overflow rounds to infinity, as
    round-to-nearest requires.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return r


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to fp32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(F32)


def bf16_round(x):
    """fp32 -> bf16 -> fp32 (the value a bf16 operand carries)."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# OCP E4M3FN
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode E4M3FN bytes to float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    sub = m / 8.0 * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2((e - 7).astype(F64))
    v = s * np.where(e == 0, sub, nor)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def e4m3_encode(x):
    """Encode float64 values with |x| <= 448 to E4M3FN, round to nearest even.

    The input must already be an exact binary value (it is fp32 data times a
    power of two here), so |x| / quantum below is exact.
    """
    x = np.asarray(x, dtype=F64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: |x| > 448 would saturate")
    sign = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    _, e1 = np.frexp(a)                   # a = m * 2**e1, m in [0.5, 1)
    E = np.maximum(e1.astype(np.int64) - 1, -6)   # binade; the subnormal range shares 2**-6
    quantum = np.exp2((E - 3).astype(F64))
    n = np.rint(a / quantum).astype(np.int64)     # 3 fraction bits, ties to even
    carry = n == 16
    E = np.where(carry, E + 1, E)
    n = np.where(carry, 8, n)
    subnormal = (E == -6) & (n < 8)
    exp_field = np.where(subnormal, 0, E + 7)
    man_field = np.where(subnormal, n, n - 8)
    code = (sign << 7) | (exp_field << 3) | man_field
    code = np.where(a == 0, sign << 7, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# UE8M0 scale exponent
# --------------------------------------------------------------------------

def ue8m0_exponent(amax):
    """Smallest integer e with amax <= 448 * 2**e (0 for amax == 0), clamped to [-127, 127].

    With amax = m * 2**E (frexp, m in [0.5, 1)) and 448 = 0.875 * 2**9 this is
    e = E - 9 when m <= 0.875 and E - 8 otherwise.
    """
    a = np.asarray(amax, dtype=F64)
    m, E = np.frexp(a)
    e = E.astype(np.int64) - 9 + (m > 0.875).astype(np.int64)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127)


def quantize_fp8_blocks(x32, block):
    """Quantise fp32 data to E4M3FN with one UE8M0 scale per ``block`` trailing elements.

    ``x32`` has shape [..., D] with D % block == 0. Returns (codes uint8 [..., D],
    scale codes uint8 [..., D // block]). Per-vector FP8 is ``block = D``.
    """
    x = np.asarray(x32, dtype=F32).astype(F64)
    D = x.shape[-1]
    xb = x.reshape(x.shape[:-1] + (D // block, block))
    amax = np.max(np.abs(xb), axis=-1)
    e = ue8m0_exponent(amax)
    scaled = xb * np.exp2(-e.astype(F64))[..., None]     # exact power-of-two scaling
    codes = e4m3_encode(scaled).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_fp8_blocks(codes, scales, block):
    """Exact value of E4M3FN codes with UE8M0 block scales, as float64."""
    v = e4m3_decode(codes)
    D = v.shape[-1]
    vb = v.reshape(v.shape[:-1] + (D // block, block))
    e = np.asarray(scales, dtype=np.int64) - 127
    return (vb * np.exp2(e.astype(F64))[..., None]).reshape(v.shape)


# --------------------------------------------------------------------------
# fp32 fused multiply-add, correctly rounded
# --------------------------------------------------------------------------

def fma32(a, b, c):
    """fl32(a*b + c) with a single rounding, for fp32 a, b, c.

    a*b is exact in float64 (24 + 24 significand bits). The float64 sum s is
    rounded once; its exact error comes from Knuth's TwoSum. Converting s to
    fp32 can only mis-round when s sits exactly on an fp32 midpoint while the
    exact value does not; the error's sign then decides.
    """
    a64 = np.asarray(a, dtype=F32).astype(F64)
    b64 = np.asarray(b, dtype=F32).astype(F64)
    c64 = np.asarray(c, dtype=F32).astype(F64)
    p = a64 * b64
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    r = s.astype(F32)
    rb = r.astype(F64)
    other = np.where(s > rb, np.nextafter(r, F32(np.inf)), np.nextafter(r, F32(-np.inf)))
    mid = (rb + other.astype(F64)) * 0.5
    tie = (s == mid) & (err != 0) & np.isfinite(s)
    fixed = np.where(err > 0, np.maximum(r, other), np.minimum(r, other))
    return np.where(tie, fixed, r).astype(F32)


def ldexp32(p, n):
    """fl32(p * 2**n) for fp32 p and integer n (exact in float64, one rounding to fp32)."""
    return (np.asarray(p, dtype=F32).astype(F64) * np.exp2(np.asarray(n, dtype=F64))).astype(F32)


# --------------------------------------------------------------------------
# Pinned exponential for the KPool softmax
# --------------------------------------------------------------------------

def _f32_bits(b):
    return np.array([b], dtype=np.uint32).view(F32)[0]


LOG2E_F32 = _f32_bits(0x3FB8AA3B)      # fp32(1 / ln 2)
LN2_HI_F32 = _f32_bits(0x3F317200)     # leading bits of ln 2 (low 9 bits zero)
LN2_LO_F32 = _f32_bits(0x35BFBE8E)     # ln 2 - LN2_HI, rounded to fp32


def _rn32_fraction(q):
    """Round an exact rational to the nearest fp32 (ties to even); normal range only."""
    if q == 0:
        return F32(0.0)
    sgn = -1 if q < 0 else 1
    a = abs(q)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    quantum = Fraction(2) ** (E - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return F32(sgn * float(fl * quantum))


# c_k = fp32 value nearest to 1/k!, k = 0..7
EXP_POLY_F32 = [_rn32_fraction(Fraction(1, math.factorial(k))) for k in range(8)]


def pexp(z):
    """Pinned fp32 exp for z <= 0 (the KPool softmax numerators).

    0 for z < -104. Otherwise n = rint(fl32(z * log2e)) (ties to even),
    r = fma(-n, ln2_lo, fma(-n, ln2_hi, z)), p = sum_k r**k / k! for k <= 7 by
    Horner's rule with fused multiply-adds, result fl32(p * 2**n).
    """
    z_in = np.asarray(z, dtype=F32)
    z = np.maximum(z_in, F32(-104.0))          # below -104 the result is 0 (masked at the end)
    t = z * LOG2E_F32
    n = np.rint(t).astype(F32)
    negn = -n
    r = fma32(negn, LN2_HI_F32, z)
    r = fma32(negn, LN2_LO_F32, r)
    p = np.full(z.shape, EXP_POLY_F32[7], dtype=F32)
    for k in range(6, -1, -1):
        p = fma32(p, r, EXP_POLY_F32[k])
    out = ldexp32(p, n.astype(F64))
    return np.where(z_in < F32(-104.0), F32(0.0), out).astype(F32)
