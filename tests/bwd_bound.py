"""Per-element error bound of the GPU backward against the oracle's fp64 gradients.

For every gradient element g (of dQ, dK or dV) with oracle value r and term magnitude M (the sum of the
absolute values of the terms of its defining sum, each dS_ij counted with P_ij A_i for the size of D_i's
expansion; ``oracle.attention_bwd_ex(..., mags=True)``), the test requires

    |g - r| <= (2 u + c eps) M + 1e-6,      c = n/4 + 2 D + 128,

with u the unit roundoff of the 16-bit input format (2^-8 for bf16, 2^-11 for fp16; 0 for fp32 inputs,
whose path has no 16-bit rounding), eps = 2^-24 (fp32) and n the longest sum (max of query and key
counts).  Derivation, to first order in u and eps, for 16-bit inputs:

* The forward's O is a sum of P_ij v_jd with P rounded to the input format before the product, then O
  is rounded once more: |O^ - O| <= u sum_j P_ij |v_jd| + u |O_id| <= 2 u sum_j P_ij |v_jd|.  So the
  backward's D_i = sum_d dO_id O^_id is off by at most 2 u A_i, A_i = sum_d |dO_id| sum_j P_ij |v_jd|.
* dS_ij = P_ij (dP_ij - D_i) then carries P_ij 2 u A_i from D, and its rounding to the input format
  (it is an MFMA operand of dQ and dK) adds u |dS_ij|.  P itself is recomputed in fp32 from the
  forward's lse (relative error a few tens of eps), dP_ij is an fp32 dot product over D (error at most
  D eps sum_d |dO_id| |v_jd|, and P_ij times that is at most D eps A_i).
* dK_jd = scale sum_i dS_ij q_id in fp32 (an MFMA chain: blocks of 32 or 4 products, at most n/4 blocked
  additions), rounded once at the end: the error is at most |scale| sum_i |q_id| (2 u P_ij A_i +
  u |dS_ij|) + u |dK_jd| <= 2 u MdK_jd, plus the fp32 terms, which c eps MdK covers.  dQ likewise with
  k_jd, including the atomic mode, whose fp32 partial sums only add in another order.
* dV_jd = sum_i P^_ij dO_id with P rounded: error <= u sum_i P_ij |dO_id| + u |dV_jd| <= 2 u MdV_jd.

fp32 inputs: no 16-bit roundings (u = 0); what is left are the fp32 terms above and, through D, the
forward's fp32 O (at most n/4 + 64 eps of sum_j P_ij |v_jd| per element), all inside c eps M.

fp16 values below 2^-14 (subnormal) round with an absolute error of at most 2^-25 instead of a relative
one.  For the rounded P and dS operands and the rounded outputs this adds at most 2^-25 (n A + 1) to an
element, A = max(max |dO|, |scale| max |q|, |scale| max |k|) (at most n operands per sum, each times a
factor of at most A); ``atol`` adds that for fp16.  Through the forward's O the same underflow stays
within the relative 2 u A_i term as long as the P-weighted mean sum_j P_ij |v_jd| of every column of V is
at least 2^-14 (then max(u |O_id|, 2^-25) <= u sum_j P_ij |v_jd|): true for value rows of unit scale,
as here.  bf16 and fp32 share fp32's exponent range, where such values are below 2^-126.

The absolute 1e-6 otherwise only covers fp32 rounding of values whose exact result is 0 with M = 0 (no
term at all: such elements must come out as 0 anyway).  A 1e-2 * max |g| bound per tensor, which this
replaces, let a small element be wrong by 1 % of the tensor's largest.
"""
import sys

import numpy as np

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 0.0}
EPS32 = 2.0 ** -24
ATOL = 1e-6


def _values(bits, dtype):
    """Stored elements (the tests' numpy arrays of raw 16-bit patterns, or fp32) as float64."""
    x = np.ascontiguousarray(bits)
    if dtype == "fp16":
        return x.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (x.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def atol(dtype, n, scale, q, k, do):
    """The absolute term: 1e-6, plus for fp16 the subnormal rounding of at most n operands per sum."""
    if dtype != "fp16":
        return ATOL
    a = max(np.abs(_values(do, dtype)).max(), abs(scale) * np.abs(_values(q, dtype)).max(),
            abs(scale) * np.abs(_values(k, dtype)).max())
    return ATOL + 2.0 ** -25 * (n * a + 1.0)


def bound(mag, dtype, n, d, abs_term=ATOL):
    return (2.0 * U[dtype] + (n / 4.0 + 2.0 * d + 128.0) * EPS32) * mag + abs_term


def check(name, g, r, m, dtype, n, d, what, abs_term=ATOL):
    """Assert the per-element bound; print the worst element's error in units of its bound."""
    g, r, m = (np.asarray(x, dtype=np.float64) for x in (g, r, m))
    assert g.shape == r.shape == m.shape, (g.shape, r.shape, m.shape)
    assert np.all(np.isfinite(g)), "%s %s: non-finite" % (what, name)
    if g.size == 0:
        return 0.0
    err = np.abs(g - r)
    b = bound(m, dtype, n, d, abs_term)
    ratio = err / b
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    over = int((err > b).sum())
    print("%s %s: worst err/bound %.3f at %s (err %.3e, M %.3e), max|err| %.3e, %d over" %
          (what, name, ratio[worst], tuple(int(x) for x in worst), err[worst], m[worst], err.max(), over), flush=True)
    sys.stdout.flush()
    assert over == 0, "%s %s: %d elements over the per-element bound; worst err %.3e bound %.3e at %s" % (
        what, name, over, err[worst], b[worst], tuple(int(x) for x in worst))
    return float(ratio[worst])


def check_all(got, ref, dtype, n, d, what, abs_term=ATOL):
    """got: (dQ, dK, dV) as float64 arrays; ref: the oracle's six arrays (gradients, then magnitudes)."""
    for i, name in enumerate(("dQ", "dK", "dV")):
        check(name, got[i], ref[i], ref[i + 3], dtype, n, d, what, abs_term)
