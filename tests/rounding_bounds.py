"""Elementwise rounding-error bounds of the bf16 Newton-Schulz path.

The HIP library stores every intermediate of the iteration in bf16 (round to
nearest even) and accumulates every product in fp32 on the matrix cores.  For
an iteration whose terms do not cancel (e.g. one or two steps of
(a, b, c) = (0, 1, 0) or (0, 0, 1)), the usual first-order forward error
analysis gives a bound on |X_gpu - X| for every element, where X is the exact
result of the same iteration on the same input.  That bound is computed here
in float64 alongside the exact iteration, and a test can then check every
element of the GPU's output against the oracle.

This is a test helper.  It does not compute the expected values (those come
from oracle.newton_schulz, and `ns_with_bound` is checked against it); it
computes how far a correct implementation can be from them.

Rounding points assumed, per iteration (X = the iterate, in the wide
orientation, zero padded to s_pad x l_pad):
  * the norm factor f = 1 / (||U||_F + eps) from fp32 partial sums of at most
    a few hundred squares (relative error NORM_REL); the first Gram and the
    first product apply f^2 and f in fp32 as they store;
  * A = rnd(s_g * X X^T), s_g = 1 (or b when c = 0), with l_pad-term fp32 sums;
  * B = rnd(c * (A A + (b/c) A)) when c != 0, the (b/c) A term added through
    bf16 hi + lo parts of b/c (relative error SPLIT) inside the fp32 sum;
  * X' = rnd(a X + B X) (B = A when c = 0), the a X term likewise.
Here rnd is the bf16 rounding (relative error at most U_BF16) and an fp32 sum
of k terms, in any order and with faithful rounding, errs by at most
gamma(k) times the sum of the terms' magnitudes.  The coefficients reach the
GPU as fp32 values (one fp32 rounding each; b/c is formed in fp32).
Second-order terms (products of two errors) are kept.
"""
from __future__ import annotations

import math

import numpy as np

U_BF16 = 2.0 ** -8        # round to nearest even, 8 significant bits: half an ulp, relative
U_FP32 = 2.0 ** -24
SPLIT = 2.0 ** -16        # a scalar as bf16 hi + rnd(s - hi): |s - hi - lo| <= 2^-16 |s|
NORM_REL = 64 * U_FP32    # the norm factor from fp32 sums of squares (all terms positive)
TILE = 256                # padding granularity of the iterate


def gamma(k: int) -> float:
    """Error of an fp32 sum of k terms relative to the sum of their magnitudes
    (two ulps per addition: covers any summation order and faithful rounding)."""
    return 2.0 * k * U_FP32


def _pad(n: int) -> int:
    return -(-n // TILE) * TILE


def ns_with_bound(u, steps: int, coeffs, eps: float = 1e-7):
    """Exact iteration (float64) on the bf16 input u and the elementwise bound.

    Returns (X, E): X the exact result in u's shape, E >= |X_gpu - X| to first
    order for a bf16 run of `steps` iterations through the rounding points above.
    """
    a, b, c = (float(t) for t in coeffs)
    u = np.asarray(u, np.float64)
    tall = u.shape[0] > u.shape[1]
    x = u.T if tall else u
    s_pad, l_pad = _pad(x.shape[0]), _pad(x.shape[1])
    f = 1.0 / (math.sqrt(float(np.sum(x * x))) + eps)
    X = f * x
    E = np.zeros_like(X)  # the iterate starts as U itself (exact in bf16); f enters below
    if steps == 0:
        # the finish pass stores rnd(f * U)
        E = U_BF16 * np.abs(X) + (NORM_REL + U_FP32) * np.abs(X)
    for k in range(steps):
        first = k == 0
        aX, aE = np.abs(X), E
        # Gram: A = rnd(s_g * X X^T)
        s_g = 1.0 if c != 0.0 else b
        A = s_g * (X @ X.T)
        absXX = aX @ aX.T
        ea = abs(s_g) * (aE @ aX.T + aX @ aE.T + aE @ aE.T + gamma(l_pad) * absXX)
        ea = ea + 2 * U_FP32 * np.abs(A)  # s_g as an fp32 value, times the sum in fp32
        if first:  # f^2 formed and applied in fp32
            ea = ea + (2 * NORM_REL + 2 * U_FP32) * np.abs(A)
        EA = U_BF16 * np.abs(A) + ea * (1 + U_BF16)
        aA = np.abs(A)
        if c != 0.0:
            r = b / c
            B = c * (A @ A) + b * A
            eb = abs(c) * (EA @ aA + aA @ EA + EA @ EA + gamma(s_pad + 2) * (aA @ aA + abs(r) * aA)
                           + abs(r) * EA + abs(r) * (SPLIT + 3 * U_FP32) * aA)
            eb = eb + 2 * U_FP32 * np.abs(c) * (aA @ aA + abs(r) * aA)  # c in fp32, c * sum
            EB = U_BF16 * np.abs(B) + eb * (1 + U_BF16)
        else:
            B, EB = A, EA
        aB = np.abs(B)
        # product: X' = rnd(a X + B X)
        Xn = a * X + B @ X
        ex = (EB @ aX + aB @ aE + EB @ aE + gamma(s_pad + 2) * (aB @ aX + abs(a) * aX)
              + abs(a) * (aE + (SPLIT + U_FP32) * aX))
        if first:  # times f in fp32
            ex = ex + (NORM_REL + U_FP32) * np.abs(Xn)
        E = U_BF16 * np.abs(Xn) + ex * (1 + U_BF16)
        X = Xn
    return (X.T, E.T) if tall else (X, E)
