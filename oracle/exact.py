"""Exact rational brute force for tiny shapes (test infrastructure only).

Every f32 value is a dyadic rational, so the sum of A[m,k] * W[k,n] * S[k/32,n]
over k ("Q8_0 matvec", section "The tensors") is computed here with no rounding
at all, one term at a time with Python's Fraction.  Used to pin the f64 oracle.
"""

from fractions import Fraction

import numpy as np

_BLOCK = 32  # block length along K, "The tensors"


def q8_matvec_exact(A, W, S):
    """Exact C[m][n] as a nested list of Fractions (plain Python loops)."""
    A = np.asarray(A)
    W = np.asarray(W)
    S = np.asarray(S)
    M, K = A.shape
    N = W.shape[1]
    a = [[Fraction(float(A[m, k])) for k in range(K)] for m in range(M)]
    s = [[Fraction(float(S[b, n])) for n in range(N)] for b in range(S.shape[0])]
    w = W.astype(int).tolist()
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += a[m][k] * w[k][n] * s[k // _BLOCK][n]
            row.append(acc)
        out.append(row)
    return out


def dot_t_loops(A, W):
    """sum_k A[m,k] * W[n,k] with Python integers (no wrap), as a nested list."""
    A = np.asarray(A).astype(int).tolist()
    W = np.asarray(W).astype(int).tolist()
    return [[sum(x * y for x, y in zip(a_row, w_row)) for w_row in W] for a_row in A]


def q8_epilogue_exact(A, W, S, alpha, corr=None, C_old=None):
    """Exact alpha * C[m][n] + corr[m] * C_old[m][n] ("dot and tensor cores",
    "The fused epilogue"), with C the exact Q8_0 matvec; nested Fractions."""
    P = q8_matvec_exact(A, W, S)
    al = Fraction(float(alpha))
    out = []
    for m, row in enumerate(P):
        r = []
        for n, p in enumerate(row):
            y = al * p
            if corr is not None:
                y += Fraction(float(corr[m])) * Fraction(float(C_old[m][n]))
            r.append(y)
        out.append(r)
    return out


def dense_exact(A, B, transposed=False):
    """Exact sum_k A[m,k] * B[k,n] (B read as [N,K] when transposed) for f32
    operands ("dot and tensor cores", table of built-ins), as nested Fractions
    built one term at a time."""
    A = np.asarray(A)
    B = np.asarray(B)
    M, K = A.shape
    N = B.shape[0] if transposed else B.shape[1]
    a = [[Fraction(float(A[m, k])) for k in range(K)] for m in range(M)]
    b = [[Fraction(float(B[n, k] if transposed else B[k, n])) for n in range(N)] for k in range(K)]
    return [[sum((a[m][k] * b[k][n] for k in range(K)), Fraction(0)) for n in range(N)] for m in range(M)]
