"""f64 reference for the dense f32 contractions dot and dot_t (test
infrastructure only).

Page: "dot and tensor cores".
  * Table of built-ins: dot(a, b) takes a [M,K] and b [K,N] and gives a @ b;
    dot_t(a, b) takes a [M,K] and b [N,K] and gives a @ b^T (it contracts the
    last axis of both operands: attention scores q @ k^T, or weights stored
    one output row per row).
  * Section "The k loop": the product is accumulated over panels of the
    contraction axis into an f32 accumulator tile; the panel order only
    changes rounding, so the f64 reference is the plain definition.
  * Section "Hardware paths": f32 operands with an f32 accumulator take the
    FMA path (full f32 products, no operand rounding).
  * Section "The fused epilogue": the elementwise statement that consumes a
    product (s = s * scale; acc = acc * corr + dot) runs as the product is
    written; the epilogue is the same y = alpha * P + corr[m] * C_old as the
    Q8_0 one.

Readings taken where the page is silent: layouts are
dense row-major; K == 0 gives a zero product; C is overwritten unless the
epilogue's row factors read it.
"""

import numpy as np

from .q8_oracle import q8_epilogue


def _check(A, B, transposed):
    A = np.asarray(A)
    B = np.asarray(B)
    if A.ndim != 2 or B.ndim != 2:
        raise ValueError("operands must be rank 2")
    K = A.shape[1]
    kb = B.shape[1] if transposed else B.shape[0]
    if kb != K:
        what = "[N,K]" if transposed else "[K,N]"
        raise ValueError(f"B must be {what} with K={K}, got {B.shape}")
    if A.dtype != np.float32 or B.dtype != np.float32:
        raise ValueError("dense operands must be float32")
    return A.astype(np.float64), B.astype(np.float64)


def dot_f32(A, B):
    """C[m,n] = sum_k A[m,k] * B[k,n] in f64 (dot: [M,K] x [K,N] -> a @ b)."""
    A64, B64 = _check(A, B, False)
    return A64 @ B64


def dot_t_f32(A, B):
    """C[m,n] = sum_k A[m,k] * B[n,k] in f64 (dot_t: [M,K] x [N,K] -> a @ b^T)."""
    A64, B64 = _check(A, B, True)
    return A64 @ B64.T


def dense_normaliser(A, B, transposed=False):
    """D[m,n] = sum_k |A[m,k] * B[k,n]| (B read as [N,K] when transposed):
    the sum of the magnitudes of one output's terms, the scale of its
    rounding error."""
    A64, B64 = _check(A, B, transposed)
    Bt = B64.T if transposed else B64
    return np.abs(A64) @ np.abs(Bt)


def dense_fused(A, B, transposed=False, alpha=1.0, corr=None, C_old=None):
    """The product through the fused epilogue: alpha * P + corr[m] * C_old."""
    P = dot_t_f32(A, B) if transposed else dot_f32(A, B)
    return q8_epilogue(P, alpha, corr, C_old)


def dense_fused_normaliser(A, B, transposed=False, alpha=1.0, corr=None, C_old=None):
    """|alpha| * D + |corr[m] * C_old[m,n]|, D from dense_normaliser."""
    D = abs(float(alpha)) * dense_normaliser(A, B, transposed)
    if corr is not None:
        D = D + np.abs(np.asarray(corr, dtype=np.float64).reshape(-1, 1) * np.asarray(C_old, dtype=np.float64))
    return D
