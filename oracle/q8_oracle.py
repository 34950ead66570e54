"""f64 reference for the Q8_0 matvec and the i8 dot_t (test infrastructure only).

Pages: "Q8_0 matvec" (sections "The tensors", "Factoring out the scale",
"Bounds") and "dot and tensor cores" (table of built-ins, "Hardware paths").

Readings taken where the pages are silent:
  * M > 1: the pages show one activation row; each row of A is an independent
    matvec with the same formula.
  * K not a multiple of 32: KB = ceil(K/32) scale rows; the last one applies to
    the K - 32*(KB-1) rows that exist (the K loop is whole blocks plus one
    masked remainder, "Bounds").
  * Layouts are dense row-major: A [M,K], W [K,N], S [KB,N], C [M,N]; for
    dot_t, A [M,K] and W [N,K] (weights stored one output row per row).
  * C is overwritten, never accumulated into.
  * dot_t contracts the full K and returns the exact sum reduced modulo 2^32
    into int32 (two's complement); that is the exact integer result whenever
    |sum| < 2^31.
"""

import numpy as np

#: Q8_0 block length along the contraction axis ("The tensors": row b of S
#: scales rows 32*b up to 32*b + 32 of W).
BLK = 32


def num_blocks(K):
    """KB, the number of scale rows: ceil(K / 32)."""
    return (int(K) + BLK - 1) // BLK


def _check_q8(A, W, S):
    if A.ndim != 2 or W.ndim != 2 or S.ndim != 2:
        raise ValueError("A, W, S must be rank 2")
    M, K = A.shape
    if W.shape[0] != K:
        raise ValueError(f"W has {W.shape[0]} rows, A has K={K}")
    N = W.shape[1]
    if S.shape != (num_blocks(K), N):
        raise ValueError(f"S must be [{num_blocks(K)}, {N}], got {S.shape}")
    if W.dtype != np.int8:
        raise ValueError("W must be int8")
    return M, K, N


def _block_rows(b, K):
    """Rows [k0, k1) of W covered by block b; the last block may be short."""
    k0 = b * BLK
    return k0, min(int(K), k0 + BLK)


def _scale_rows(S, k0, k1):
    """Scale row of each weight row k in [k0, k1): S[k // 32] ("The tensors")."""
    return S[np.arange(k0, k1) // BLK]


def q8_matvec_factored(A, W, S):
    """C = sum over blocks b of S[b,:] * (A[:, rows_b] @ W[rows_b, :]), in f64.

    This is the loop of the "Q8_0 matvec" page taken block by block: the
    unscaled partial of each block (a library matmul over at most 32 rows),
    then one multiply by that block's scales ("Factoring out the scale"), then
    the accumulate.  All inputs are upcast to f64 exactly (f32 and i8 embed
    in f64).  Returns an f64 array [M, N].
    """
    M, K, N = _check_q8(A, W, S)
    C = np.zeros((M, N), dtype=np.float64)
    A64 = np.asarray(A, dtype=np.float64)
    for b in range(num_blocks(K)):
        k0, k1 = _block_rows(b, K)
        part = A64[:, k0:k1] @ W[k0:k1].astype(np.float64)
        C += part * S[b].astype(np.float64)
    return C


def q8_matvec_per_weight(A, W, S, chunk=256):
    """C = sum_k A[:, k] (x) (W[k, :] * S[k // 32, :]), in f64.

    The definition of "The tensors" with the scale applied to every weight
    (no factoring).  Rows of W are processed ``chunk`` at a time, each chunk's
    dequantised weights contracted with a library matmul.
    """
    M, K, N = _check_q8(A, W, S)
    C = np.zeros((M, N), dtype=np.float64)
    A64 = np.asarray(A, dtype=np.float64)
    for k0 in range(0, K, chunk):
        k1 = min(K, k0 + chunk)
        dq = W[k0:k1].astype(np.float64) * _scale_rows(S, k0, k1).astype(np.float64)
        C += A64[:, k0:k1] @ dq
    return C


def q8_normaliser(A, W, S, chunk=256):
    """D[m,n] = sum_k |A[m,k] * W[k,n] * S[k//32, n]| in f64.

    The scale of the error bound: every rounding error of any summation order
    of the terms of C[m,n] is a multiple of a term's magnitude, so
    |C_computed - C| / D is the order-independent relative error.
    """
    M, K, N = _check_q8(A, W, S)
    D = np.zeros((M, N), dtype=np.float64)
    A64 = np.abs(np.asarray(A, dtype=np.float64))
    for k0 in range(0, K, chunk):
        k1 = min(K, k0 + chunk)
        dq = np.abs(W[k0:k1].astype(np.float64) * _scale_rows(S, k0, k1).astype(np.float64))
        D += A64[:, k0:k1] @ dq
    return D


#: The oracle's default form.
q8_matvec = q8_matvec_factored


def normalised_error(C_test, C_ref, D):
    """max over outputs of |C_test - C_ref| / D.

    Where D == 0 every term is zero, so the exact result is 0 and C_test must
    be exactly zero (either sign): such an output contributes 0 if it is, and
    +inf if it is not.
    """
    C_test = np.asarray(C_test, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    if C_test.shape != C_ref.shape or C_ref.shape != D.shape:
        raise ValueError("shape mismatch")
    if C_test.size == 0:
        return 0.0
    diff = np.abs(C_test - C_ref)
    zero = D == 0
    err = np.where(zero, np.where(diff == 0, 0.0, np.inf), diff / np.where(zero, 1.0, D))
    return float(err.max())


def q8_epilogue(P, alpha=1.0, corr=None, C_old=None):
    """The fused epilogue of "dot and tensor cores" ("The fused epilogue"), f64.

    The page lets the elementwise statement that consumes a product run while
    the product is being written, with no separate pass over the result; its
    examples multiply a product by a scale (s = s * scale) and multiply an
    existing accumulator by a factor before adding a product (acc = acc * corr
    + dot).  Here y[m,n] = alpha * P[m,n] + corr[m] * C_old[m,n], or
    alpha * P[m,n] without row factors.
    """
    y = float(alpha) * np.asarray(P, dtype=np.float64)
    if corr is not None:
        corr64 = np.asarray(corr, dtype=np.float64).reshape(-1, 1)
        y = y + corr64 * np.asarray(C_old, dtype=np.float64)
    return y


def q8_matvec_fused(A, siblings, alpha=1.0, corr=None, C_olds=None):
    """Sibling projections sharing A, each through the epilogue: for sibling g
    with weights (W_g, S_g), q8_epilogue(q8_matvec(A, W_g, S_g), alpha, corr,
    C_olds[g]).  Returns a list of f64 arrays [M, N]."""
    out = []
    for g, (W, S) in enumerate(siblings):
        C_old = None if C_olds is None else C_olds[g]
        out.append(q8_epilogue(q8_matvec(A, W, S), alpha, corr, C_old))
    return out


def q8_fused_normaliser(A, W, S, alpha=1.0, corr=None, C_old=None):
    """|alpha| * D + |corr[m] * C_old[m,n]|: the sum of the magnitudes of the
    terms of one fused output (D is q8_normaliser)."""
    D = abs(float(alpha)) * q8_normaliser(A, W, S)
    if corr is not None:
        D = D + np.abs(np.asarray(corr, dtype=np.float64).reshape(-1, 1) * np.asarray(C_old, dtype=np.float64))
    return D


def wrap_i32(x):
    """Reduce integers modulo 2^32 into the int32 range (two's complement)."""
    x = np.asarray(x, dtype=np.int64)
    return (((x + (1 << 31)) % (1 << 32)) - (1 << 31)).astype(np.int32)


def dot_t(A, W):
    """C[m,n] = sum_k A[m,k] * W[n,k] for i8 A [M,K] and i8 W [N,K].

    "dot and tensor cores": dot_t contracts the last axis of both operands
    (a @ b^T); i8 operands accumulate in i32.  Computed exactly in int64 and
    reduced to int32 (exact whenever the sum fits, which holds for
    K <= 131071).
    """
    A = np.asarray(A)
    W = np.asarray(W)
    if A.ndim != 2 or W.ndim != 2 or A.shape[1] != W.shape[1]:
        raise ValueError("dot_t needs A [M,K] and W [N,K]")
    if A.dtype != np.int8 or W.dtype != np.int8:
        raise ValueError("dot_t operands must be int8")
    return wrap_i32(A.astype(np.int64) @ W.astype(np.int64).T)
