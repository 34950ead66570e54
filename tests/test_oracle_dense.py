"""Pins of the dense f32 oracle (dot, dot_t and their fused epilogue) against
things other than itself (CPU only):
  * a hand-derived fixture of the definitions ("dot and tensor cores", table
    of built-ins; "The fused epilogue") under tests/golden/;
  * exact rational brute force (oracle/exact.py) on tiny, non-square shapes;
  * closed forms (all-ones A against an affine B; identity B);
  * the empty contraction (K == 0).
The mutation tests at the end plant plausible mistakes (a missing transpose,
a transposed operand, a signed normaliser) and check that the pins catch them.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import dense as od
from oracle.exact import dense_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS64 = 2.0 ** -53


def _rand(M, K, N, seed, transposed=False):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K) if transposed else (K, N)).astype(np.float32)
    return A, B


def pin_golden(dot=od.dot_f32, dot_t=od.dot_t_f32, norm=od.dense_normaliser):
    with open(os.path.join(GOLDEN, "dense_hand_example.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], np.float32)
    Bkn = np.array(g["B_kn"], np.float32)
    Bnk = np.array(g["B_nk"], np.float32)
    try:
        ok = np.array_equal(dot(A, Bkn), np.array(g["expected_dot"]))
        ok &= np.array_equal(dot_t(A, Bnk), np.array(g["expected_dot_t"]))
        ok &= np.array_equal(norm(A, Bnk, True), np.array(g["expected_dot_t_D"]))
        ok &= np.array_equal(g["scale"] * dot_t(A, Bnk), np.array(g["expected_scaled_dot_t"]))
    except ValueError:
        return False
    return bool(ok)


def pin_exact(fn, A, B, transposed):
    """|fn - exact| <= K * 2^-53 * sum |terms| (f64 rounding of K terms)."""
    try:
        got = fn(A, B)
    except ValueError:
        return False
    ex = dense_exact(A, B, transposed)
    D = dense_exact(np.abs(A), np.abs(B), transposed)
    K = A.shape[1]
    M, N = got.shape
    if (M, N) != (len(ex), len(ex[0]) if ex else 0):
        return False
    for m in range(M):
        for n in range(N):
            bound = (K + 1) * EPS64 * float(D[m][n])
            if abs(float(got[m, n]) - float(ex[m][n])) > bound:
                return False
    return True


def test_golden_hand_example():
    assert pin_golden()


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 7, 5), (5, 33, 2), (4, 64, 4), (2, 3, 9)])
def test_dot_matches_exact(M, K, N):
    A, B = _rand(M, K, N, (40, M, K, N))
    assert pin_exact(od.dot_f32, A, B, False)


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 7, 5), (5, 33, 2), (4, 64, 4), (2, 3, 9)])
def test_dot_t_matches_exact(M, K, N):
    A, B = _rand(M, K, N, (41, M, K, N), transposed=True)
    assert pin_exact(od.dot_t_f32, A, B, True)


@pytest.mark.parametrize("M,K,N", [(3, 7, 5), (4, 64, 4)])
def test_normaliser_is_the_sum_of_term_magnitudes(M, K, N):
    for tr in (False, True):
        A, B = _rand(M, K, N, (42, M, K, N, tr), transposed=tr)
        D = od.dense_normaliser(A, B, tr)
        ex = dense_exact(np.abs(A), np.abs(B), tr)
        assert np.allclose(D, np.array([[float(x) for x in r] for r in ex]), rtol=(K + 1) * EPS64, atol=0)
        C = od.dot_t_f32(A, B) if tr else od.dot_f32(A, B)
        assert np.all(np.abs(C) <= D * (1 + 1e-12))


@pytest.mark.parametrize("M,K,N", [(2, 100, 3), (1, 4100, 7), (6, 1, 1)])
def test_closed_form_affine(M, K, N):
    # A all ones, B[k,n] = k + 1000 n: C[m,n] = K(K-1)/2 + 1000 n K (exact in f64)
    A = np.ones((M, K), np.float32)
    k = np.arange(K, dtype=np.float64)[:, None]
    n = np.arange(N, dtype=np.float64)[None, :]
    B = (k + 1000 * n).astype(np.float32)
    want = np.broadcast_to(K * (K - 1) / 2 + 1000 * n * K, (M, N))
    assert np.array_equal(od.dot_f32(A, B), want)
    assert np.array_equal(od.dot_t_f32(A, np.ascontiguousarray(B.T)), want)


def test_identity():
    A, _ = _rand(5, 9, 1, 43)
    I = np.eye(9, dtype=np.float32)
    assert np.array_equal(od.dot_f32(A, I), A.astype(np.float64))
    assert np.array_equal(od.dot_t_f32(A, I), A.astype(np.float64))


def test_empty_contraction_and_shapes():
    A = np.zeros((3, 0), np.float32)
    assert np.array_equal(od.dot_f32(A, np.zeros((0, 4), np.float32)), np.zeros((3, 4)))
    assert np.array_equal(od.dot_t_f32(A, np.zeros((4, 0), np.float32)), np.zeros((3, 4)))
    with pytest.raises(ValueError):
        od.dot_f32(np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32))
    with pytest.raises(ValueError):
        od.dot_t_f32(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32))
    with pytest.raises(ValueError):
        od.dot_f32(np.zeros((2, 3), np.float64), np.zeros((3, 2), np.float32))


def test_fused_epilogue_of_the_dense_product():
    A, B = _rand(3, 20, 4, 44, transposed=True)
    rng = np.random.default_rng(45)
    corr = rng.standard_normal(3).astype(np.float32)
    old = rng.standard_normal((3, 4)).astype(np.float32)
    P = od.dot_t_f32(A, B)
    y = od.dense_fused(A, B, True, 0.125, corr, old)
    assert np.array_equal(y, 0.125 * P + corr[:, None].astype(np.float64) * old)
    D = od.dense_fused_normaliser(A, B, True, -0.5, corr, old)
    assert np.array_equal(D, 0.5 * od.dense_normaliser(A, B, True) + np.abs(corr[:, None].astype(np.float64) * old))
    assert np.array_equal(od.dense_fused(A, B, True), P)


# ------------------------------------------------------------------ mutants

def _mut_dot_t_no_transpose(A, B):
    return np.asarray(A, np.float64) @ np.asarray(B, np.float64)


def _mut_dot_transposed_b(A, B):
    return np.asarray(A, np.float64) @ np.asarray(B, np.float64).T


def _mut_signed_norm(A, B, transposed=False):
    A64 = np.asarray(A, np.float64)
    B64 = np.asarray(B, np.float64)
    return np.abs(A64) @ (B64.T if transposed else B64)


def test_mutant_missing_transpose_is_caught():
    A, B = _rand(4, 4, 4, 46, transposed=True)  # square: shapes alone do not tell
    assert not (pin_golden(dot_t=_mut_dot_t_no_transpose) and pin_exact(_mut_dot_t_no_transpose, A, B, True))


def test_mutant_transposed_operand_is_caught():
    A, B = _rand(4, 4, 4, 47)
    assert not (pin_golden(dot=_mut_dot_transposed_b) and pin_exact(_mut_dot_transposed_b, A, B, False))


def test_mutant_signed_normaliser_is_caught():
    assert not pin_golden(norm=_mut_signed_norm)


# ------------------------------------------ fused epilogue: hand-derived pin

def pin_golden_fused(fused=od.dense_fused, norm=od.dense_fused_normaliser):
    """dense_fused and dense_fused_normaliser against the hand-derived example
    with a negative alpha and row factors of both signs, for dot and dot_t."""
    with open(os.path.join(GOLDEN, "dense_hand_example.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], np.float32)
    f_ = g["fused"]
    corr = np.array(f_["corr"], np.float32)
    old = np.array(f_["C_old"], np.float32)
    ok = True
    for B, tr, key in ((np.array(g["B_nk"], np.float32), True, "dot_t"), (np.array(g["B_kn"], np.float32), False, "dot")):
        ok &= np.array_equal(fused(A, B, tr, f_["alpha"], corr, old), np.array(f_[f"expected_{key}_y"]))
        ok &= np.array_equal(norm(A, B, tr, f_["alpha"], corr, old), np.array(f_[f"expected_{key}_D"]))
    return bool(ok)


def test_golden_fused_hand_example():
    assert pin_golden_fused()


def _mut_fused_alpha_on_old(A, B, transposed=False, alpha=1.0, corr=None, C_old=None):
    P = od.dot_t_f32(A, B) if transposed else od.dot_f32(A, B)
    return P + float(alpha) * np.asarray(corr, np.float64).reshape(-1, 1) * np.asarray(C_old, np.float64)


def _mut_fused_corr_by_column(A, B, transposed=False, alpha=1.0, corr=None, C_old=None):
    P = od.dot_t_f32(A, B) if transposed else od.dot_f32(A, B)
    return float(alpha) * P + np.asarray(corr, np.float64).reshape(1, -1) * np.asarray(C_old, np.float64)


def _mut_fused_norm_signed_corr(A, B, transposed=False, alpha=1.0, corr=None, C_old=None):
    D = abs(float(alpha)) * od.dense_normaliser(A, B, transposed)
    return D + np.asarray(corr, np.float64).reshape(-1, 1) * np.asarray(C_old, np.float64)


def _mut_fused_norm_signed_alpha(A, B, transposed=False, alpha=1.0, corr=None, C_old=None):
    D = float(alpha) * od.dense_normaliser(A, B, transposed)
    return D + np.abs(np.asarray(corr, np.float64).reshape(-1, 1) * np.asarray(C_old, np.float64))


@pytest.mark.parametrize("mutant", [_mut_fused_alpha_on_old, _mut_fused_corr_by_column])
def test_mutant_dense_fused_is_caught(mutant):
    assert not pin_golden_fused(fused=mutant)


@pytest.mark.parametrize("mutant", [_mut_fused_norm_signed_corr, _mut_fused_norm_signed_alpha])
def test_mutant_dense_fused_normaliser_is_caught(mutant):
    assert not pin_golden_fused(norm=mutant)
