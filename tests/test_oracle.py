"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin checks the oracle against what the pages and mathematics fix:
  * hand-derived fixtures of the definition ("Q8_0 matvec", "The tensors";
    "dot and tensor cores", table of built-ins) under tests/golden/;
  * exact rational brute force (oracle/exact.py) on tiny shapes;
  * the factoring identity ("Q8_0 matvec", "Factoring out the scale"):
    factored form against per-weight form;
  * special cases that reduce to a library routine (S == 1 is a plain
    matmul, numpy and torch);
  * closed forms (one-hot A, all-ones A and W, single block);
  * the masking reading ("Bounds"): zero-padding K is invisible.
The mutation tests at the end plant plausible mistakes in the oracle (on the
CPU, by monkeypatching its helpers) and check that the pins catch each one.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from oracle import q8_oracle as qo
from quantized_decode_gemv_q8_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS64 = 2.0 ** -53


def _rand_q8(M, K, N, seed, a_scale=1.0, s_lo=0.001, s_hi=0.02, signed_s=False):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((M, K)) * a_scale).astype(np.float32)
    W = rng.integers(-128, 128, (K, N), dtype=np.int8)
    S = rng.uniform(s_lo, s_hi, (oracle.num_blocks(K), N)).astype(np.float32)
    if signed_s:
        S *= rng.choice(np.array([-1, 1], np.float32), S.shape)
    return A, W, S


# ---------------------------------------------------------------- pin helpers

def hand_fixture_q8():
    with open(os.path.join(GOLDEN, "q8_hand_example.json")) as f:
        g = json.load(f)
    K, N = 34, 2
    A = np.zeros((1, K), np.float32)
    A[0, :32] = 0.5
    A[0, 32] = 2.0
    A[0, 33] = -1.0
    W = np.zeros((K, N), np.int8)
    W[:32, 0] = 1
    W[32, 0] = 3
    W[33, 0] = 4
    W[:32, 1] = np.arange(32) - 16
    W[32, 1] = -128
    W[33, 1] = 127
    S = np.array(g["inputs"]["S"], np.float32)
    return A, W, S, np.array(g["expected_C"]), np.array(g["expected_D"])


def pin_golden_q8(fn=None):
    fn = fn or oracle.q8_matvec
    A, W, S, C_exp, D_exp = hand_fixture_q8()
    return np.array_equal(fn(A, W, S), C_exp) and np.array_equal(oracle.q8_normaliser(A, W, S), D_exp)


def pin_exact(fn, A, W, S):
    """|fn - exact| <= (K + 64) * 2^-52 * D elementwise (rounding of an f64 sum)."""
    C = fn(A, W, S)
    D = oracle.q8_normaliser(A, W, S)
    ex = oracle.q8_matvec_exact(A, W, S)
    K = A.shape[1]
    for m in range(A.shape[0]):
        for n in range(W.shape[1]):
            diff = abs(Fraction(float(C[m, n])) - ex[m][n])
            if diff > Fraction((K + 64) * 2.0 ** -52) * Fraction(float(D[m, n])):
                return False
    return True


# ---------------------------------------------------------------- golden fixtures

def test_golden_q8_hand_example():
    A, W, S, C_exp, D_exp = hand_fixture_q8()
    assert np.array_equal(oracle.q8_matvec_factored(A, W, S), C_exp)
    assert np.array_equal(oracle.q8_matvec_per_weight(A, W, S), C_exp)
    assert np.array_equal(oracle.q8_normaliser(A, W, S), D_exp)
    assert pin_golden_q8()


def test_golden_dot_t_hand_example():
    with open(os.path.join(GOLDEN, "dot_t_hand_example.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], np.int8)
    W = np.array(g["W"], np.int8)
    C = oracle.dot_t(A, W)
    assert C.dtype == np.int32
    assert np.array_equal(C, np.array(g["expected_C"], np.int32))


# ---------------------------------------------------------------- exact brute force

@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (1, 5, 3), (2, 31, 4), (1, 32, 7), (3, 33, 5),
                                   (1, 64, 3), (2, 65, 2), (1, 100, 9)])
def test_oracle_matches_exact(M, K, N):
    A, W, S = _rand_q8(M, K, N, seed=[M, K, N])
    assert pin_exact(oracle.q8_matvec_factored, A, W, S)
    assert pin_exact(oracle.q8_matvec_per_weight, A, W, S)


def test_tiny_workload_matches_exact():
    A, W, S = workloads.make("tiny")
    assert A.shape == (1, 256) and W.shape == (256, 128) and S.shape == (8, 128)
    assert pin_exact(oracle.q8_matvec, A, W, S)


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(M=st.integers(1, 3), K=st.integers(1, 90), N=st.integers(1, 6),
       seed=st.integers(0, 2 ** 32 - 1), aexp=st.integers(-20, 20), sexp=st.integers(-10, 10))
def test_oracle_matches_exact_adversarial(M, K, N, seed, aexp, sexp):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((M, K)) * 2.0 ** aexp).astype(np.float32)
    # extreme bytes and wildly scaled, signed scales
    W = rng.choice(np.array([-128, -127, -1, 0, 1, 126, 127], np.int8), (K, N))
    S = (rng.uniform(-1, 1, (oracle.num_blocks(K), N)) * 2.0 ** sexp).astype(np.float32)
    assert pin_exact(oracle.q8_matvec, A, W, S)


# ---------------------------------------------------------------- factoring identity

@pytest.mark.parametrize("M,K,N", [(1, 256, 128), (4, 4100, 300), (1, 4096, 64), (2, 8192, 33)])
def test_factoring_identity(M, K, N):
    """Factored (one scale per block and column) equals per-weight scaling."""
    A, W, S = _rand_q8(M, K, N, seed=[7, M, K, N])
    Cf = oracle.q8_matvec_factored(A, W, S)
    Cp = oracle.q8_matvec_per_weight(A, W, S)
    D = oracle.q8_normaliser(A, W, S)
    assert np.all(np.abs(Cf - Cp) <= 4 * (K + 64) * EPS64 * D)


# ---------------------------------------------------------------- library special cases

@pytest.mark.parametrize("M,K,N", [(1, 256, 128), (4, 4100, 50), (3, 31, 17)])
def test_unit_scales_is_matmul(M, K, N):
    A, W, _ = _rand_q8(M, K, N, seed=[11, K])
    S = np.ones((oracle.num_blocks(K), N), np.float32)
    C = oracle.q8_matvec(A, W, S)
    ref_np = A.astype(np.float64) @ W.astype(np.float64)
    ref_t = (torch.from_numpy(A).double() @ torch.from_numpy(W).double()).numpy()
    D = np.abs(A.astype(np.float64)) @ np.abs(W.astype(np.float64))
    tol = (K + 64) * EPS64 * 2 * D
    assert np.all(np.abs(C - ref_np) <= tol)
    assert np.all(np.abs(C - ref_t) <= tol)


def test_column_constant_scale():
    M, K, N = 2, 300, 40
    A, W, _ = _rand_q8(M, K, N, seed=12)
    c = np.random.default_rng(13).uniform(0.001, 0.02, N).astype(np.float32)
    S = np.tile(c, (oracle.num_blocks(K), 1))
    ref = c.astype(np.float64) * (A.astype(np.float64) @ W.astype(np.float64))
    C = oracle.q8_matvec(A, W, S)
    D = oracle.q8_normaliser(A, W, S)
    assert np.all(np.abs(C - ref) <= 4 * (K + 64) * EPS64 * D)


@pytest.mark.parametrize("K", [1, 7, 31, 32])
def test_single_block(K):
    A, W, S = _rand_q8(3, K, 20, seed=[14, K])
    assert S.shape[0] == 1
    ref = S[0].astype(np.float64) * (A.astype(np.float64) @ W.astype(np.float64))
    C = oracle.q8_matvec(A, W, S)
    D = oracle.q8_normaliser(A, W, S)
    assert np.all(np.abs(C - ref) <= 4 * (K + 64) * EPS64 * D)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("K,k", [(256, 0), (256, 31), (256, 32), (4100, 4099), (4100, 4096), (33, 32)])
def test_one_hot_activation(K, k):
    N = 64
    _, W, S = _rand_q8(1, K, N, seed=[15, K, k])
    A = np.zeros((1, K), np.float32)
    A[0, k] = 1.0
    C = oracle.q8_matvec(A, W, S)
    # w * s has at most 8 + 24 significant bits: exact in f64
    assert np.array_equal(C[0], W[k].astype(np.float64) * S[k // 32].astype(np.float64))


@pytest.mark.parametrize("K", [256, 4100, 33, 1])
def test_all_ones(K):
    N = 16
    S = np.random.default_rng(16).uniform(0.001, 0.02, (oracle.num_blocks(K), N)).astype(np.float32)
    A = np.ones((1, K), np.float32)
    W = np.ones((K, N), np.int8)
    rows = np.array([min(32, K - 32 * b) for b in range(oracle.num_blocks(K))], np.float64)
    ref = (rows[:, None] * S.astype(np.float64)).sum(axis=0)
    C = oracle.q8_matvec(A, W, S)
    assert np.allclose(C[0], ref, rtol=8 * EPS64 * oracle.num_blocks(K), atol=0)
    if K == 4100:
        assert rows[-1] == 4  # the masked remainder holds 4 rows


@pytest.mark.parametrize("K", [1, 33, 4100, 100])
def test_zero_padding_is_invisible(K):
    """Masked rows contribute nothing: padding K to 32*KB with zeros changes nothing."""
    M, N = 2, 24
    A, W, S = _rand_q8(M, K, N, seed=[17, K])
    Kp = 32 * oracle.num_blocks(K)
    Ap = np.zeros((M, Kp), np.float32)
    Ap[:, :K] = A
    Wp = np.zeros((Kp, N), np.int8)
    Wp[:K] = W
    assert np.array_equal(oracle.q8_matvec(Ap, Wp, S), oracle.q8_matvec(A, W, S))


# ---------------------------------------------------------------- normaliser and error

def test_normaliser_properties():
    A, W, S = _rand_q8(3, 500, 50, seed=18, signed_s=True)
    C = oracle.q8_matvec(A, W, S)
    D = oracle.q8_normaliser(A, W, S)
    assert np.all(D >= np.abs(C) * (1 - 1e-12))
    # all terms positive: D == C up to f64 rounding
    Ap = np.abs(A)
    Wp = np.abs(W.astype(np.int16)).clip(0, 127).astype(np.int8)
    Sp = np.abs(S)
    Cp = oracle.q8_matvec(Ap, Wp, Sp)
    Dp = oracle.q8_normaliser(Ap, Wp, Sp)
    assert np.allclose(Cp, Dp, rtol=1e-12, atol=0)
    # a zero row of A gives D == 0 and C == 0
    A[1] = 0
    assert np.all(oracle.q8_normaliser(A, W, S)[1] == 0)
    assert np.all(oracle.q8_matvec(A, W, S)[1] == 0)


def test_normalised_error_semantics():
    D = np.array([[1.0, 0.0, 2.0]])
    ref = np.array([[1.0, 0.0, -1.0]])
    assert oracle.normalised_error(ref, ref, D) == 0.0
    assert oracle.normalised_error(np.array([[1.5, 0.0, -1.0]]), ref, D) == 0.5
    assert oracle.normalised_error(np.array([[1.0, -0.0, -1.0]]), ref, D) == 0.0
    assert oracle.normalised_error(np.array([[1.0, 1e-30, -1.0]]), ref, D) == np.inf
    assert oracle.normalised_error(np.zeros((0, 3)), np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


def test_empty_and_k0():
    A = np.zeros((2, 0), np.float32)
    W = np.zeros((0, 5), np.int8)
    S = np.zeros((0, 5), np.float32)
    assert np.array_equal(oracle.q8_matvec(A, W, S), np.zeros((2, 5)))
    assert oracle.q8_matvec(np.zeros((0, 4), np.float32), np.zeros((4, 3), np.int8),
                            np.zeros((1, 3), np.float32)).shape == (0, 3)


def test_shape_validation():
    with pytest.raises(ValueError):
        oracle.q8_matvec(np.zeros((1, 33), np.float32), np.zeros((33, 4), np.int8), np.zeros((1, 4), np.float32))
    with pytest.raises(ValueError):
        oracle.q8_matvec(np.zeros((1, 32), np.float32), np.zeros((32, 4), np.uint8), np.zeros((1, 4), np.float32))


# ---------------------------------------------------------------- dot_t

@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 7, 5), (4, 64, 4), (17, 33, 9)])
def test_dot_t_matches_loops(M, K, N):
    rng = np.random.default_rng([19, M, K, N])
    A = rng.integers(-128, 128, (M, K), dtype=np.int8)
    W = rng.integers(-128, 128, (N, K), dtype=np.int8)
    assert np.array_equal(oracle.dot_t(A, W), np.array(oracle.dot_t_loops(A, W), np.int64))


def test_dot_t_matches_f64_blas_and_torch():
    A, W = workloads.dot_t_inputs(16, 4096, 256, seed=(5, 9))
    C = oracle.dot_t(A, W)
    # |partial sums| <= 4096 * 2^14 < 2^53: f64 BLAS is exact here
    ref = (A.astype(np.float64) @ W.astype(np.float64).T).astype(np.int64)
    assert np.array_equal(C, ref)
    ref_t = (torch.from_numpy(A).long() @ torch.from_numpy(W).long().T).numpy()
    assert np.array_equal(C, ref_t)


def test_dot_t_closed_forms():
    K = 4096
    A = np.full((2, K), -128, np.int8)
    W = np.full((3, K), -128, np.int8)
    assert np.all(oracle.dot_t(A, W) == K * 16384)
    W[1] = 127
    assert np.all(oracle.dot_t(A, W)[:, 1] == -128 * 127 * K)
    # the exact sum 2^31 does not fit: reduced modulo 2^32 it is -2^31
    K = 131072
    A = np.full((1, K), -128, np.int8)
    W = np.full((1, K), -128, np.int8)
    assert oracle.dot_t(A, W)[0, 0] == -(2 ** 31)
    assert oracle.dot_t(A[:, :K - 1], W[:, :K - 1])[0, 0] == 2 ** 31 - 16384


def test_wrap_i32():
    x = np.array([0, 1, -1, 2 ** 31 - 1, 2 ** 31, -(2 ** 31), -(2 ** 31) - 1, 2 ** 32 + 5], np.int64)
    assert oracle.wrap_i32(x).tolist() == [0, 1, -1, 2 ** 31 - 1, -(2 ** 31), -(2 ** 31), 2 ** 31 - 1, 5]


# ---------------------------------------------------------------- mutation tests
# Each planted mistake is a plausible slip in the oracle; at least one pin must catch it.

def _mut_drop_remainder(b, K):
    k0 = b * 32
    return (k0, k0 + 32) if k0 + 32 <= K else (k0, k0)


def _mut_scale_modulo(S, k0, k1):
    return S[np.arange(k0, k1) % S.shape[0]]


def _mut_scale_next_row(S, k0, k1):
    return S[np.minimum(np.arange(k0, k1) // 32 + 1, S.shape[0] - 1)]


def test_mutant_drop_remainder_is_caught(monkeypatch):
    monkeypatch.setattr(qo, "_block_rows", _mut_drop_remainder)
    assert not pin_golden_q8(qo.q8_matvec_factored)
    A, W, S = _rand_q8(1, 33, 3, seed=20)
    assert not pin_exact(qo.q8_matvec_factored, A, W, S)


@pytest.mark.parametrize("mutant", [_mut_scale_modulo, _mut_scale_next_row])
def test_mutant_scale_index_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(qo, "_scale_rows", mutant)
    assert not pin_golden_q8(qo.q8_matvec_per_weight)
    A, W, S = _rand_q8(1, 100, 3, seed=21)
    assert not pin_exact(qo.q8_matvec_per_weight, A, W, S)


def test_mutant_transposed_dot_t_is_caught():
    rng = np.random.default_rng(22)
    A = rng.integers(-128, 128, (5, 5), dtype=np.int8)
    W = rng.integers(-128, 128, (5, 5), dtype=np.int8)
    wrong = oracle.wrap_i32(A.astype(np.int64) @ W.astype(np.int64))  # a @ b instead of a @ b^T
    assert not np.array_equal(wrong, np.array(oracle.dot_t_loops(A, W)))


def test_mutant_sign_of_masked_scale_is_caught():
    """Using |S| in the value (a sign slip) is caught by the exact pin with signed scales."""
    A, W, S = _rand_q8(1, 40, 4, seed=23, signed_s=True)
    assert not pin_exact(lambda a, w, s: oracle.q8_matvec(a, w, np.abs(s)), A, W, S)


# ---------------------------------------------------------------- fused epilogue and siblings

def _epilogue_fixture():
    with open(os.path.join(GOLDEN, "q8_epilogue_hand_example.json")) as f:
        g = json.load(f)
    A, W, S, _, _ = hand_fixture_q8()
    inp = g["inputs"]
    corr = np.array(inp["corr"], np.float32)
    C_old = np.array(inp["C_old"], np.float32)
    return A, W, S, inp["alpha"], corr, C_old, np.array(g["expected_y"]), np.array(g["expected_D"])


def pin_golden_epilogue(fn=None):
    fn = fn or oracle.q8_epilogue
    A, W, S, alpha, corr, C_old, y_exp, D_exp = _epilogue_fixture()
    y = fn(oracle.q8_matvec(A, W, S), alpha, corr, C_old)
    return np.array_equal(y, y_exp) and np.array_equal(oracle.q8_fused_normaliser(A, W, S, alpha, corr, C_old), D_exp)


def pin_exact_epilogue(fn, A, W, S, alpha, corr, C_old):
    """|fn - exact| <= (K + 64) * 2^-52 * D_fused elementwise."""
    y = fn(oracle.q8_matvec(A, W, S), alpha, corr, C_old)
    D = oracle.q8_fused_normaliser(A, W, S, alpha, corr, C_old)
    ex = oracle.q8_epilogue_exact(A, W, S, alpha, corr, C_old)
    K = A.shape[1]
    for m in range(A.shape[0]):
        for n in range(W.shape[1]):
            if abs(Fraction(float(y[m, n])) - ex[m][n]) > Fraction((K + 64) * 2.0 ** -52) * Fraction(float(D[m, n])):
                return False
    return True


def test_golden_epilogue_hand_example():
    assert pin_golden_epilogue()


@pytest.mark.parametrize("seed", [30, 31, 32])
def test_epilogue_exact(seed):
    rng = np.random.default_rng(seed)
    A, W, S = _rand_q8(3, 70, 5, seed=seed, signed_s=True)
    alpha = float(rng.choice([-3.0, 0.5, 1.0, 1.75]))
    corr = rng.standard_normal(3).astype(np.float32)
    C_old = rng.standard_normal((3, 5)).astype(np.float32)
    assert pin_exact_epilogue(oracle.q8_epilogue, A, W, S, alpha, corr, C_old)


def test_epilogue_special_cases():
    A, W, S = _rand_q8(2, 100, 7, seed=33)
    P = oracle.q8_matvec(A, W, S)
    C_old = np.random.default_rng(34).standard_normal((2, 7)).astype(np.float32)
    # alpha 1 without row factors is the plain product; alpha 0 keeps only corr * C_old
    assert np.array_equal(oracle.q8_epilogue(P), P)
    corr = np.array([0.5, -2.0], np.float32)
    assert np.array_equal(oracle.q8_epilogue(P, 0.0, corr, C_old), corr[:, None].astype(np.float64) * C_old)
    # zero row factors leave the scaled product
    assert np.array_equal(oracle.q8_epilogue(P, 3.0, np.zeros(2, np.float32), C_old), 3.0 * P)


def test_fused_siblings_are_independent_matvecs():
    A, W0, S0 = _rand_q8(2, 300, 9, seed=35)
    _, W1, S1 = _rand_q8(2, 300, 9, seed=36)
    corr = np.array([1.5, -0.25], np.float32)
    olds = [np.full((2, 9), 2.0, np.float32), np.full((2, 9), -1.0, np.float32)]
    ys = oracle.q8_matvec_fused(A, [(W0, S0), (W1, S1)], 0.75, corr, olds)
    assert len(ys) == 2
    for (W, S), y, old in zip([(W0, S0), (W1, S1)], ys, olds):
        assert np.array_equal(y, oracle.q8_epilogue(oracle.q8_matvec(A, W, S), 0.75, corr, old))


def _mut_corr_by_column(P, alpha=1.0, corr=None, C_old=None):
    y = float(alpha) * np.asarray(P, dtype=np.float64)
    if corr is not None:
        c = np.asarray(corr, dtype=np.float64)
        y = y + np.resize(c, y.shape[1])[None, :] * np.asarray(C_old, dtype=np.float64)
    return y


def _mut_alpha_on_old(P, alpha=1.0, corr=None, C_old=None):
    y = np.asarray(P, dtype=np.float64)
    if corr is not None:
        y = y + float(alpha) * np.asarray(corr, dtype=np.float64).reshape(-1, 1) * np.asarray(C_old, dtype=np.float64)
    return y


@pytest.mark.parametrize("mutant", [_mut_corr_by_column, _mut_alpha_on_old])
def test_mutant_epilogue_is_caught(mutant):
    rng = np.random.default_rng(37)
    A, W, S = _rand_q8(3, 40, 4, seed=38)
    corr = np.array([2.0, -1.0, 0.5], np.float32)
    C_old = rng.standard_normal((3, 4)).astype(np.float32)
    assert not (pin_golden_epilogue(mutant) and pin_exact_epilogue(mutant, A, W, S, 0.5, corr, C_old))


# ------------------------------------------- fused siblings: hand-derived pin

def _fused_fixture():
    with open(os.path.join(GOLDEN, "q8_fused_hand_example.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    A = np.array(inp["A"], np.float32)
    sib = [(np.array(s["W"], np.int8), np.array(s["S"], np.float32)) for s in inp["siblings"]]
    olds = [np.array(s["C_old"], np.float32) for s in inp["siblings"]]
    corr = np.array(inp["corr"], np.float32)
    return A, sib, inp["alpha"], corr, olds, g


def pin_golden_fused(fused=None, norm=None):
    """q8_matvec_fused and q8_fused_normaliser against the hand-derived
    two-sibling example (negative alpha, row factors of both signs)."""
    fused = fused or oracle.q8_matvec_fused
    norm = norm or oracle.q8_fused_normaliser
    A, sib, alpha, corr, olds, g = _fused_fixture()
    ys = fused(A, sib, alpha, corr, olds)
    ok = len(ys) == len(sib)
    ok = ok and all(np.array_equal(y, np.array(e)) for y, e in zip(ys, g["expected_y"]))
    ok = ok and all(np.array_equal(oracle.q8_matvec(A, W, S), np.array(e)) for (W, S), e in zip(sib, g["expected_P"]))
    ok = ok and all(np.array_equal(norm(A, W, S, alpha, corr, old), np.array(e))
                    for (W, S), old, e in zip(sib, olds, g["expected_D"]))
    return bool(ok)


def test_golden_fused_hand_example():
    assert pin_golden_fused()


def _mut_fused_swapped_olds(A, siblings, alpha=1.0, corr=None, C_olds=None):
    return oracle.q8_matvec_fused(A, siblings, alpha, corr, None if C_olds is None else C_olds[::-1])


def _mut_fused_alpha_on_old(A, siblings, alpha=1.0, corr=None, C_olds=None):
    out = []
    for g, (W, S) in enumerate(siblings):
        y = oracle.q8_matvec(A, W, S)
        if corr is not None:
            y = y + float(alpha) * np.asarray(corr, np.float64).reshape(-1, 1) * np.asarray(C_olds[g], np.float64)
        out.append(y)
    return out


def _mut_fused_first_weights(A, siblings, alpha=1.0, corr=None, C_olds=None):
    return oracle.q8_matvec_fused(A, [siblings[0]] * len(siblings), alpha, corr, C_olds)


def _mut_norm_signed_corr(A, W, S, alpha=1.0, corr=None, C_old=None):
    D = abs(float(alpha)) * oracle.q8_normaliser(A, W, S)
    if corr is not None:
        D = D + np.asarray(corr, np.float64).reshape(-1, 1) * np.asarray(C_old, np.float64)
    return D


def _mut_norm_signed_alpha(A, W, S, alpha=1.0, corr=None, C_old=None):
    D = float(alpha) * oracle.q8_normaliser(A, W, S)
    if corr is not None:
        D = D + np.abs(np.asarray(corr, np.float64).reshape(-1, 1) * np.asarray(C_old, np.float64))
    return D


@pytest.mark.parametrize("mutant", [_mut_fused_swapped_olds, _mut_fused_alpha_on_old, _mut_fused_first_weights])
def test_mutant_fused_siblings_is_caught(mutant):
    assert not pin_golden_fused(fused=mutant)


@pytest.mark.parametrize("mutant", [_mut_norm_signed_corr, _mut_norm_signed_alpha])
def test_mutant_fused_normaliser_is_caught(mutant):
    assert not pin_golden_fused(norm=mutant)
