"""Seeded random sweep of shapes and explicit launch plans, on the GPU,
against the oracle.

The fixed sweeps cover each kernel instance on chosen shapes; this one draws
shapes and plans at random (a fixed seed per case, so every run checks the
same cases): ragged K and N, every stream instance (vec, m_tile) with any
workgroup count the run-length cap allows, matrix-core plans with any valid
split count, fused siblings through the epilogue, and the i8 dot_t and dense
f32 products on random extents.  A
plan the library refuses up front (a run whose segments exceed the LDS
budget) must be refused with Q8_ERR_INVALID; every other case must meet the
oracle's bar.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_gemv_q8_amd import binding, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-5
CASES = 40
INSTANCES = [(v, m) for v in (16, 8, 4, 2, 1) for m in (1, 2, 4, 8) if v * m <= 32]


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def draw_stream_case(i):
    rng = np.random.default_rng((700, i))
    vec, m_tile = INSTANCES[int(rng.integers(len(INSTANCES)))]
    M = int(rng.integers(1, 10))
    N = vec * int(rng.integers(1, 3000 // vec + 1))
    K = int(rng.integers(1, 4001))
    units = math.ceil(N / (64 * vec)) * math.ceil(math.ceil(K / 32) / 4)
    lo = math.ceil(units / (16 // m_tile))
    n_wg = int(rng.integers(lo, units + 1))
    return M, K, N, {"vec": vec, "m_tile": m_tile, "workgroups": n_wg, "kind": binding.PLAN_STREAM}


def draw_matrix_case(i):
    rng = np.random.default_rng((701, i))
    M = int(rng.integers(2, 65))
    N = 4 * int(rng.integers(1, 801))  # any N % 4 == 0: 16-, 8- and 4-byte W loads
    K = int(rng.integers(1, 5001))
    KB = math.ceil(K / 32)
    s = int(rng.integers(1, min(KB, 80) + 1))
    splits = math.ceil(KB / math.ceil(KB / s))  # no empty split
    return M, K, N, {"kind": binding.PLAN_MATRIX, "workgroups": math.ceil(N / 512) * splits}


def run_q8_case(M, K, N, plan, seed):
    A, W, S = workloads.q8_inputs(M, K, N, seed)
    print(f"[random] q8 M={M} K={K} N={N} plan={plan}", flush=True)
    try:
        C = binding.q8_matvec_with_plan(to_dev(A), to_dev(W), to_dev(S), plan)
    except binding.Q8Error as e:
        assert e.status == binding.Q8_ERR_INVALID, str(e)
        return False
    torch.cuda.synchronize()
    err = oracle.normalised_error(C.cpu().numpy(), oracle.q8_matvec(A, W, S), oracle.q8_normaliser(A, W, S))
    assert err <= TOL, f"M={M} K={K} N={N} plan={plan}: normalised error {err:.3e}"
    return True


def test_random_stream_plans():
    ran = sum(run_q8_case(*draw_stream_case(i), (702, i)) for i in range(CASES))
    assert ran >= CASES * 3 // 4


def test_random_matrix_plans():
    ran = sum(run_q8_case(*draw_matrix_case(i), (703, i)) for i in range(CASES))
    assert ran == CASES


def test_random_dot_t_shapes():
    for i in range(CASES):
        rng = np.random.default_rng((704, i))
        M, K, N = int(rng.integers(1, 80)), int(rng.integers(1, 700)), int(rng.integers(1, 700))
        if i % 4 == 0:
            K = 16 * max(1, K // 16)  # the i8 matrix cores need K % 16 == 0
        A, W = workloads.dot_t_inputs(M, K, N, (705, i))
        print(f"[random] dot_t M={M} K={K} N={N}", flush=True)
        C = binding.q8_dot_t(to_dev(A), to_dev(W))
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), oracle.dot_t(A, W)), f"M={M} K={K} N={N}"


@pytest.mark.parametrize("transposed", [False, True])
def test_random_dense_shapes(transposed):
    for i in range(CASES // 2):
        rng = np.random.default_rng((706, int(transposed), i))
        M, K, N = int(rng.integers(1, 600)), int(rng.integers(1, 300)), int(rng.integers(1, 600))
        alpha = float(rng.choice([1.0, 0.5, 1.0 / math.sqrt(K)]))
        A, B = workloads.dense_inputs(M, K, N, (707, int(transposed), i), transposed)
        fn = binding.q8_dot_t_f32 if transposed else binding.q8_dot_f32
        print(f"[random] {fn.__name__} M={M} K={K} N={N} alpha={alpha}", flush=True)
        C = fn(to_dev(A), to_dev(B), alpha=alpha)
        torch.cuda.synchronize()
        ref = oracle.dense_fused(A, B, transposed, alpha)
        D = oracle.dense_fused_normaliser(A, B, transposed, alpha)
        err = oracle.normalised_error(C.cpu().numpy(), ref, D)
        assert err <= TOL, f"M={M} K={K} N={N}: normalised error {err:.3e}"


def test_random_fused_siblings():
    """1-4 sibling weight sets sharing A, through the epilogue with random
    alpha and (every other case) row factors, under random stream plans."""
    ran = 0
    for i in range(CASES // 2):
        rng = np.random.default_rng((708, i))
        M, K, N, plan = draw_stream_case(1000 + i)
        n_sib = int(rng.integers(1, 5))
        alpha = float(rng.choice([1.0, -0.5, 3.0]))
        A, Ws, Ss = workloads.q8_fused_inputs(M, K, N, n_sib, (709, i))
        corr = rng.standard_normal(M).astype(np.float32) if i % 2 else None
        C_olds = [rng.standard_normal((M, N)).astype(np.float32) for _ in range(n_sib)] if i % 2 else None
        units = n_sib * math.ceil(N / (64 * plan["vec"])) * math.ceil(math.ceil(K / 32) / 4)
        lo = math.ceil(units / (16 // plan["m_tile"]))
        plan["workgroups"] = int(rng.integers(lo, units + 1))  # the units of every sibling
        print(f"[random] fused M={M} K={K} N={N} siblings={n_sib} alpha={alpha} corr={corr is not None} "
              f"plan={plan}", flush=True)
        outs = [to_dev(C) for C in C_olds] if C_olds else None
        try:
            got = binding.q8_matvec_fused(to_dev(A), [to_dev(W) for W in Ws], [to_dev(S) for S in Ss], outs=outs,
                                          alpha=alpha, corr=to_dev(corr) if corr is not None else None, plan=plan)
        except binding.Q8Error as e:
            assert e.status == binding.Q8_ERR_INVALID, str(e)
            continue
        torch.cuda.synchronize()
        refs = oracle.q8_matvec_fused(A, list(zip(Ws, Ss)), alpha, corr, C_olds)
        for g in range(n_sib):
            D = oracle.q8_fused_normaliser(A, Ws[g], Ss[g], alpha, corr, C_olds[g] if C_olds else None)
            err = oracle.normalised_error(got[g].cpu().numpy(), refs[g], D)
            assert err <= TOL, f"case {i} sibling {g}: normalised error {err:.3e}"
        ran += 1
    assert ran >= CASES // 2 * 3 // 4
