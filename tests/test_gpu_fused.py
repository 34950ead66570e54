"""GPU parity of q8_matvec_fused (sibling projections + the fused epilogue)
against the CPU oracle, called through the C ABI.

Bar: max over outputs of |C_gpu - y_oracle| / D_fused <= 1e-5, where D_fused is
|alpha| * sum |A W S| + |corr[m] * C_old[m,n]| (the oracle's fused normaliser);
D_fused == 0 requires an exact zero.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_gemv_q8_amd import binding, workloads

pytestmark = pytest.mark.gpu
TOL = 1e-5
DEV = "cuda:0"


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def rand_sibs(M, K, N, n, seed):
    A, Ws, Ss = workloads.q8_fused_inputs(M, K, N, n, seed)
    return A, list(zip(Ws, Ss))


def gpu_fused(A, sibs, alpha=1.0, corr=None, olds=None, plan=None):
    A_d = to_dev(A)
    Ws = [to_dev(W) for W, _ in sibs]
    Ss = [to_dev(S) for _, S in sibs]
    outs = [to_dev(o).clone() for o in olds] if olds is not None else None
    corr_d = to_dev(corr) if corr is not None else None
    res = binding.q8_matvec_fused(A_d, Ws, Ss, outs=outs, alpha=alpha, corr=corr_d, plan=plan)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res]


def assert_fused_parity(A, sibs, alpha, corr, olds, Cs):
    refs = oracle.q8_matvec_fused(A, sibs, alpha, corr, olds)
    worst = 0.0
    for g, ((W, S), ref, C) in enumerate(zip(sibs, refs, Cs)):
        old = None if olds is None else olds[g]
        D = oracle.q8_fused_normaliser(A, W, S, alpha, corr, old)
        err = oracle.normalised_error(C, ref, D)
        assert err <= TOL, f"sibling {g}: normalised error {err:.3e} > {TOL}"
        worst = max(worst, err)
    return worst


# ------------------------------------------------------------------ siblings

@pytest.mark.parametrize("n_sib", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(1, 4100, 5000), (3, 1000, 777), (1, 256, 128)])
def test_siblings_parity(n_sib, shape):
    M, K, N = shape
    A, sibs = rand_sibs(M, K, N, n_sib, (200, n_sib, M, K, N))
    print(f"[fused] siblings={n_sib} M={M} K={K} N={N}", flush=True)
    assert_fused_parity(A, sibs, 1.0, None, None, gpu_fused(A, sibs))


@pytest.mark.parametrize("name", ["attn_qkv_4096", "mlp_gate_up_8192x28672"])
def test_fused_workloads(name):
    A, Ws, Ss = workloads.make(name, 0)
    sibs = list(zip(Ws, Ss))
    print(f"[fused] workload {name}", flush=True)
    Cs = gpu_fused(A, sibs)
    assert all(np.isfinite(C).all() for C in Cs)
    assert_fused_parity(A, sibs, 1.0, None, None, Cs)


def test_single_sibling_matches_q8_matvec_bitwise():
    # (16, 2048, 4096) takes the matrix cores on both entry points
    for M, K, N, seed in [(1, 4096, 4096, 201), (4, 4100, 5000, 202), (16, 2048, 4096, 212)]:
        A, W, S = workloads.q8_inputs(M, K, N, seed)
        C = binding.q8_matvec(to_dev(A), to_dev(W), to_dev(S))
        torch.cuda.synchronize()
        (Cf,) = gpu_fused(A, [(W, S)])
        assert np.array_equal(C.cpu().numpy().view(np.uint32), Cf.view(np.uint32))


# ------------------------------------------------------------------ the epilogue

@pytest.mark.parametrize("alpha", [0.5, -3.0, 1.0])
def test_epilogue_parity(alpha):
    M, K, N = 4, 4100, 5000
    A, sibs = rand_sibs(M, K, N, 2, (203, int(alpha * 4) + 100))
    rng = np.random.default_rng(204)
    corr = rng.standard_normal(M).astype(np.float32)
    olds = [rng.standard_normal((M, N)).astype(np.float32) * 50 for _ in sibs]
    Cs = gpu_fused(A, sibs, alpha, corr, olds)
    assert_fused_parity(A, sibs, alpha, corr, olds, Cs)


def test_alpha_power_of_two_is_exact():
    A, sibs = rand_sibs(2, 2000, 1500, 2, 205)
    base = gpu_fused(A, sibs)
    for j in (-6, -1, 3, 7):
        scaled = gpu_fused(A, sibs, alpha=2.0 ** j)
        for b, s in zip(base, scaled):
            assert np.array_equal(s, b * np.float32(2.0 ** j))


def test_alpha_zero_keeps_corr_times_old():
    M, N = 3, 700
    A, sibs = rand_sibs(M, 500, N, 1, 206)
    rng = np.random.default_rng(207)
    corr = rng.standard_normal(M).astype(np.float32)
    old = rng.standard_normal((M, N)).astype(np.float32)
    (C,) = gpu_fused(A, sibs, 0.0, corr, [old])
    # one rounding of the exact product corr * old
    assert np.array_equal(C, (corr[:, None].astype(np.float64) * old.astype(np.float64)).astype(np.float32))


def test_zero_row_factors_leave_the_scaled_product():
    M, N = 2, 900
    A, sibs = rand_sibs(M, 1000, N, 2, 208)
    olds = [np.full((M, N), np.float32(123.0)) for _ in sibs]
    ref = gpu_fused(A, sibs, alpha=0.25)
    got = gpu_fused(A, sibs, 0.25, np.zeros(M, np.float32), olds)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)


def test_k_zero():
    M, N = 2, 300
    corr = np.array([2.0, -0.5], np.float32)
    olds = [np.full((M, N), 3.0, np.float32), np.full((M, N), -4.0, np.float32)]
    A = np.zeros((M, 0), np.float32)
    sibs = [(np.zeros((0, N), np.int8), np.zeros((0, N), np.float32)) for _ in range(2)]
    Cs = gpu_fused(A, sibs, 1.5, corr, olds)
    for C, old in zip(Cs, olds):
        assert np.array_equal(C, corr[:, None] * old)
    zeros = gpu_fused(A, sibs, 1.5, None, None)
    assert all(np.all(C == 0) for C in zeros)


# ------------------------------------------------------------------ every instance, runs across siblings

PLANS = [(v, mt) for v in (16, 8, 4, 2, 1) for mt in (1, 2, 4, 8) if v * mt <= 32]


@pytest.mark.parametrize("vec,m_tile", PLANS)
def test_every_instance_with_siblings(vec, m_tile):
    M, K, N, n_sib = 5, 3000, 2048, 3
    A, sibs = rand_sibs(M, K, N, n_sib, (209, vec, m_tile))
    units = n_sib * math.ceil(N / (64 * vec)) * math.ceil(math.ceil(K / 32) / 4)
    cap = 16 // m_tile
    corr = np.linspace(-1, 1, M).astype(np.float32)
    olds = [np.full((M, N), float(g + 1), np.float32) for g in range(n_sib)]
    ran = 0
    for n_wg in sorted({1, 7, 25, units // 3, units // 2, units, math.ceil(units / cap)}):
        if not 1 <= n_wg <= units or math.ceil(units / n_wg) > cap:
            continue
        try:
            Cs = gpu_fused(A, sibs, 0.5, corr, olds, plan={"vec": vec, "m_tile": m_tile, "workgroups": n_wg})
        except binding.Q8Error as e:
            assert e.status == binding.Q8_ERR_INVALID  # LDS budget of long runs, rejected up front
            continue
        assert_fused_parity(A, sibs, 0.5, corr, olds, Cs)
        ran += 1
    assert ran >= 2


def test_mixed_alignment_picks_a_common_vec():
    M, K, N = 2, 200, 1024
    A, sibs = rand_sibs(M, K, N, 2, 210)
    A_d = to_dev(A)
    Ws, Ss = [], []
    for g, (W, S) in enumerate(sibs):
        off = 1 if g == 1 else 0
        wbuf = torch.zeros(K * N + 16, dtype=torch.int8, device=DEV)
        Wd = wbuf[off:off + K * N].view(K, N)
        Wd.copy_(to_dev(W))
        Ws.append(Wd)
        Ss.append(to_dev(S))
    Cs = binding.q8_matvec_fused(A_d, Ws, Ss)
    torch.cuda.synchronize()
    assert_fused_parity(A, sibs, 1.0, None, None, [C.cpu().numpy() for C in Cs])


def test_invalid_fused_calls():
    A, sibs = rand_sibs(1, 64, 100, 1, 211)
    A_d, W_d, S_d = to_dev(A), to_dev(sibs[0][0]), to_dev(sibs[0][1])
    with pytest.raises(ValueError):
        binding.q8_matvec_fused(A_d, [], [])
    with pytest.raises(ValueError):
        binding.q8_matvec_fused(A_d, [W_d] * 5, [S_d] * 5)
    # straight through the C ABI: sibling counts outside 1..4 and null pointers
    L = binding.load()
    C = torch.empty((1, 100), device=DEV)
    one = (binding.Q8Sibling * 5)(*[binding.Q8Sibling(W_d.data_ptr(), S_d.data_ptr(), C.data_ptr())] * 5)
    for n in (0, 5):
        assert L.q8_matvec_fused(A_d.data_ptr(), one, n, 1, 64, 100, None, None, None) == binding.Q8_ERR_INVALID
    bad = (binding.Q8Sibling * 1)(binding.Q8Sibling(None, S_d.data_ptr(), C.data_ptr()))
    assert L.q8_matvec_fused(A_d.data_ptr(), bad, 1, 1, 64, 100, None, None, None) == binding.Q8_ERR_INVALID
    assert L.q8_matvec_fused(A_d.data_ptr(), None, 1, 1, 64, 100, None, None, None) == binding.Q8_ERR_INVALID
    ep = binding.Q8Epilogue(1.0, None)
    assert L.q8_matvec_fused(A_d.data_ptr(), one, 1, 1, 64, 100, ctypes.byref(ep), None, None) == binding.Q8_OK
    torch.cuda.synchronize()


def test_fused_deterministic():
    A, Ws, Ss = workloads.make("attn_qkv_4096", 0)
    sibs = list(zip(Ws, Ss))
    r1 = gpu_fused(A, sibs)
    r2 = gpu_fused(A, sibs)
    for a, b in zip(r1, r2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
