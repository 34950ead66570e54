"""GPU parity of the dense f32 products q8_dot_f32 (C = A B) and q8_dot_t_f32
(C = A B^T), with the fused epilogue, against the CPU oracle through the C ABI.

Bar: max over outputs of |C_gpu - y_oracle| / D <= 1e-5, where D is
|alpha| * sum_k |A B| + |corr[m] * C_old[m,n]| (the oracle's normaliser);
D == 0 requires an exact zero.  The GPU forms each product from an exact
three-part bf16 split of both operands, dropping the three smallest part
products (together below 2^-24 |a b|), and accumulates in f32: the error
stays below about K * 2^-23 * D in the worst case and near sqrt(K) * 2^-24 * D
for these inputs, far inside the bar.  Integer-valued inputs whose sums stay
below 2^24 are exact (their high parts hold them whole) and are compared bit
for bit.
"""

import ctypes

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


def gpu_dense(A, B, transposed, alpha=1.0, corr=None, old=None):
    fn = binding.q8_dot_t_f32 if transposed else binding.q8_dot_f32
    out = to_dev(old).clone() if old is not None else None
    C = fn(to_dev(A), to_dev(B), out=out, alpha=alpha, corr=to_dev(corr) if corr is not None else None)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def assert_parity(A, B, transposed, C, alpha=1.0, corr=None, old=None):
    ref = oracle.dense_fused(A, B, transposed, alpha, corr, old)
    D = oracle.dense_fused_normaliser(A, B, transposed, alpha, corr, old)
    err = oracle.normalised_error(C, ref, D)
    assert err <= TOL, f"normalised error {err:.3e} > {TOL}"
    return err


SHAPES = [(128, 32, 128), (256, 4096, 384), (130, 1000, 77), (61, 1001, 200), (1, 5, 1),
          (300, 33, 129), (7, 7, 300), (129, 64, 257), (512, 96, 4)]


@pytest.mark.parametrize("transposed", [False, True])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_dense_parity(M, K, N, transposed):
    A, B = workloads.dense_inputs(M, K, N, (400, M, K, N, transposed), transposed)
    print(f"[dense] {'dot_t' if transposed else 'dot'} M={M} K={K} N={N}", flush=True)
    assert_parity(A, B, transposed, gpu_dense(A, B, transposed))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 31, 32, 33, 63, 64, 65, 96, 97, 127])
def test_panel_edges(K):
    # K around the 32-wide panels (4-byte and 16-byte load paths), M and N around the 128 tile
    for M, N in ((127, 129), (129, 128), (1, 256)):
        for tr in (False, True):
            A, B = workloads.dense_inputs(M, K, N, (411, M, K, N, tr), tr)
            assert_parity(A, B, tr, gpu_dense(A, B, tr))


@pytest.mark.parametrize("name", ["dot_f32_4096", "scores_4096x4096_d128"])
def test_dense_full_size_sampled_rows(name):
    wl = workloads.WORKLOADS[name]
    tr = wl.op == "dot_t_f32"
    A, B = workloads.make(name, 0)
    print(f"[dense] workload {name}", flush=True)
    alpha = 1.0 / np.sqrt(wl.K) if tr else 1.0
    C = gpu_dense(A, B, tr, alpha)
    assert np.isfinite(C).all()
    rows = np.random.default_rng(401).choice(wl.M, 48, replace=False)
    rows = np.union1d(rows, [0, 127, 128, wl.M - 1])
    assert_parity(A[rows], B, tr, C[rows], alpha)


@pytest.mark.parametrize("transposed", [False, True])
def test_more_tiles_than_workgroups(transposed):
    # 17 x 32 = 544 tiles of 128 x 128, more than two per CU, so workgroups take
    # several tiles in turn; ragged M, N and K, and the epilogue with row factors
    M, K, N = 2100, 40, 4000
    A, B = workloads.dense_inputs(M, K, N, (412, transposed), transposed)
    rng = np.random.default_rng(413)
    corr = rng.standard_normal(M).astype(np.float32)
    old = rng.standard_normal((M, N)).astype(np.float32)
    print(f"[dense] {'dot_t' if transposed else 'dot'} M={M} K={K} N={N} with row factors", flush=True)
    assert_parity(A, B, transposed, gpu_dense(A, B, transposed, 0.5, corr, old), 0.5, corr, old)
    assert_parity(A, B, transposed, gpu_dense(A, B, transposed))


@pytest.mark.parametrize("transposed", [False, True])
def test_integer_inputs_are_exact(transposed):
    rng = np.random.default_rng(402)
    M, K, N = 200, 1000, 300
    A = rng.integers(-8, 9, (M, K)).astype(np.float32)
    B = rng.integers(-8, 9, (N, K) if transposed else (K, N)).astype(np.float32)
    C = gpu_dense(A, B, transposed)
    ref = oracle.dot_t_f32(A, B) if transposed else oracle.dot_f32(A, B)
    assert np.array_equal(C, ref.astype(np.float32))  # |sum| <= 64000 < 2^24: every partial is exact


def test_dot_t_equals_dot_of_the_transpose():
    # both walk K in the same order, so the sums round identically
    A, B = workloads.dense_inputs(150, 300, 170, 403)
    C = gpu_dense(A, B, False)
    Ct = gpu_dense(A, np.ascontiguousarray(B.T), True)
    assert np.array_equal(C.view(np.uint32), Ct.view(np.uint32))


@pytest.mark.parametrize("transposed", [False, True])
def test_one_hot_rows_pick_out_b(transposed):
    K, N = 100, 260
    _, B = workloads.dense_inputs(1, K, N, 404, transposed)
    ks = [0, 1, 15, 16, 31, 32, 63, 99]
    A = np.zeros((len(ks), K), np.float32)
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = gpu_dense(A, B, transposed)
    for m, k in enumerate(ks):
        assert np.array_equal(C[m], B[:, k] if transposed else B[k])


@pytest.mark.parametrize("transposed", [False, True])
def test_epilogue(transposed):
    M, K, N = 140, 500, 150
    A, B = workloads.dense_inputs(M, K, N, (405, transposed), transposed)
    rng = np.random.default_rng(406)
    corr = rng.standard_normal(M).astype(np.float32)
    old = (rng.standard_normal((M, N)) * 30).astype(np.float32)
    for alpha in (0.125, -2.0):
        assert_parity(A, B, transposed, gpu_dense(A, B, transposed, alpha, corr, old), alpha, corr, old)
    # alpha == 0 leaves one rounding of corr * old
    C0 = gpu_dense(A, B, transposed, 0.0, corr, old)
    assert np.array_equal(C0, (corr[:, None].astype(np.float64) * old.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("transposed", [False, True])
def test_wide_dynamic_range(transposed):
    # operands spanning 2^-20 .. 2^20 with mixed signs: every part of the split matters
    rng = np.random.default_rng(410)
    M, K, N = 96, 700, 130
    A = (rng.standard_normal((M, K)) * 2.0 ** rng.integers(-20, 21, (M, K))).astype(np.float32)
    shape = (N, K) if transposed else (K, N)
    B = (rng.standard_normal(shape) * 2.0 ** rng.integers(-20, 21, shape)).astype(np.float32)
    assert_parity(A, B, transposed, gpu_dense(A, B, transposed))


def test_power_of_two_scale_is_exact():
    A, B = workloads.dense_inputs(100, 400, 100, 407, True)
    C = gpu_dense(A, B, True)
    for j in (-7, 3):
        assert np.array_equal(gpu_dense(A, B, True, 2.0 ** j), C * np.float32(2.0 ** j))


def test_misaligned_rows_take_the_narrow_loads():
    M, K, N = 70, 260, 90
    A, B = workloads.dense_inputs(M, K, N, 408)
    Ab = torch.zeros(M * K + 1, dtype=torch.float32, device=DEV)
    A_d = Ab[1:].view(M, K)  # 4-byte aligned only
    A_d.copy_(to_dev(A))
    C = binding.q8_dot_f32(A_d, to_dev(B))
    torch.cuda.synchronize()
    assert_parity(A, B, False, C.cpu().numpy())


def test_empty_and_k_zero():
    M, N = 3, 70
    corr = np.array([2.0, -1.0, 0.5], np.float32)
    old = np.full((M, N), 4.0, np.float32)
    A = np.zeros((M, 0), np.float32)
    for tr in (False, True):
        B = np.zeros((N, 0) if tr else (0, N), np.float32)
        assert np.all(gpu_dense(A, B, tr) == 0)
        assert np.array_equal(gpu_dense(A, B, tr, 3.0, corr, old), corr[:, None] * old)
    L = binding.load()
    assert L.q8_dot_f32(None, None, None, 0, 5, 0, None, None) == binding.Q8_OK


def test_canaries_and_determinism():
    M, K, N = 131, 333, 133
    A, B = workloads.dense_inputs(M, K, N, 409, True)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    buf[:pad] = 1.0
    buf[-pad:] = -2.0
    out = buf[pad:pad + M * N].view(M, N)
    binding.q8_dot_t_f32(to_dev(A), to_dev(B), out=out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 1.0) and np.all(host[-pad:] == -2.0)
    C = out.cpu().numpy()
    assert_parity(A, B, True, C)
    again = gpu_dense(A, B, True)
    assert np.array_equal(C.view(np.uint32), again.view(np.uint32))


def test_invalid_dense_calls():
    L = binding.load()
    A = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    p = A.data_ptr()
    ep = binding.Q8Epilogue(1.0, None)
    assert L.q8_dot_f32(p, p, p, -1, 8, 4, ctypes.byref(ep), None) == binding.Q8_ERR_INVALID
    assert L.q8_dot_f32(p, None, p, 4, 8, 4, ctypes.byref(ep), None) == binding.Q8_ERR_INVALID
    assert L.q8_dot_t_f32(p + 2, p, p, 4, 8, 4, ctypes.byref(ep), None) == binding.Q8_ERR_INVALID
    assert L.q8_dot_t_f32(p, p, p, 1 << 20, 1 << 12, 4, ctypes.byref(ep), None) == binding.Q8_ERR_TOO_LARGE
    torch.cuda.synchronize()
