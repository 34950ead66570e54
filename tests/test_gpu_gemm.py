"""GPU parity of the matrix-core Q8_0 product (q8_matvec with 2..64 rows,
plan kind Q8_PLAN_MATRIX) against the CPU oracle, through the C ABI.

Bar: max over outputs of |C_gpu - C_oracle| / D <= 1e-5 (D = sum of |A W S|);
D == 0 requires an exact zero.  A is split into three bf16 parts on the GPU,
so the bar holds for any f32 activations.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_gemv_q8_amd import binding, workloads

pytestmark = pytest.mark.gpu
TOL = 1e-5
DEV = "cuda:0"
MATRIX = {"kind": binding.PLAN_MATRIX}
STREAM = {"kind": binding.PLAN_STREAM}


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def gpu_q8(A, W, S, plan=None):
    A_d, W_d, S_d = to_dev(A), to_dev(W), to_dev(S)
    C = binding.q8_matvec(A_d, W_d, S_d) if plan is None else binding.q8_matvec_with_plan(A_d, W_d, S_d, plan)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def assert_parity(A, W, S, C):
    err = oracle.normalised_error(C, oracle.q8_matvec(A, W, S), oracle.q8_normaliser(A, W, S))
    assert err <= TOL, f"normalised error {err:.3e} > {TOL}"
    return err


@pytest.mark.parametrize("M", [2, 5, 8, 16, 17, 24, 32, 33, 48, 64])
@pytest.mark.parametrize("K,N", [(4100, 4096), (1000, 1040), (96, 512), (32, 16)])
def test_matrix_parity(M, K, N):
    A, W, S = workloads.q8_inputs(M, K, N, (300, M, K, N))
    print(f"[gemm] M={M} K={K} N={N}", flush=True)
    assert_parity(A, W, S, gpu_q8(A, W, S, MATRIX))


def test_matrix_full_size_batch():
    A, W, S = workloads.make("batch16_8192x28672", 0)
    print("[gemm] batch16_8192x28672", flush=True)
    C = gpu_q8(A, W, S)
    assert binding.q8_matvec_choose_plan(16, 8192, 28672)["kind"] == binding.PLAN_MATRIX
    assert np.isfinite(C).all()
    assert_parity(A, W, S, C)


@pytest.mark.parametrize("M,K,N,kind,wgs", [
    (8, 14336, 4096, binding.PLAN_MATRIX, 8 * 32),   # a narrow W: 32 splits, one workgroup per CU
    (4, 14336, 4096, binding.PLAN_MATRIX, 8 * 32),   # 4 rows take the matrix cores there
    (8, 4100, 4096, binding.PLAN_MATRIX, 8 * 15),    # splits of at least 8 blocks (129 blocks: 15 splits of 9, the last 3)
    (16, 4096, 1024, binding.PLAN_STREAM, None),     # too narrow to fill half the device: the stream
    (2, 8192, 8192, binding.PLAN_STREAM, None),      # 2 rows below K*N = 2^27: the stream
])
def test_automatic_plans_on_narrow_weights(M, K, N, kind, wgs):
    plan = binding.q8_matvec_choose_plan(M, K, N)
    assert plan["kind"] == kind
    if wgs is not None:
        assert plan["workgroups"] == wgs
    A, W, S = workloads.q8_inputs(M, K, N, (320, M, K, N))
    print(f"[gemm] automatic plan M={M} K={K} N={N}: {plan}", flush=True)
    assert_parity(A, W, S, gpu_q8(A, W, S))


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 40])
def test_matrix_every_split(splits):
    M, K, N = 20, 1280, 1536  # KB = 40, three tiles
    A, W, S = workloads.q8_inputs(M, K, N, (301, splits))
    C = gpu_q8(A, W, S, {"kind": binding.PLAN_MATRIX, "workgroups": 3 * splits})
    assert_parity(A, W, S, C)


@pytest.mark.parametrize("M,K,N,splits", [
    (16, 18432, 1024, 64),    # eight groups of splits: the plain sequential sum
    (16, 18432, 1024, 72),    # nine groups: the cascade, one piece at a time
    (40, 18432, 1024, 576),   # 72 groups of one-block splits: two cascade levels, 64-row instance
    (16, 1 << 20, 16, None),  # automatic: 512 splits of 64 blocks
])
def test_matrix_many_splits(M, K, N, splits):
    plan = {"kind": binding.PLAN_MATRIX}
    if splits is not None:
        plan["workgroups"] = (N // 512 or 1) * splits
    else:
        assert binding.q8_matvec_choose_plan(M, K, N)["workgroups"] == 512
    A, W, S = workloads.q8_inputs(M, K, N, (330, M, K, N))
    print(f"[gemm] M={M} K={K} N={N} splits={splits}", flush=True)
    C = gpu_q8(A, W, S, plan)
    assert_parity(A, W, S, C)
    assert np.array_equal(gpu_q8(A, W, S, plan), C)  # a fixed summation order
    assert np.array_equal(gpu_q8(A, W, np.float32(4.0) * S, plan), np.float32(4.0) * C)


def test_matrix_and_stream_agree_with_the_oracle():
    A, W, S = workloads.q8_inputs(12, 3000, 2048, 302)
    assert_parity(A, W, S, gpu_q8(A, W, S, MATRIX))
    assert_parity(A, W, S, gpu_q8(A, W, S, STREAM))


def test_matrix_extreme_values():
    rng = np.random.default_rng(303)
    M, K, N = 9, 300, 1024
    A = (rng.standard_normal((M, K)) * 2.0 ** rng.integers(-20, 20, (M, K))).astype(np.float32)
    W = rng.choice(np.array([-128, -127, 0, 127], np.int8), (K, N))
    S = (rng.uniform(-1, 1, (math.ceil(K / 32), N)) * 2.0 ** rng.integers(-10, 10, (math.ceil(K / 32), N))).astype(np.float32)
    assert_parity(A, W, S, gpu_q8(A, W, S, MATRIX))


def test_matrix_one_hot_is_exact():
    K, N = 4100, 2048
    _, W, S = workloads.q8_inputs(1, K, N, 304)
    A = np.zeros((8, K), np.float32)
    ks = [0, 31, 32, 1000, 2049, 4096, 4099, 77]
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = gpu_q8(A, W, S, MATRIX)
    for m, k in enumerate(ks):
        ref = (W[k].astype(np.float64) * S[k // 32].astype(np.float64)).astype(np.float32)
        assert np.array_equal(C[m], ref)


def test_matrix_rows_are_independent():
    A, W, S = workloads.q8_inputs(24, 2000, 1024, 305)
    C24 = gpu_q8(A, W, S, MATRIX)
    C8 = gpu_q8(A[:8], W, S, MATRIX)
    assert np.array_equal(C24[:8].view(np.uint32), C8.view(np.uint32))


def test_matrix_row_blocks_are_independent():
    # the 64-row instance's rows equal calls on 32 rows (and on the 29 left over)
    A, W, S = workloads.q8_inputs(61, 2000, 1024, 312)
    C = gpu_q8(A, W, S, MATRIX)
    for lo, hi in ((0, 32), (32, 61)):
        part = gpu_q8(A[lo:hi], W, S, MATRIX)
        assert np.array_equal(C[lo:hi].view(np.uint32), part.view(np.uint32))
    assert_parity(A, W, S, C)


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_matrix_64_row_instance_every_split(splits):
    M, K, N = 40, 1280, 1536
    A, W, S = workloads.q8_inputs(M, K, N, (313, splits))
    assert_parity(A, W, S, gpu_q8(A, W, S, {"kind": binding.PLAN_MATRIX, "workgroups": 3 * splits}))


def test_matrix_deterministic_and_zero_rows():
    A, W, S = workloads.q8_inputs(16, 4100, 4096, 306)
    A[3] = 0
    C1 = gpu_q8(A, W, S, MATRIX)
    C2 = gpu_q8(A, W, S, MATRIX)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    assert np.all(C1[3] == 0)
    assert_parity(A, W, S, C1)


def test_matrix_power_of_two_scaling_is_exact():
    A, W, S = workloads.q8_inputs(10, 1500, 1024, 307)
    C = gpu_q8(A, W, S, MATRIX)
    for j in (-5, 4):
        f = np.float32(2.0 ** j)
        assert np.array_equal(gpu_q8(A * f, W, S, MATRIX), C * f)
        assert np.array_equal(gpu_q8(A, W, S * f, MATRIX), C * f)


def test_matrix_invalid_plans():
    A, W, S = (to_dev(x) for x in workloads.q8_inputs(16, 256, 1024, 308))
    for bad in ({"kind": 2, "vec": 8}, {"kind": 2, "m_tile": 4}, {"kind": 2, "workgroups": 3},
                {"kind": 3}, {"kind": 2, "workgroups": 2 * 9}, {"kind": 2, "waves": 4}):
        with pytest.raises(binding.Q8Error):
            binding.q8_matvec_with_plan(A, W, S, bad)
    A1, W1, S1 = (to_dev(x) for x in workloads.q8_inputs(1, 256, 1024, 309))
    with pytest.raises(binding.Q8Error):
        binding.q8_matvec_with_plan(A1, W1, S1, MATRIX)  # one row
    # one tile's split partials must stay below 2 GiB of 32-bit offsets:
    # 64 rows x 512 columns x 4 B x 16384 splits is 2 GiB
    Abig = torch.zeros((40, 16384 * 32), dtype=torch.float32, device=DEV)
    Wbig = torch.zeros((16384 * 32, 16), dtype=torch.int8, device=DEV)
    Sbig = torch.zeros((16384, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.Q8Error):
        binding.q8_matvec_with_plan(Abig, Wbig, Sbig, {"kind": binding.PLAN_MATRIX, "workgroups": 16384})
    A65, W65, S65 = (to_dev(x) for x in workloads.q8_inputs(65, 256, 1024, 314))
    with pytest.raises(binding.Q8Error):
        binding.q8_matvec_with_plan(A65, W65, S65, MATRIX)  # above 64 rows
    A2, W2, S2 = (to_dev(x) for x in workloads.q8_inputs(16, 256, 1002, 310))
    with pytest.raises(binding.Q8Error):
        binding.q8_matvec_with_plan(A2, W2, S2, MATRIX)  # N % 4 != 0: W rows not 4-byte aligned
    Wbuf = torch.empty(256 * 1024 + 16, dtype=torch.int8, device=DEV)
    W3 = Wbuf[2:2 + 256 * 1024].view(256, 1024)
    with pytest.raises(binding.Q8Error):
        binding.q8_matvec_with_plan(A, W3, S, MATRIX)  # W's address not 4-byte aligned


@pytest.mark.parametrize("M", [17, 45])
def test_matrix_canaries(M):
    K, N = 1000, 1040
    A, W, S = workloads.q8_inputs(M, K, N, (311, M))
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    buf[:pad] = 1.0
    buf[-pad:] = -2.0
    out = buf[pad:pad + M * N].view(M, N)
    binding.q8_matvec_with_plan(to_dev(A), to_dev(W), to_dev(S), MATRIX, out=out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 1.0) and np.all(host[-pad:] == -2.0)
    assert_parity(A, W, S, out.cpu().numpy())


# "Bounds": N need not fill the 512-column tiles nor be a multiple of 16.  W
# is then read in 8- or 4-byte pieces (the widest that N and W's address
# allow), and the columns past N in the last tile are not stored.
@pytest.mark.parametrize("M", [2, 4, 16, 24, 64])
@pytest.mark.parametrize("K,N", [(4100, 5000), (1000, 1000), (96, 516), (64, 4), (4100, 1028), (300, 2056)])
def test_matrix_ragged_n(M, K, N):
    A, W, S = workloads.q8_inputs(M, K, N, (330, M, K, N))
    print(f"[gemm] ragged N: M={M} K={K} N={N}", flush=True)
    assert_parity(A, W, S, gpu_q8(A, W, S, MATRIX))


def w_at_offset(W, off):
    """A device copy of W whose address is `off` bytes past a 256-byte boundary."""
    K, N = W.shape
    buf = torch.zeros(K * N + 256, dtype=torch.int8, device=DEV)
    view = buf[off:off + K * N].view(K, N)
    view.copy_(torch.from_numpy(np.ascontiguousarray(W)).to(DEV))
    assert view.data_ptr() % 16 == off % 16
    return view


# The load width changes which lanes bring in which bytes, not the sums: the
# results are bitwise the same for 16-, 8- and 4-byte loads.
@pytest.mark.parametrize("M,K,N", [(16, 4100, 4096), (64, 1000, 1536), (3, 8192, 2048), (32, 256, 512)])
def test_matrix_load_widths_agree(M, K, N):
    A, W, S = workloads.q8_inputs(M, K, N, (331, M, K, N))
    A_d, S_d = to_dev(A), to_dev(S)
    outs = []
    for off in (0, 8, 4):
        print(f"[gemm] W offset {off}: M={M} K={K} N={N}", flush=True)
        C = binding.q8_matvec_with_plan(A_d, w_at_offset(W, off), S_d, MATRIX)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy())
    assert_parity(A, W, S, outs[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
