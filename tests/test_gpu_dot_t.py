"""GPU parity of q8_dot_t against the CPU oracle: bit-exact int32 results."""

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_gemv_q8_amd import binding, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_dot_t(A, W):
    C = binding.q8_dot_t(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    return C.cpu().numpy()


def test_workload_bit_exact():
    A, W = workloads.make("dot_t_16x4096x4096", 0)
    print("[dot_t] 16x4096x4096", flush=True)
    assert np.array_equal(gpu_dot_t(A, W), oracle.dot_t(A, W))


def test_workload_every_rotated_copy():
    """Every rotated copy the bench streams (63), bit-exact."""
    n = workloads.COPIES["dot_t_16x4096x4096"]
    print(f"[dot_t] 16x4096x4096: {n} rotated copies", flush=True)
    for j in range(1, n):
        if j % 16 == 0:
            print(f"[dot_t] copy {j}", flush=True)
        A, W = workloads.make("dot_t_16x4096x4096", j)
        assert np.array_equal(gpu_dot_t(A, W), oracle.dot_t(A, W)), f"copy {j}"


@pytest.mark.parametrize("M", list(range(1, 18)) + [31, 32, 33, 64])
def test_rows_mfma_and_sdot4(M):
    for K, N in [(4096, 300), (128, 17), (4100, 64), (64, 1000)]:
        A, W = workloads.dot_t_inputs(M, K, N, (200, M, K, N))
        assert np.array_equal(gpu_dot_t(A, W), oracle.dot_t(A, W)), (M, K, N)


@pytest.mark.parametrize("K", [1, 3, 4, 5, 15, 16, 17, 63, 64, 65, 127, 128, 129, 1000, 4097])
def test_k_ragged_all_paths(K):
    for M, N in [(1, 33), (16, 40), (20, 7)]:
        A, W = workloads.dot_t_inputs(M, K, N, (201, M, K, N))
        assert np.array_equal(gpu_dot_t(A, W), oracle.dot_t(A, W)), (M, K, N)


def test_extremes_and_wraparound():
    for M in (1, 16):
        K = 131072
        A = np.full((M, K), -128, np.int8)
        W = np.full((3, K), -128, np.int8)
        W[1] = 127
        W[2, ::2] = 1
        C = gpu_dot_t(A, W)
        assert np.array_equal(C, oracle.dot_t(A, W))
        assert C[0, 0] == -(2 ** 31)


def test_misaligned_operands():
    M, K, N = 16, 256, 48
    A, W = workloads.dot_t_inputs(M, K, N, 202)
    buf = torch.zeros(M * K + 8, dtype=torch.int8, device=DEV)
    Ad = buf[1:1 + M * K].view(M, K)
    Ad.copy_(torch.from_numpy(A).to(DEV))
    C = binding.q8_dot_t(Ad, torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), oracle.dot_t(A, W))


def test_k_zero_and_empty():
    out = torch.full((2, 3), 7, dtype=torch.int32, device=DEV)
    binding.q8_dot_t(torch.zeros((2, 0), dtype=torch.int8, device=DEV),
                     torch.zeros((3, 0), dtype=torch.int8, device=DEV), out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    assert binding.q8_dot_t(torch.zeros((0, 4), dtype=torch.int8, device=DEV),
                            torch.zeros((3, 4), dtype=torch.int8, device=DEV)).shape == (0, 3)
