"""GPU parity of q8_matvec against the CPU oracle (called through the C ABI).

Bar: max over outputs of |C_gpu - C_oracle| / D <= 1e-5, where D is the sum of
|A W S| terms (the oracle's normaliser); D == 0 requires an exact zero.
"""

import math
import os

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


def gpu_q8(A, W, S, plan=None, out=None, stream=None):
    A_d, W_d, S_d = to_dev(A), to_dev(W), to_dev(S)
    if plan is None:
        C = binding.q8_matvec(A_d, W_d, S_d, out=out, stream=stream)
    else:
        C = binding.q8_matvec_with_plan(A_d, W_d, S_d, plan, out=out, stream=stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def assert_parity(A, W, S, C):
    ref = oracle.q8_matvec(A, W, S)
    D = oracle.q8_normaliser(A, W, S)
    err = oracle.normalised_error(C, ref, D)
    assert err <= TOL, f"normalised error {err:.3e} > {TOL}"
    return err


def rand_q8(M, K, N, seed):
    return workloads.q8_inputs(M, K, N, seed)


# ------------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name", ["tiny", "attn4096", "ragged_m4", "mlp_up_8192x28672", "mlp_down_28672x8192"])
def test_workload_parity(name):
    A, W, S = workloads.make(name, 0)
    print(f"[q8] workload {name} M={A.shape[0]} K={A.shape[1]} N={W.shape[1]}", flush=True)
    C = gpu_q8(A, W, S)
    assert np.isfinite(C).all()
    assert_parity(A, W, S, C)


@pytest.mark.parametrize("name", ["attn4096", "ragged_m4"])
def test_workload_rotated_copies(name):
    """Every rotated copy the bench streams (57 and 47), each against the oracle."""
    n = workloads.COPIES[name]
    assert n > 1
    print(f"[q8] workload {name}: {n} rotated copies", flush=True)
    for j in range(1, n):
        if j % 16 == 0:
            print(f"[q8] {name}: copy {j}", flush=True)
        A, W, S = workloads.make(name, j)
        assert_parity(A, W, S, gpu_q8(A, W, S))


# ------------------------------------------------------------------ masking sweeps

@pytest.mark.parametrize("K", [1, 31, 32, 33, 63, 64, 65, 100, 4100])
def test_k_remainder(K):
    for M, N in [(1, 256), (3, 1025), (4, 5000)]:
        A, W, S = rand_q8(M, K, N, (100, M, K, N))
        assert_parity(A, W, S, gpu_q8(A, W, S))


@pytest.mark.parametrize("N", [1, 7, 8, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 5000])
def test_n_ragged(N):
    for M, K in [(1, 96), (2, 300), (5, 64)]:
        A, W, S = rand_q8(M, K, N, (101, M, K, N))
        assert_parity(A, W, S, gpu_q8(A, W, S))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 9, 16, 17])
def test_rows(M):
    A, W, S = rand_q8(M, 1000, 777, (102, M))
    assert_parity(A, W, S, gpu_q8(A, W, S))


# ------------------------------------------------------------------ every kernel instance

PLANS = [(v, mt) for v in (16, 8, 4, 2, 1) for mt in (1, 2, 4, 8) if v * mt <= 32]


def units_of(M, K, N, vec):
    return math.ceil(N / (64 * vec)) * math.ceil(math.ceil(K / 32) / 4)


@pytest.mark.parametrize("vec,m_tile", PLANS)
def test_every_instance(vec, m_tile):
    M, K, N = 5, 3000, 2048  # KB = 94 (24-row remainder), 24 groups; two m passes at m_tile < 5
    A, W, S = rand_q8(M, K, N, (103, vec, m_tile))
    units = units_of(M, K, N, vec)
    cap = 16 // m_tile
    ran = 0
    for n_wg in sorted({1, 2, 3, 5, 7, 23, 24, 25, units // 2, units - 1, units, math.ceil(units / cap)}):
        if not 1 <= n_wg <= units or math.ceil(units / n_wg) > cap:
            continue
        try:
            C = gpu_q8(A, W, S, plan={"vec": vec, "m_tile": m_tile, "workgroups": n_wg})
        except binding.Q8Error as e:
            # long runs over many tiles can exceed the LDS budget: rejected up front
            assert e.status == binding.Q8_ERR_INVALID
            continue
        assert_parity(A, W, S, C)
        ran += 1
    assert ran >= 3


def test_invalid_plans_are_rejected():
    A, W, S = (to_dev(x) for x in rand_q8(1, 64, 100, 104))
    # N=100 allows vec 4 at most; K=64 has 2 blocks (one group), 2 column tiles at vec 4
    for bad in ({"vec": 16}, {"vec": 3}, {"m_tile": 3}, {"vec": 4, "m_tile": 16}, {"workgroups": 3},
                {"waves": 8}, {"workgroups": -1}):
        with pytest.raises(binding.Q8Error):
            binding.q8_matvec_with_plan(A, W, S, bad)


# ------------------------------------------------------------------ guards and edge cases

def test_outputs_that_overlap_inputs_are_refused():
    M, K, N = 2, 64, 32
    A, W, S = (to_dev(x) for x in rand_q8(M, K, N, 106))
    buf = torch.zeros(M * K + M * N, dtype=torch.float32, device=DEV)
    buf[:M * K].copy_(A.flatten())
    A_in = buf[:M * K].view(M, K)
    with pytest.raises(ValueError, match="overlaps A"):
        binding.q8_matvec(A_in, W, S, out=buf[M * K - 1:M * K - 1 + M * N].view(M, N))
    binding.q8_matvec(A_in, W, S, out=buf[M * K:].view(M, N))  # adjacent, not overlapping
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="overlaps outs"):
        binding.q8_matvec_fused(A, [W, W], [S, S], outs=[C, C])
    torch.cuda.synchronize()


def test_canaries_and_full_overwrite():
    M, K, N = 3, 4100, 5000
    A, W, S = rand_q8(M, K, N, 105)
    pad = 1024
    buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    buf[:pad] = 12345.0
    buf[-pad:] = -6789.0
    out = buf[pad:pad + M * N].view(M, N)
    C = gpu_q8(A, W, S, out=out)
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 12345.0) and np.all(host[-pad:] == -6789.0)
    assert np.isfinite(C).all()
    assert_parity(A, W, S, C)


def test_k_zero_writes_zeros():
    M, N = 2, 300
    out = torch.full((M, N), float("nan"), device=DEV)
    A = torch.zeros((M, 0), dtype=torch.float32, device=DEV)
    W = torch.zeros((0, N), dtype=torch.int8, device=DEV)
    S = torch.zeros((0, N), dtype=torch.float32, device=DEV)
    binding.q8_matvec(A, W, S, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_empty_outputs():
    A = torch.zeros((0, 64), dtype=torch.float32, device=DEV)
    W = torch.zeros((64, 5), dtype=torch.int8, device=DEV)
    S = torch.zeros((2, 5), dtype=torch.float32, device=DEV)
    assert binding.q8_matvec(A, W, S).shape == (0, 5)


def test_zero_rows_are_exact_zero():
    A, W, S = rand_q8(3, 500, 300, 106)
    A[1] = 0
    S[:, 7] = 0
    C = gpu_q8(A, W, S)
    assert np.all(C[1] == 0) and np.all(C[:, 7] == 0)
    assert_parity(A, W, S, C)


def test_misaligned_inputs_pick_narrow_loads():
    M, K, N = 2, 200, 1024
    A, W, S = rand_q8(M, K, N, 107)
    for w_off, s_off in [(1, 0), (2, 0), (4, 0), (0, 1), (0, 2), (3, 3)]:
        wbuf = torch.zeros(K * N + 16, dtype=torch.int8, device=DEV)
        sbuf = torch.zeros(S.size + 16, dtype=torch.float32, device=DEV)
        Wd = wbuf[w_off:w_off + K * N].view(K, N)
        Sd = sbuf[s_off:s_off + S.size].view(S.shape)
        Wd.copy_(to_dev(W))
        Sd.copy_(to_dev(S))
        C = binding.q8_matvec(to_dev(A), Wd, Sd)
        torch.cuda.synchronize()
        assert_parity(A, W, S, C.cpu().numpy())


def test_extreme_values():
    rng = np.random.default_rng(108)
    M, K, N = 2, 300, 512
    A = (rng.standard_normal((M, K)) * 2.0 ** rng.integers(-20, 20, (M, K))).astype(np.float32)
    W = rng.choice(np.array([-128, -127, 0, 127], np.int8), (K, N))
    S = (rng.uniform(-1, 1, (math.ceil(K / 32), N)) * 2.0 ** rng.integers(-10, 10, (math.ceil(K / 32), N))).astype(np.float32)
    assert_parity(A, W, S, gpu_q8(A, W, S))


# ------------------------------------------------------------------ bitwise invariants

def test_deterministic():
    A, W, S = workloads.make("attn4096", 0)
    C1 = gpu_q8(A, W, S)
    C2 = gpu_q8(A, W, S)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_one_hot_is_exact():
    K, N = 4100, 5000
    _, W, S = rand_q8(1, K, N, 109)
    for k in (0, 31, 32, 2049, 4099):
        A = np.zeros((1, K), np.float32)
        A[0, k] = 1.0
        C = gpu_q8(A, W, S)
        ref = (W[k].astype(np.float64) * S[k // 32].astype(np.float64)).astype(np.float32)
        assert np.array_equal(C[0], ref)


def test_power_of_two_scaling_is_exact():
    A, W, S = rand_q8(2, 2000, 1500, 110)
    C = gpu_q8(A, W, S)
    for j in (-8, -3, 5, 8):
        f = np.float32(2.0 ** j)
        assert np.array_equal(gpu_q8(A * f, W, S), C * f)
        assert np.array_equal(gpu_q8(A, W, S * f), C * f)


def test_rows_are_independent():
    A, W, S = rand_q8(4, 4100, 5000, 111)
    plan = {"vec": 8, "workgroups": 165}  # 330 units, 2 per workgroup: fits m_tile 4 and 1
    C = gpu_q8(A, W, S, plan=dict(plan, m_tile=4))
    for m in range(4):
        Cm = gpu_q8(A[m:m + 1], W, S, plan=dict(plan, m_tile=1))
        assert np.array_equal(Cm[0], C[m])


def test_columns_are_independent():
    A, W, S = rand_q8(1, 1000, 1024, 112)
    C = gpu_q8(A, W, S)
    W2 = W.copy()
    W2[:, 500] = -W2[:, 500]
    C2 = gpu_q8(A, W2, S)
    mask = np.ones(1024, bool)
    mask[500] = False
    assert np.array_equal(C[0, mask], C2[0, mask])


# ------------------------------------------------------------------ streams and workspace

def test_non_default_stream():
    A, W, S = rand_q8(1, 8192, 4096, 113)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        A_d, W_d, S_d = to_dev(A), to_dev(W), to_dev(S)
        C = binding.q8_matvec(A_d, W_d, S_d, stream=s)
    s.synchronize()
    assert_parity(A, W, S, C.cpu().numpy())


@pytest.mark.parametrize("M,K,N,contributors", [(1, 1 << 20, 64, 512), (3, 1 << 20, 64, 2048)])
def test_long_k_many_contributors(M, K, N, contributors):
    """A long K over one column tile: 512 (one row) and 2048 (three rows, four
    units per workgroup) workgroups share the tile, so the combine sums 64
    and 256 groups of eight partials through its cascade."""
    plan = {"kind": binding.PLAN_STREAM}
    A, W, S = rand_q8(M, K, N, (140, M, K, N))
    print(f"[q8] long K M={M} K={K} N={N} stream, {contributors} contributors", flush=True)
    C = gpu_q8(A, W, S, plan)
    assert_parity(A, W, S, C)
    # The cascade's order depends only on the contributor count: repeated
    # calls agree bitwise, and scaling A by a power of two scales C exactly.
    assert np.array_equal(gpu_q8(A, W, S, plan), C)
    assert np.array_equal(gpu_q8(np.float32(0.25) * A, W, S, plan), np.float32(0.25) * C)


@pytest.mark.parametrize("vec", [8, 16])
@pytest.mark.parametrize("contributors", [2, 3, 4, 5, 8])
def test_few_contributors(vec, contributors):
    """Tiles shared by 2-8 workgroups at the wide lanes: up to four
    contributors the last arrival adds the partials as one pairwise tree, more
    go through the general combine.  Parity, zero columns come out +0 exactly,
    repeated calls agree bitwise and a power-of-two scale of A scales C
    exactly."""
    M, K, N = 2, 4096, 2048
    A, W, S = rand_q8(M, K, N, (141, vec, contributors))
    S[:, 5] = 0  # a column whose every partial is zero
    tiles = N // (64 * vec)
    plan = {"vec": vec, "m_tile": 1, "workgroups": tiles * contributors, "kind": binding.PLAN_STREAM}
    print(f"[q8] few contributors vec={vec} contributors={contributors}", flush=True)
    C = gpu_q8(A, W, S, plan)
    assert_parity(A, W, S, C)
    assert np.all(C[:, 5].view(np.uint32) == 0)
    assert np.array_equal(gpu_q8(A, W, S, plan).view(np.uint32), C.view(np.uint32))
    C4 = gpu_q8(np.float32(4.0) * A, W, S, plan)
    assert np.array_equal(C4.view(np.uint32), (np.float32(4.0) * C).view(np.uint32))


def _with_xcd_mode(mode, fn):
    old = os.environ.get("Q8_XCD_LOCAL")
    if mode is None:
        os.environ.pop("Q8_XCD_LOCAL", None)
    else:
        os.environ["Q8_XCD_LOCAL"] = mode
    try:
        return fn()
    finally:
        if old is None:
            os.environ.pop("Q8_XCD_LOCAL", None)
        else:
            os.environ["Q8_XCD_LOCAL"] = old


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (2, 8192, 8192), (1, 28672, 4096),
                                   (16, 8192, 4096), (48, 4096, 4096), (8, 4096, 8192)])
def test_xcd_local_combine_is_bitwise_the_same(M, K, N, capfd):
    """Tiles whose runs all sit on one XCD keep their split-K partials in that
    XCD's L2; the sums are the same bit for bit as with device-coherent
    partials (same partials, same order)."""
    A, W, S = rand_q8(M, K, N, (142, M, K, N))
    os.environ["Q8_LOG"] = "debug"
    try:
        C_local = _with_xcd_mode(None, lambda: gpu_q8(A, W, S))
        C_dev = _with_xcd_mode("0", lambda: gpu_q8(A, W, S))
    finally:
        os.environ.pop("Q8_LOG", None)
    err = capfd.readouterr().err
    print(f"[q8] xcd-local M={M} K={K} N={N}", flush=True)
    assert "kept in the XCD L2" in err, err
    assert_parity(A, W, S, C_local)
    assert np.array_equal(C_local.view(np.uint32), C_dev.view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (16, 8192, 4096)])
def test_xcd_local_stray_contributors_give_nan(M, K, N):
    """If a tile's contributors report different XCDs, the tile's outputs are
    NaN (its partials may not be readable from one L2); the counters are
    re-armed, so the next call is correct.  Stream path and matrix cores."""
    A, W, S = rand_q8(M, K, N, (143, M))
    print(f"[q8] xcd-local stray contributors M={M} K={K} N={N}", flush=True)
    C = _with_xcd_mode("stray", lambda: gpu_q8(A, W, S))
    assert np.all(np.isnan(C))
    assert_parity(A, W, S, gpu_q8(A, W, S))


def test_many_counters():
    # 8 row chunks x 128 column tiles: 1024 split-K counters, each on a line of
    # its own, far more than the smallest counter allocation
    M, K, N = 8, 2048, 8192
    A, W, S = rand_q8(M, K, N, 116)
    plan = {"vec": 1, "m_tile": 1, "workgroups": 512}
    C = gpu_q8(A, W, S, plan=plan)
    assert_parity(A, W, S, C)
    again = gpu_q8(A, W, S, plan=plan)  # the counters were left at zero
    assert np.array_equal(C.view(np.uint32), again.view(np.uint32))


def test_workspace_grows_and_release():
    small = rand_q8(1, 640, 256, 114)
    big = rand_q8(4, 8192, 8192, 115)
    assert_parity(*small, gpu_q8(*small, plan={"workgroups": 4}))
    assert_parity(*big, gpu_q8(*big, plan={"workgroups": 512}))
    assert_parity(*small, gpu_q8(*small, plan={"workgroups": 5}))
    binding.q8_release()
    assert_parity(*big, gpu_q8(*big))
