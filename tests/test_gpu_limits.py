"""GPU parity at the size limits of the C ABI.

The library indexes with 32-bit offsets: q8_matvec and q8_dot_t accept K*N
(and M*K, M*N) below 2^31 elements, the matrix-core path also needs A's
bytes below 2^31, and the dense products keep their byte offsets, with a
tile of overhang, below 2^32.  These cases sit just under those limits, with
ragged K and N where the limit allows, so that the largest row and column
offsets are the ones a wrong width would wrap.  The operands (up to 4 GiB)
are drawn on the device with a seeded generator; the oracle checks the
first, last and randomly chosen columns or rows of each result, read back
with their inputs, to the same bar as the other parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_gemv_q8_amd import binding, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-5
LIMIT = 1 << 31


def sample(n, seed, k=64):
    """Sorted distinct indices: the first k, the last k and k drawn at random."""
    rng = np.random.default_rng(seed)
    idx = set(range(min(k, n))) | set(range(max(0, n - k), n)) | set(rng.integers(0, n, k).tolist())
    return sorted(idx)


def pick(t, dim, idx):
    return t.index_select(dim, torch.tensor(idx, device=t.device)).cpu().numpy()


def release():
    torch.cuda.synchronize()
    binding.q8_release()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,K,N", [
    (1, 65536, 32752),    # the stream at 8-byte lanes; the last tile ragged
    (16, 65536, 32752),   # the matrix cores
    (1, 65535, 32767),    # ragged K (the last block has 31 rows) and odd N (1-byte lanes)
])
def test_q8_matvec_at_the_offset_limit(M, K, N):
    assert LIMIT - (1 << 21) < K * N < LIMIT
    A, W, S = workloads.device_q8_inputs(M, K, N, 600 + M, DEV)
    plan = binding.q8_matvec_choose_plan(M, K, N)
    print(f"[limits] q8_matvec M={M} K={K} N={N} plan={plan}", flush=True)
    C = binding.q8_matvec(A, W, S)
    torch.cuda.synchronize()
    cols = sample(N, 601)
    Ah, Wc, Sc = A.cpu().numpy(), pick(W, 1, cols), pick(S, 1, cols)
    Cc = pick(C, 1, cols)
    del A, W, S, C
    release()
    err = oracle.normalised_error(Cc, oracle.q8_matvec(Ah, Wc, Sc), oracle.q8_normaliser(Ah, Wc, Sc))
    assert err <= TOL, f"normalised error {err:.3e}"


def test_matrix_path_refuses_a_past_its_offsets():
    """4*M*K = 2^31: an explicit matrix plan is refused; the automatic plan
    takes the stream, whose A offsets are 64-bit."""
    M, K, N = 64, 1 << 23, 16
    A, W, S = workloads.device_q8_inputs(M, K, N, 602, DEV)
    print(f"[limits] q8_matvec M={M} K={K} N={N}: matrix plan refused, automatic plan", flush=True)
    with pytest.raises(binding.Q8Error) as e:
        binding.q8_matvec_with_plan(A, W, S, {"kind": binding.PLAN_MATRIX})
    assert e.value.status == binding.Q8_ERR_TOO_LARGE
    assert binding.q8_matvec_choose_plan(M, K, N)["kind"] == binding.PLAN_STREAM
    C = binding.q8_matvec(A, W, S)
    torch.cuda.synchronize()
    rows, cols = [0, 1, 31, 62, 63], [0, 7, 15]
    Ar, Wc, Sc = pick(A, 0, rows), pick(W, 1, cols), pick(S, 1, cols)
    Cc = pick(C, 1, cols)[rows]
    del A, W, S, C
    release()
    err = oracle.normalised_error(Cc, oracle.q8_matvec(Ar, Wc, Sc), oracle.q8_normaliser(Ar, Wc, Sc))
    assert err <= TOL, f"normalised error {err:.3e}"


def test_dot_t_at_the_offset_limit():
    M, K, N = 16, 65536, 32767
    assert LIMIT - (1 << 21) < N * K < LIMIT
    A, W = workloads.device_dot_t_inputs(M, K, N, 603, DEV)
    print(f"[limits] q8_dot_t M={M} K={K} N={N}", flush=True)
    C = binding.q8_dot_t(A, W)
    torch.cuda.synchronize()
    rows = sample(N, 604)
    Ah, Wr, Cc = A.cpu().numpy(), pick(W, 0, rows), pick(C, 1, rows)
    del A, W, C
    release()
    assert np.array_equal(Cc, oracle.dot_t(Ah, Wr))


@pytest.mark.parametrize("transposed", [False, True])
def test_dense_at_the_byte_limit(transposed):
    """The large operand is A for dot ([262015, 4064]) and B for dot_t
    ([262015, 4064]): with a tile of overhang its bytes reach 2^32 - 16 KiB."""
    K, big, small = 4064, 262015, 64
    assert (big + 128) * (K + 32) < (1 << 30) <= (big + 129) * (K + 32)
    M, N = (small, big) if transposed else (big, small)
    A, B = workloads.device_dense_inputs(M, K, N, 605, transposed, DEV)
    alpha = 1.0 / np.sqrt(K) if transposed else 1.0
    fn = binding.q8_dot_t_f32 if transposed else binding.q8_dot_f32
    print(f"[limits] {fn.__name__} M={M} K={K} N={N}", flush=True)
    C = fn(A, B, alpha=alpha)
    torch.cuda.synchronize()
    idx = sample(big, 606)
    if transposed:  # sampled rows of B: columns of C
        Ah, Bs, Cs = A.cpu().numpy(), pick(B, 0, idx), pick(C, 1, idx)
        ref = oracle.dense_fused(Ah, Bs, True, alpha)
        D = oracle.dense_fused_normaliser(Ah, Bs, True, alpha)
    else:           # sampled rows of A: rows of C
        As, Bh, Cs = pick(A, 0, idx), B.cpu().numpy(), pick(C, 0, idx)
        ref = oracle.dense_fused(As, Bh, False, alpha)
        D = oracle.dense_fused_normaliser(As, Bh, False, alpha)
    del A, B, C
    release()
    err = oracle.normalised_error(Cs, ref, D)
    assert err <= TOL, f"normalised error {err:.3e}"


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def test_tall_a_runs_in_row_slabs():
    """600 000 rows in chunks of 8 are 75 000 row chunks, more than the grid's
    second dimension holds (65 535): the library launches slabs of rows in
    order.  Two siblings and row factors check that every slab offsets A,
    each C and corr alike."""
    M, K, N, alpha = 600_000, 64, 64, 0.75
    assert binding.q8_matvec_choose_plan(M, K, N)["m_tile"] == 8
    A, Ws, Ss = workloads.q8_fused_inputs(M, K, N, 2, (607, 0))
    rng = np.random.default_rng(608)
    corr = rng.standard_normal(M).astype(np.float32)
    C_olds = [rng.standard_normal((M, N)).astype(np.float32) for _ in range(2)]
    print(f"[limits] q8_matvec_fused M={M} K={K} N={N} siblings=2 with corr", flush=True)
    outs = [to_dev(C) for C in C_olds]
    binding.q8_matvec_fused(to_dev(A), [to_dev(W) for W in Ws], [to_dev(S) for S in Ss], outs=outs,
                            alpha=alpha, corr=to_dev(corr))
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    del outs
    release()
    refs = oracle.q8_matvec_fused(A, list(zip(Ws, Ss)), alpha, corr, C_olds)
    for g in range(2):
        D = oracle.q8_fused_normaliser(A, Ws[g], Ss[g], alpha, corr, C_olds[g])
        err = oracle.normalised_error(got[g], refs[g], D)
        assert err <= TOL, f"sibling {g}: normalised error {err:.3e}"


@pytest.mark.parametrize("K", [16, 20])  # the i8 matrix cores; sdot4 with 16 rows per grid row
def test_dot_t_tall_a_runs_in_row_slabs(K):
    M, N = 1_100_000, 16
    A, W = workloads.dot_t_inputs(M, K, N, (609, K))
    print(f"[limits] q8_dot_t M={M} K={K} N={N}", flush=True)
    C = binding.q8_dot_t(to_dev(A), to_dev(W))
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    del C
    release()
    assert np.array_equal(got, oracle.dot_t(A, W))
