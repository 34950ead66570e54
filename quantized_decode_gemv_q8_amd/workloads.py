"""Seeded synthetic inputs for the Q8_0 matvec, the i8 dot_t and the dense
f32 dot / dot_t.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the library's tests/bench and the CPU oracle can consume
its arrays.  numpy ``Generator(PCG64)``; draw order is A, then W, then S.

Shapes and value ranges follow the decode-step projections the "Q8_0 matvec"
page describes (one activation row against a large i8 weight matrix with one
f32 scale per 32-row block and column).  The layer shapes stand in for
attention / MLP projections of 7B- and 70B-class models; no trained weights
are involved.  The dense f32 workloads stand in for a square f32 GEMM and for
attention scores q @ k^T (head dimension 128), with N(0,1) operands.
"""

from dataclasses import dataclass

import numpy as np

BLOCK = 32  # Q8_0 block length along K


@dataclass(frozen=True)
class Workload:
    name: str
    op: str          # "q8", "q8_fused" (siblings sharing A), "dot_t" (i8), "dot_f32" or "dot_t_f32"
    M: int
    K: int
    N: int
    a_dist: str      # "u11" (f32 U[-1,1]), "normal" (f32 N(0,1)), "i8full" (U{-128..127})
    w_dist: str      # "i8sym" (U{-127..127}) or "i8full" (U{-128..127})
    seed: tuple      # base seed; copy j uses seed + (j,) unless ``fixed_seed``
    fixed_seed: bool = False
    siblings: int = 1  # weight sets sharing A ("q8_fused")

    @property
    def KB(self):
        return (self.K + BLOCK - 1) // BLOCK

    def algorithmic_bytes(self):
        """Bytes the method must move once each (reads of A, W, S; write of C)."""
        if self.op in ("q8", "q8_fused"):
            per = self.K * self.N + 4 * self.KB * self.N + 4 * self.M * self.N
            return self.siblings * per + 4 * self.M * self.K
        if self.op in ("dot_f32", "dot_t_f32"):
            return 4 * (self.M * self.K + self.K * self.N + self.M * self.N)
        return self.M * self.K + self.N * self.K + 4 * self.M * self.N

    def algorithmic_flops(self):
        """Multiply-adds of the contraction, two flops each."""
        return 2 * self.siblings * self.M * self.N * self.K


WORKLOADS = {
    # tiny case that the exact brute force and the oracle finish in a blink
    "tiny": Workload("tiny", "q8", 1, 256, 128, "u11", "i8sym", (0,), fixed_seed=True),
    # 7B-class attention projection
    "attn4096": Workload("attn4096", "q8", 1, 4096, 4096, "normal", "i8sym", (2, 0)),
    # 70B-class MLP up-projection and its transpose (the headline shape)
    "mlp_up_8192x28672": Workload("mlp_up_8192x28672", "q8", 1, 8192, 28672, "normal", "i8sym", (3, 0)),
    "mlp_down_28672x8192": Workload("mlp_down_28672x8192", "q8", 1, 28672, 8192, "normal", "i8sym", (3, 1)),
    # a batch of 16 decode rows against the up-projection (matrix-core product)
    "batch16_8192x28672": Workload("batch16_8192x28672", "q8", 16, 8192, 28672, "normal", "i8sym", (8, 0)),
    # 64 rows: the matrix-core product's 64-row instance
    "batch64_8192x28672": Workload("batch64_8192x28672", "q8", 64, 8192, 28672, "normal", "i8sym", (9, 0)),
    # ragged batched case: 4 rows, K=4100 (last block 4 rows), N=5000
    "ragged_m4": Workload("ragged_m4", "q8", 4, 4100, 5000, "normal", "i8sym", (4, 0)),
    # sibling projections sharing one activation row: an MLP's gate and up
    # projections, and an attention block's q, k and v
    "mlp_gate_up_8192x28672": Workload("mlp_gate_up_8192x28672", "q8_fused", 1, 8192, 28672, "normal", "i8sym",
                                       (6, 0), siblings=2),
    "attn_qkv_4096": Workload("attn_qkv_4096", "q8_fused", 1, 4096, 4096, "normal", "i8sym", (7, 0), siblings=3),
    # the fixed cost of one launch of the matvec kernel: 256 workgroups that
    # each read a single 32-row block of 256 columns (M=1, K=32, N=65536)
    "launch_floor_1x32x65536": Workload("launch_floor_1x32x65536", "q8", 1, 32, 65536, "normal", "i8sym", (12, 0)),
    # integer dot_t, weights stored one output row per row
    "dot_t_16x4096x4096": Workload("dot_t_16x4096x4096", "dot_t", 16, 4096, 4096, "i8full", "i8full", (5, 0)),
    # dense f32 product (square GEMM) and attention scores q @ k^T * 1/sqrt(128)
    "dot_f32_4096": Workload("dot_f32_4096", "dot_f32", 4096, 4096, 4096, "normal", "normal", (10, 0)),
    "scores_4096x4096_d128": Workload("scores_4096x4096_d128", "dot_t_f32", 4096, 128, 4096, "normal", "normal",
                                      (11, 0)),
}


# Rotated copies per workload: enough to exceed the 256 MB Infinity Cache
# (at least 1 GiB of weights), so that a timed pass reads its weights from
# HBM.  Copy j draws from its own seed (``make(name, j)``).
COPIES = {"tiny": 1, "attn4096": 57, "mlp_up_8192x28672": 4, "mlp_down_28672x8192": 4,
          "ragged_m4": 47, "dot_t_16x4096x4096": 63, "mlp_gate_up_8192x28672": 2, "attn_qkv_4096": 19,
          "batch16_8192x28672": 4, "batch64_8192x28672": 4, "dot_f32_4096": 1, "scores_4096x4096_d128": 1,
          "launch_floor_1x32x65536": 1}


def _draw(rng, dist, shape):
    if dist == "u11":
        return rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "i8sym":
        return rng.integers(-127, 128, shape, dtype=np.int8)
    if dist == "i8full":
        return rng.integers(-128, 128, shape, dtype=np.int8)
    if dist == "scale":
        return rng.uniform(0.001, 0.02, shape).astype(np.float32)
    raise ValueError(dist)


def rng_for(seed):
    return np.random.default_rng(list(seed) if isinstance(seed, (tuple, list)) else seed)


def q8_inputs(M, K, N, seed, a_dist="normal", w_dist="i8sym"):
    """(A f32 [M,K], W i8 [K,N], S f32 [ceil(K/32),N]) drawn in that order."""
    rng = rng_for(seed)
    A = _draw(rng, a_dist, (M, K))
    W = _draw(rng, w_dist, (K, N))
    S = _draw(rng, "scale", ((K + BLOCK - 1) // BLOCK, N))
    return A, W, S


def q8_fused_inputs(M, K, N, siblings, seed, a_dist="normal", w_dist="i8sym"):
    """(A f32 [M,K], [W_g i8 [K,N]], [S_g f32 [ceil(K/32),N]]) drawn as A, W_0, S_0, W_1, S_1, ..."""
    rng = rng_for(seed)
    A = _draw(rng, a_dist, (M, K))
    Ws, Ss = [], []
    for _ in range(siblings):
        Ws.append(_draw(rng, w_dist, (K, N)))
        Ss.append(_draw(rng, "scale", ((K + BLOCK - 1) // BLOCK, N)))
    return A, Ws, Ss


def dot_t_inputs(M, K, N, seed, dist="i8full"):
    """(A i8 [M,K], W i8 [N,K]) drawn in that order."""
    rng = rng_for(seed)
    A = _draw(rng, dist, (M, K))
    W = _draw(rng, dist, (N, K))
    return A, W


def dense_inputs(M, K, N, seed, transposed=False, dist="normal"):
    """(A f32 [M,K], B f32 [K,N], or [N,K] when transposed) drawn in that order."""
    rng = rng_for(seed)
    A = _draw(rng, dist, (M, K))
    B = _draw(rng, dist, (N, K) if transposed else (K, N))
    return A, B


# ---------------------------------------------------------------- device draws
# Inputs of several GiB (the cases at the library's 32-bit offset limits) are
# drawn on the device with a seeded torch generator, in the distributions of
# _draw; a host draw and copy of that size would dominate the test.  The tests
# read back only the slices they check against the oracle.

def device_generator(seed, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def device_draw(gen, dist, shape, device):
    import torch
    if dist == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if dist == "u11":
        return torch.empty(shape, device=device, dtype=torch.float32).uniform_(-1.0, 1.0, generator=gen)
    if dist == "i8sym":
        return torch.randint(-127, 128, shape, generator=gen, device=device, dtype=torch.int8)
    if dist == "i8full":
        return torch.randint(-128, 128, shape, generator=gen, device=device, dtype=torch.int8)
    if dist == "scale":
        return torch.empty(shape, device=device, dtype=torch.float32).uniform_(0.001, 0.02, generator=gen)
    raise ValueError(dist)


def device_q8_inputs(M, K, N, seed, device):
    """q8_inputs' shapes and distributions, drawn on `device` (A, W, S in that order)."""
    g = device_generator(seed, device)
    A = device_draw(g, "normal", (M, K), device)
    W = device_draw(g, "i8sym", (K, N), device)
    S = device_draw(g, "scale", ((K + BLOCK - 1) // BLOCK, N), device)
    return A, W, S


def device_dot_t_inputs(M, K, N, seed, device):
    """dot_t_inputs' shapes and distribution, drawn on `device` (A, W)."""
    g = device_generator(seed, device)
    return device_draw(g, "i8full", (M, K), device), device_draw(g, "i8full", (N, K), device)


def device_dense_inputs(M, K, N, seed, transposed, device):
    """dense_inputs' shapes and distribution, drawn on `device` (A, B)."""
    g = device_generator(seed, device)
    A = device_draw(g, "normal", (M, K), device)
    return A, device_draw(g, "normal", (N, K) if transposed else (K, N), device)


def make(name, copy=0):
    """Inputs of a named workload; copy j of a rotated set uses its own seed."""
    wl = WORKLOADS[name]
    seed = wl.seed if wl.fixed_seed else tuple(wl.seed) + (copy,)
    if wl.op == "q8":
        if wl.fixed_seed:
            seed = wl.seed[0]
        return q8_inputs(wl.M, wl.K, wl.N, seed, wl.a_dist, wl.w_dist)
    if wl.op == "q8_fused":
        return q8_fused_inputs(wl.M, wl.K, wl.N, wl.siblings, seed, wl.a_dist, wl.w_dist)
    if wl.op in ("dot_f32", "dot_t_f32"):
        return dense_inputs(wl.M, wl.K, wl.N, seed, wl.op == "dot_t_f32", wl.a_dist)
    return dot_t_inputs(wl.M, wl.K, wl.N, seed, wl.a_dist)
