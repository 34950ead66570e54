"""CPU oracle for the Q8_0 matvec, the i8 ``dot_t`` product and the dense f32
``dot`` / ``dot_t`` contractions.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
library (``quantized_decode_gemv_q8_amd``) never imports it, and this package
imports nothing from the library: the two share no code.  The only thing both
sides consume is the seeded input generator module
(``quantized_decode_gemv_q8_amd.workloads``), which draws random numbers and
holds none of the method's arithmetic.

Sources (Phobos documentation pages):
  * "Q8_0 matvec" (docs/examples/q8-matvec), section "The tensors": the
    layouts of A, W, S, C and the definition
    C[0,n] = sum_k A[0,k] * W[k,n] * S[k/32, n].
  * same page, section "Factoring out the scale": the per-block identity
    sum_{k in b} A[k] W[k,n] S[b,n] = S[b,n] * sum_{k in b} A[k] W[k,n].
  * same page, section "Bounds": N need not be a multiple of the tile, and
    when K is not a multiple of 32 the last block is short (its missing rows
    are masked out).
  * "dot and tensor cores" (docs/language/dot-and-tensor-cores), the table of
    built-ins: dot_t(a, b) with a [M,K], b [N,K] computes a @ b^T; section
    "Hardware paths": i8 operands accumulate in i32, f32 operands in f32;
    section "The k loop": dot(a, b) with a [M,K], b [K,N] is a @ b,
    accumulated over panels of K; section "The fused epilogue": the
    elementwise statement that consumes a product (a scale, or a rescale of
    the existing value followed by an add) runs as the product is written.

Every function is pinned by tests in ``tests/test_oracle.py`` against exact
rational arithmetic, closed forms, library special cases and hand-derived
fixtures; none is "parity unpinned".
"""

from .q8_oracle import (  # noqa: F401
    BLK,
    num_blocks,
    q8_matvec_factored,
    q8_matvec_per_weight,
    q8_normaliser,
    q8_matvec,
    q8_epilogue,
    q8_matvec_fused,
    q8_fused_normaliser,
    normalised_error,
    dot_t,
    wrap_i32,
)
from .dense import (  # noqa: F401
    dot_f32,
    dot_t_f32,
    dense_normaliser,
    dense_fused,
    dense_fused_normaliser,
)
from .exact import q8_matvec_exact, q8_epilogue_exact, dot_t_loops, dense_exact  # noqa: F401
