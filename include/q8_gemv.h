/*
 * q8_gemv.h -- C ABI of the MI355X (gfx950) Q8_0 matvec and i8 dot_t library.
 *
 * Operations (Phobos documentation pages):
 *   q8_matvec  "Q8_0 matvec" (docs/examples/q8-matvec), section "The tensors":
 *              C[m,n] = sum_k A[m,k] * W[k,n] * S[k/32, n], with i8 weights,
 *              one f32 scale per block of 32 rows along K and per column.
 *              Section "Factoring out the scale": the scale is applied once
 *              per block and column to the block's unscaled partial.
 *              Section "Bounds": N and K need not be multiples of any tile;
 *              the ragged column tile and the K remainder block are masked.
 *   q8_dot_t   "dot and tensor cores" (docs/language/dot-and-tensor-cores),
 *              table of built-ins and section "Hardware paths":
 *              C[m,n] = sum_k A[m,k] * W[n,k], i8 operands, i32 result.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (memory of the current HIP
 *     device) to dense row-major arrays; there are no leading-dimension
 *     arguments.  The caller owns them; the library only reads the inputs
 *     and overwrites the output.  It reads C only through an epilogue with
 *     row factors (corr != NULL, below).  C must not alias an input.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous on that stream: a status of Q8_OK means the work
 *     was enqueued; faults surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued.  No
 *     C++ exception crosses this boundary.
 *   - Sizes: every extent must be >= 0.  M == 0 or N == 0 is a no-op.  The
 *     library uses 32-bit element offsets, so K*N, M*K and M*N must each be
 *     below 2^31 (otherwise Q8_ERR_TOO_LARGE).
 *   - Thread safety: concurrent calls are safe on distinct streams.  Host
 *     threads that share one stream must serialise their calls.
 *   - Workspace: the split-K workspace (partial sums and arrival counters)
 *     is owned by the library, one per (device, stream).  It is allocated by
 *     the first call that needs it on that stream and grown by a later call
 *     that needs more; buffers it grows out of stay allocated (a graph
 *     captured earlier may still use them) until q8_release() frees them
 *     all.  Allocation cannot be recorded into a graph, so a call made while
 *     its stream is being captured and that would have to allocate or grow
 *     the workspace returns Q8_ERR_INVALID and enqueues nothing: make one
 *     eager call of the same (or a larger) shape on that stream first.
 *     Captured calls replay correctly: their arrival counters return to zero
 *     inside every launch, and no call records a memset.
 *   - XCD placement: when a matvec plan cuts every column tile into whole
 *     K runs and the tiles and workgroups are multiples of 8, the library
 *     places all runs of a tile on one XCD (the dispatcher deals workgroups
 *     to the eight XCDs in turn) and keeps the tile's split-K partials in
 *     that XCD's L2.  The first such call on a device, unless its stream is
 *     being captured, first runs a small probe kernel on the stream and
 *     waits for it (once per device and process) to confirm that placement;
 *     without it the partials go through the device's coherence point as for
 *     other plans.  If the contributors of a tile are ever found on
 *     different XCDs, that tile's outputs are written as NaN, never as a
 *     wrong sum.  The environment variable Q8_XCD_LOCAL=0 turns this off;
 *     results are bitwise the same either way.
 */
#ifndef Q8_GEMV_H
#define Q8_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q8_status {
  Q8_OK = 0,
  Q8_ERR_INVALID = 1,            /* negative extent, null pointer with a non-zero extent, bad plan */
  Q8_ERR_TOO_LARGE = 2,          /* an offset would not fit the library's 32-bit indexing */
  Q8_ERR_UNSUPPORTED_DEVICE = 3, /* the current device is not gfx950 */
  Q8_ERR_HIP = 4                 /* a HIP call failed; see q8_last_hip_error() */
} q8_status;

/* Q8_0 block length along K ("The tensors": row b of S scales rows 32b..32b+31). */
#define Q8_BLOCK 32

/*
 * q8_matvec -- C = A (x) dequant(W, S).
 *   A  f32 [M, K]            activations, row-major
 *   W  i8  [K, N]            quantized weights, one column per output
 *   S  f32 [ceil(K/32), N]   scales; row b scales rows 32b .. min(32b+32, K)
 *   C  f32 [M, N]            output, overwritten (K == 0 writes zeros)
 * Errors: Q8_ERR_INVALID, Q8_ERR_TOO_LARGE, Q8_ERR_UNSUPPORTED_DEVICE,
 * Q8_ERR_HIP.  Deterministic: the same inputs give bitwise-equal outputs.
 */
q8_status q8_matvec(const float *A, const int8_t *W, const float *S, float *C,
                    int64_t M, int64_t K, int64_t N, void *stream);

/*
 * q8_matvec_noalloc -- q8_matvec that allocates nothing, for callers that
 * cannot call hipMalloc (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, plan choice, kernels
 * and results (bitwise) as q8_matvec.  Instead of the library's workspace it
 * uses a fixed scratch array that every device the library runs on holds for
 * the life of the process: 32 MiB of split-K partial sums and 64 KiB of
 * arrival counters.  The counters are cleared once per device, on that
 * device's first call (a fill kernel on `stream`), and every launch leaves
 * them at zero again.  A call whose plan needs more partial space returns
 * Q8_ERR_TOO_LARGE and enqueues nothing (for example the matrix-core product
 * of 33..64 rows at N much above 28672); q8_matvec has no such limit.
 * All calls on one device share the scratch array: calls that overlap in
 * time on one device (on different streams, or concurrently from several
 * threads) race and give wrong results; serialise them.
 * Errors: as q8_matvec, plus Q8_ERR_TOO_LARGE for plans beyond the scratch.
 */
q8_status q8_matvec_noalloc(const float *A, const int8_t *W, const float *S, float *C,
                            int64_t M, int64_t K, int64_t N, void *stream);

/*
 * Launch plan of q8_matvec.  Every field 0 means "choose automatically".
 *   kind    Q8_PLAN_STREAM or Q8_PLAN_MATRIX (below); 0 picks one from the
 *           shape: the matrix cores, when allowed, above 16 rows; at 9..16
 *           rows when their automatic plan fills at least a quarter of the
 *           device, at 5..8 rows three eighths; at 3-4 rows when it fills
 *           half and K * N reaches 2^25; at 2 rows when it fills half and
 *           K * N reaches 2^27.
 * For Q8_PLAN_STREAM, the per-row FMA stream:
 *   vec     columns (= bytes of W) each lane loads per row: 16, 8, 4, 2 or 1.
 *           N must be a multiple of vec, W 'vec'-byte aligned and S
 *           min(16, 4*vec)-byte aligned.
 *   m_tile  activation rows per pass: 1, 2, 4 or 8, with m_tile*vec <= 32.
 *   workgroups  workgroups per pass over W.  W is cut into column tiles of
 *           64*vec columns and groups of four 32-row blocks along K; the
 *           (tile, group) units are dealt to the workgroups in contiguous runs
 *           of equal length (within one), at most 16/m_tile units each.  A
 *           tile shared by several workgroups is combined in K order.
 *   waves   waves per workgroup; 4 is the only value supported.
 * For Q8_PLAN_MATRIX, the matrix-core product of 2..64 rows ("dot and tensor
 * cores", "Hardware paths"; A is split into three bf16 parts so that the
 * result keeps f32 accuracy; one pass over W serves all rows): it needs
 * N % 4 == 0, 4-byte aligned W, 16-byte aligned S and 4*M*K < 2^31 (W is
 * read in 16-, 8- or 4-byte pieces, the widest that N and W's address both
 * allow, so a ragged last column tile is masked, "Bounds"; A's byte offsets
 * are 32-bit on this path; an explicit matrix plan beyond that returns
 * Q8_ERR_TOO_LARGE, and automatic plans use the stream), and serves
 * q8_matvec, q8_matvec_with_plan and a plain single-sibling fused call.
 *   vec, m_tile  must be 0.
 *   workgroups   tiles of 512 columns times K splits (a multiple of the tile
 *           count; every split gets at least one 32-row block; at most 65535
 *           splits, and one tile's split partials, splits x rows x 2 KiB with
 *           rows rounded up to 16, 32 or 64, below 2 GiB), or 0.
 *   waves   8 or 0 (eight waves per workgroup, 64 columns each).
 */
#define Q8_PLAN_STREAM 1
#define Q8_PLAN_MATRIX 2
#define Q8_MATRIX_MIN_ROWS 2
#define Q8_MATRIX_MAX_ROWS 64
typedef struct q8_plan {
  int32_t vec;
  int32_t m_tile;
  int32_t workgroups;
  int32_t waves;
  int32_t kind;
} q8_plan;

/*
 * q8_matvec_choose_plan -- host-only: the plan q8_matvec would use for these
 * extents on a device with `num_cus` compute units, given the byte
 * alignment of W's and S's addresses (pass the pointers' low bits, or 256
 * for allocator-aligned buffers).  Fills *out.  Touches no device.
 * Errors: Q8_ERR_INVALID (bad extents, num_cus < 1, out == NULL).
 */
q8_status q8_matvec_choose_plan(int64_t M, int64_t K, int64_t N,
                                int64_t w_align, int64_t s_align,
                                int32_t num_cus, q8_plan *out);

/*
 * q8_matvec_with_plan -- q8_matvec with explicit launch parameters (zero
 * fields are chosen automatically).  Results are equal for every valid plan
 * up to the f32 rounding of the summation order; a fixed plan is
 * deterministic.  Errors: as q8_matvec; Q8_ERR_INVALID for an unsupported
 * plan.
 */
q8_status q8_matvec_with_plan(const float *A, const int8_t *W, const float *S, float *C,
                              int64_t M, int64_t K, int64_t N, const q8_plan *plan,
                              void *stream);

/*
 * Fused matvec: sibling projections and the elementwise epilogue.
 *
 * "dot and tensor cores", section "The fused epilogue": the elementwise
 * statement that consumes a product runs on each element while the product
 * is written, with no second pass over a stored result (the page's examples
 * multiply a product by a scale, s = s * scale, and multiply an existing
 * accumulator by a factor before adding a product, acc = acc * corr +
 * dot(p, v)).  Here, for every sibling g:
 *
 *   C_g[m,n] = alpha * P_g[m,n] + corr[m] * C_g[m,n]     (corr != NULL)
 *   C_g[m,n] = alpha * P_g[m,n]                          (corr == NULL)
 *
 * where P_g = A (x) dequant(W_g, S_g) is the Q8_0 matvec of q8_matvec.  Each
 * output is rounded as fmaf(corr[m], C_old, alpha * P) (alpha * P alone
 * without corr), so alpha == 1 with no corr reproduces q8_matvec's values.
 *
 * Siblings are up to Q8_MAX_SIBLINGS weight sets of the same shape that share
 * the activation matrix A (for example the gate and up projections of an
 * MLP, or q, k and v); they run in one launch, which streams every sibling's
 * W and S once and stages A once per workgroup.
 */
#define Q8_MAX_SIBLINGS 4

typedef struct q8_sibling {
  const int8_t *W;  /* i8  [K, N], device */
  const float *S;   /* f32 [ceil(K/32), N], device */
  float *C;         /* f32 [M, N], device; read only when corr != NULL */
} q8_sibling;

typedef struct q8_epilogue {
  float alpha;        /* scale of the product */
  const float *corr;  /* f32 [M] device row factors of the existing C, or NULL */
} q8_epilogue;

/*
 * q8_matvec_fused -- the siblings' matvecs with the epilogue, in one launch.
 *   A         f32 [M, K], shared by all siblings
 *   siblings  host array of n_siblings (1..Q8_MAX_SIBLINGS) descriptors; the
 *             C arrays must be distinct and must not alias any input
 *   epilogue  host pointer, or NULL for alpha = 1 and no corr
 *   plan      as for q8_matvec_with_plan, or NULL for automatic; the
 *             siblings' tiles form one list of n_siblings * ceil(N/(64*vec))
 *             tiles, and W and S of every sibling must meet vec's alignment
 * K == 0 gives a zero product (C = corr[m] * C, or zeros).  Deterministic.
 * Errors: as q8_matvec; Q8_ERR_INVALID for n_siblings outside 1..4, a NULL
 * siblings array or pointer, or an unsupported plan.
 */
q8_status q8_matvec_fused(const float *A, const q8_sibling *siblings, int32_t n_siblings,
                          int64_t M, int64_t K, int64_t N, const q8_epilogue *epilogue,
                          const q8_plan *plan, void *stream);

/*
 * q8_dot_t -- C = A @ W^T in exact integer arithmetic.
 *   A  i8  [M, K]   row-major
 *   W  i8  [N, K]   row-major, one output row per row (K contiguous)
 *   C  i32 [M, N]   overwritten; each element is the exact sum reduced modulo
 *                   2^32 (exact whenever |sum| < 2^31, e.g. K <= 131071)
 * Errors: Q8_ERR_INVALID, Q8_ERR_TOO_LARGE, Q8_ERR_UNSUPPORTED_DEVICE,
 * Q8_ERR_HIP.
 */
q8_status q8_dot_t(const int8_t *A, const int8_t *W, int32_t *C,
                   int64_t M, int64_t K, int64_t N, void *stream);

/*
 * Dense f32 products ("dot and tensor cores": the table of built-ins, "The k
 * loop", "Hardware paths" and "The fused epilogue"):
 *   q8_dot_f32    C = alpha * (A @ B)   (+ corr[m] * C),  B f32 [K, N]
 *   q8_dot_t_f32  C = alpha * (A @ B^T) (+ corr[m] * C),  B f32 [N, K]
 *   A  f32 [M, K] row-major, device
 *   B  as above, row-major, device
 *   C  f32 [M, N] row-major, device; overwritten, read only when corr != NULL;
 *      must not alias A or B
 *   epilogue  host pointer, or NULL for alpha = 1 and no corr (an attention
 *      score tile is dot_t with alpha = 1/sqrt(head dim))
 * f32 operands and f32 accumulation: each operand is split exactly into three
 * bf16 parts and the six largest part products are accumulated in f32 on the
 * bf16 matrix cores (the three dropped ones are below 2^-24 |a b| together),
 * so the products keep f32 accuracy; each output is rounded as
 * fmaf(corr[m], C_old, alpha * P).  Any M, K, N >= 0; every pointer 4-byte
 * aligned; when K % 4 == 0 and A and B are 16-byte aligned (and N % 4 == 0
 * for q8_dot_f32), the k-contiguous operands take 16-byte loads.  Operands
 * below about 2^-110 in magnitude may lose their low parts to denormal
 * handling.  K == 0 gives a zero product.  Deterministic: the summation order
 * depends only on K.
 * Errors: Q8_ERR_INVALID (negative extent, NULL or misaligned pointer),
 * Q8_ERR_TOO_LARGE ((M + 128) * (K + 32) or (N + 128) * (K + 32) at or above
 * 2^30, or M * N at or above 2^31), Q8_ERR_UNSUPPORTED_DEVICE, Q8_ERR_HIP.
 */
q8_status q8_dot_f32(const float *A, const float *B, float *C, int64_t M, int64_t K, int64_t N,
                     const q8_epilogue *epilogue, void *stream);
q8_status q8_dot_t_f32(const float *A, const float *B, float *C, int64_t M, int64_t K, int64_t N,
                       const q8_epilogue *epilogue, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *q8_status_string(q8_status s);

/* The hipError_t behind the calling thread's most recent Q8_ERR_HIP (0 if none). */
int q8_last_hip_error(void);

/* Frees every library-owned workspace, including buffers a workspace grew out
 * of, after synchronising the device(s) that own one.  Call it when no call is
 * in flight and no captured graph that uses the workspaces will be replayed
 * again.  The scratch array of q8_matvec_noalloc is not freed. */
void q8_release(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8_GEMV_H */
