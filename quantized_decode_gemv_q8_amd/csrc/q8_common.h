// Internal declarations shared by the kernels and the host dispatch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Q8_0 block length along K ("Q8_0 matvec", section "The tensors").
constexpr int kBlock = 32;
// Waves per workgroup and threads per workgroup (the pages launch 256 threads
// per CTA; on CDNA that is four wave64s, one per SIMD of a CU).
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// LDS bank period in bytes.  A staged tile whose row pitch is a multiple of it
// gets 8 extra elements per row ("@padstage", "Which tiles it reaches").
constexpr int kLdsBankPeriodBytes = 128;

// Row pitch (in elements) of an LDS staging tile with `cols` elements of
// `elem_bytes` each: padded by 8 elements when the pitch is a multiple of the
// bank period, so that a column of the tile spreads over banks.
__host__ __device__ constexpr int padded_pitch(int cols, int elem_bytes) {
  return (cols * elem_bytes) % kLdsBankPeriodBytes == 0 ? cols + 8 : cols;
}

// XCDs of the device: the dispatcher sends workgroup b of a grid to XCD b % kXcds.
constexpr int kXcds = 8;

// Weight sets sharing one activation matrix in a single launch.
constexpr int kMaxSiblings = 4;

// Words between two split-K arrival counters: one counter per 128-byte line.
// Atomics on one line are served one after another; on a small problem every
// workgroup arrives within a microsecond, and with the counters packed
// together they queue up (K = N = 4096: 12.9 against 10.7 us).
constexpr int kCounterStride = 32;

// Arguments of the Q8_0 matvec kernel (one launch).  The column tiles of all
// siblings, sibling-major, form one list of n_tiles tiles; its (tile,
// 4-block group) units, tile-major, are dealt to the n_wg workgroups of a pass
// in contiguous runs: upw units each, one more for the first rem.
struct GemvArgs {
  const float *A;                 // [M, K]
  const int8_t *W[kMaxSiblings];  // [K, N] per sibling
  const float *S[kMaxSiblings];   // [KB, N] per sibling
  float *C[kMaxSiblings];         // [M, N] per sibling
  const float *corr;              // [M] epilogue row factors, or null
  float alpha;                    // epilogue scale of the product
  float *partial;                 // [m_chunks][n_tiles][cmax][m_tile * 64 * vec] partial sums
  uint32_t *counters;             // [m_chunks * n_tiles] arrival counters (kCounterStride apart), zero between calls
  int M, K, N, KB;
  int tiles_per;                  // column tiles of 64 * vec columns per sibling
  int n_tiles;                    // tiles over all siblings
  int groups;                     // groups of four K blocks per tile: ceil(KB / 4)
  int n_wg;                       // workgroups per pass (per chunk of m_tile rows of A)
  int upw, rem;                   // units per workgroup
  int cmax;                       // most workgroups that share one tile
  int pitch;                      // row pitch of a wave's activation stage in LDS, floats
  int band_runs;                  // > 0: runs per tile, workgroups take the runs in XCD bands (see run_of_block)
  int xcd_runs;                   // > 0: runs per tile, all runs of a tile on one XCD; the split-K
                                  //      partials then stay in that XCD's L2 (see run_of_block)
  int xcc_skew;                   // testing only: nonzero makes some contributors report another XCD
};

// Launches the Q8_0 matvec kernel instance (vec, m_tile) on `stream`.
// Returns hipErrorInvalidValue for an instance that is not compiled.
hipError_t launch_gemv(int vec, int m_tile, const GemvArgs &args, int m_chunks,
                       size_t lds_bytes, hipStream_t stream);

// Writes, for each of n_wg workgroups, the id of the XCD it ran on to out[b].
hipError_t launch_xcc_probe(uint32_t *out, int n_wg, hipStream_t stream);

// Writes `n` zero words at `p` (used for fresh counters).
hipError_t launch_zero_fill(void *p, size_t n_words, hipStream_t stream);

// The epilogue with a zero product (K == 0): C[m,n] = alpha * 0 + corr[m] * C[m,n]
// (corr null: the zero product alone).
hipError_t launch_empty_product(float *C, int M, int N, float alpha, const float *corr, hipStream_t stream);

// Largest dynamic LDS footprint (bytes) the matvec kernel may be given: a
// gfx950 workgroup may use the CU's 160 KB; 1 KB stays for static LDS.
constexpr size_t kMaxGemvLds = 159 * 1024;

// Activation values each lane stages into its wave's LDS region (registers
// per lane): m_tile * (blocks per wave in a run) * 32 <= 64 * kStageRegs.
constexpr int kStageRegs = 8;

// Most (tile, group) units one workgroup may take at a given m_tile: a wave
// stages m_tile * units * 32 activations from kStageRegs registers per lane.
constexpr int max_units_per_wg(int m_tile) { return 64 * kStageRegs / (m_tile * kBlock); }

// LDS bytes the matvec kernel needs: four private activation stages of
// m_tile rows of `count` blocks, at vec >= 8 four scale hand-over areas of
// 64 * vec floats, and parked sums for `nseg` tiles (the most tiles one
// workgroup's run touches) from each of the four waves.
inline size_t gemv_lds_bytes(int vec, int m_tile, int count, int nseg) {
  const size_t stage = (size_t)kWaves * m_tile * padded_pitch(count * kBlock, 4) * 4;
  const size_t scales = vec >= 8 ? (size_t)kWaves * 64 * vec * 4 : 0;
  const size_t slots = (size_t)nseg * kWaves * m_tile * 64 * vec * 4;
  return stage + scales + slots;
}

// Most tiles one workgroup's run may touch: the epilogue keeps one arrival
// bit and one contributor range per tile.
constexpr int kMaxSegments = 32;

// Most tiles a run of `count` (tile, group) units touches, with `groups`
// groups per tile.
constexpr int max_segments(int count, int groups) { return (count - 1 + groups - 1) / groups + 1; }

// Arguments of the Q8_0 product for 2..64 activation rows on the matrix cores:
// tiles of 512 columns, each split into `splits` contiguous ranges of `bps`
// K blocks (one workgroup each).  Rows beyond one instance's 16 * RT would run
// as passes on grid z, each with its own partials and counters.
struct GemmArgs {
  const float *A;      // [M, K]
  const int8_t *W;     // [K, N]
  const float *S;      // [KB, N]
  float *C;            // [M, N]
  float *partial;      // [passes][n_tiles][splits][16 * RT * 512] split partials (splits > 1)
  uint32_t *counters;  // [passes][n_tiles] arrival counters (kCounterStride apart), zero between calls
  int M, K, N, KB;
  int n_tiles, splits, bps;
  int xcd_local;       // nonzero: every split of a tile runs on one XCD (n_tiles a multiple of 8); partials stay in its L2
  int xcc_skew;        // testing only: nonzero makes some splits report another XCD
  int w_width;         // bytes per W load: 16, 8 or 4 (N and W's address are multiples of it)
};

// Widest W load of the matrix-core product that N and W's address allow (16,
// 8 or 4 bytes), or 0 if W rows are not 4-byte aligned.
constexpr int gemm_w_width(int64_t N, int64_t w_align) {
  return N % 16 == 0 && w_align % 16 == 0 ? 16 : N % 8 == 0 && w_align % 8 == 0 ? 8
         : N % 4 == 0 && w_align % 4 == 0                                      ? 4
                                                                               : 0;
}

// Rows of A the matrix-core product takes at most, its column tile and its
// waves per workgroup.
constexpr int kGemmMaxRows = 64;
constexpr int kGemmTileCols = 512;
constexpr int kGemmWaves = 8;
// 16-row tiles of A per pass of the matrix-core product: 1 up to 16 rows, 2 up
// to 32, 4 up to 64 (one pass reads W once for all of them).
constexpr int gemm_row_tiles(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

hipError_t launch_gemm(const GemmArgs &args, hipStream_t stream);

// Arguments of the dense f32 dot / dot_t kernels.
struct DenseArgs {
  const float *A;     // [M, K]
  const float *B;     // [K, N] (dot) or [N, K] (dot_t)
  float *C;           // [M, N]
  const float *corr;  // [M] epilogue row factors, or null
  float alpha;        // epilogue scale of the product
  int M, K, N;
};

// vec 4: every row of A and B starts 16-byte aligned; vec 1 otherwise.
// max_wgs: most workgroups to launch; more tiles than that are shared out.
hipError_t launch_dense_f32(const DenseArgs &args, bool trans_b, int vec, int max_wgs, hipStream_t stream);

// Arguments of the i8 dot_t kernels.
struct DotArgs {
  const int8_t *A;  // [M, K]
  const int8_t *W;  // [N, K]
  int32_t *C;       // [M, N]
  int M, K, N;
};

hipError_t launch_dot_t(const DotArgs &args, hipStream_t stream);

// The dot_t kernel a call takes: 2 the i8 matrix cores, 1 sdot4, 0 scalar.
int dot_t_path(int M, int K, const void *A, const void *W);

}  // namespace q8
