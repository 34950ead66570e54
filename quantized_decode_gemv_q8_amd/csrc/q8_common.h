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

// Arguments of the Q8_0 matvec kernel (one launch).
struct GemvArgs {
  const float *A;        // [M, K]
  const int8_t *W;       // [K, N]
  const float *S;        // [KB, N]
  float *C;              // [M, N]
  float *partial;        // [splits, M, N] split-K partial sums (splits > 1)
  uint32_t *counters;    // [m_chunks * n_tiles] arrival counters, zero between calls
  int M, K, N, KB;
  int n_tiles;           // column tiles of 64 * vec columns
  int splits;            // workgroups per column tile along K
  int bps;               // blocks per split
  int pitch;             // LDS row pitch of the staged activations, in floats
};

// Launches the Q8_0 matvec kernel instance (vec, m_tile) on `stream`.
// Returns hipErrorInvalidValue for an instance that is not compiled.
hipError_t launch_gemv(int vec, int m_tile, const GemvArgs &args, int m_chunks,
                       size_t lds_bytes, hipStream_t stream);

// Writes `n` zero words at `p` (used for K == 0 outputs and fresh counters).
hipError_t launch_zero_fill(void *p, size_t n_words, hipStream_t stream);

// Largest LDS footprint (bytes) the matvec kernel may be given.
constexpr size_t kMaxGemvLds = 64 * 1024;

// LDS bytes the matvec kernel needs for a plan.
inline size_t gemv_lds_bytes(int vec, int m_tile, int bps) {
  size_t stage = (size_t)m_tile * padded_pitch(bps * kBlock, 4) * 4;
  size_t red = (size_t)kWaves * m_tile * 64 * vec * 4;
  return stage > red ? stage : red;
}

// Arguments of the i8 dot_t kernels.
struct DotArgs {
  const int8_t *A;  // [M, K]
  const int8_t *W;  // [N, K]
  int32_t *C;       // [M, N]
  int M, K, N;
};

hipError_t launch_dot_t(const DotArgs &args, hipStream_t stream);

}  // namespace q8
