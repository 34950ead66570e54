// i8 dot_t for gfx950: C[m,n] = sum_k A[m,k] * W[n,k], exact in i32.
//
// Operation: "dot and tensor cores" page, table of built-ins (dot_t contracts
// the last axis of both operands, a @ b^T) and section "Hardware paths" (i8
// operands accumulate in i32; the path is picked from the shape: matrix
// cores when the output is whole tiles and K fits their k-slice, else a
// 4-byte integer dot, else scalar).  The CDNA paths mirror that choice:
//   * M >= 16 and K % 16 == 0 (16-byte aligned rows): v_mfma_i32_16x16x64_i8.
//   * else K % 4 == 0: v_dot4_i32_i8 (sdot4) with a DPP reduction.
//   * else: a scalar byte loop.
// Integer sums are exact and associative (modulo 2^32), so every path and
// every reduction order gives the same bits.
#include "q8_common.h"

namespace q8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA path
//
// Workgroup: four waves over the same 16 rows of W (16 output columns) and
// MT*16 rows of A; the waves split K into contiguous ranges of 128-byte
// chunks and are summed through LDS at the end.
//
// One 16x16x64 MFMA takes, per lane l, 16 bytes of row (l % 16) of each
// operand.  Which k positions a lane group (l / 16) supplies is free as long
// as both operands use the same assignment; here lane group g takes bytes
// [32g, 32g + 32) of each 128-byte chunk, the first 16 for one MFMA and the
// next 16 for a second, so each lane issues 32 contiguous bytes per chunk.
// The i32 result of lane l is rows 4*(l/16) .. +3 of A's tile, column l % 16.
constexpr int kChunkK = 128;
constexpr int kMfmaUnroll = 8;  // chunks per wave kept in flight (all of a wave's share at K = 4096)

// Raw buffer descriptor over `bytes` bytes: a load whose offset lies past the
// end returns zero without touching memory, so a missing chunk needs no
// branch (a conditional load would make the compiler wait for every load
// already in flight before it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dot_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// An offset past every operand (extents are below 2^31 bytes).
constexpr uint32_t kOutside = 0x80000000u;
// Cache policy of W: non-temporal (each row is read by one workgroup, once).
constexpr int kWPolicy = 2;

template <int MT>
__global__ __launch_bounds__(kThreads) void dot_t_mfma_kernel(DotArgs p) {
  __shared__ v4i red[kWaves][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16 * MT;
  const int nchunks = (p.K + kChunkK - 1) / kChunkK;
  const int cpw = (nchunks + kWaves - 1) / kWaves;
  const int c_begin = wave * cpw;
  const int c_end = min(nchunks, c_begin + cpw);

  // Rows past N or M read a valid row instead; their outputs are not stored.
  const __amdgpu_buffer_rsrc_t w_rs = dot_rsrc(p.W, (uint32_t)p.N * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t a_rs = dot_rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K);
  const uint32_t wrow = (uint32_t)min(n0 + r, p.N - 1) * (uint32_t)p.K;
  uint32_t arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) arow[t] = (uint32_t)min(m0 + 16 * t + r, p.M - 1) * (uint32_t)p.K;

  v4i acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};

  for (int c0 = c_begin; c0 < c_end; c0 += kMfmaUnroll) {
    v4i w[kMfmaUnroll][2], a[kMfmaUnroll][MT][2];
#pragma unroll
    for (int u = 0; u < kMfmaUnroll; ++u) {
      const int k = (c0 + u) * kChunkK + 32 * g;
      const bool chunk_ok = c0 + u < c_end;
      // K % 16 == 0 on this path: each 16-byte half is wholly inside or outside
      // K.  A half outside (or a chunk past this wave's range) reads zeros.
      const bool ok0 = chunk_ok && k + 16 <= p.K;
      const bool ok1 = chunk_ok && k + 32 <= p.K;
      w[u][0] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, ok0 ? wrow + k : kOutside, 0u, kWPolicy);
      w[u][1] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, ok1 ? wrow + k + 16 : kOutside, 0u, kWPolicy);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        a[u][t][0] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, ok0 ? arow[t] + k : kOutside, 0u, 0);
        a[u][t][1] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, ok1 ? arow[t] + k + 16 : kOutside, 0u, 0);
      }
    }
    // Every load of the group is issued before the first multiply waits.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kMfmaUnroll; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][t][0], w[u][0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][t][1], w[u][1], acc[t], 0, 0, 0);
      }
  }

#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const v4i s = (red[0][t][lane] + red[1][t][lane]) + (red[2][t][lane] + red[3][t][lane]);
    const int n = n0 + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 16 * t + 4 * g + e;
      if (m < p.M && n < p.N) p.C[(size_t)m * p.N + n] = s[e];
    }
  }
}

// ---------------------------------------------------------------- sdot4 path
//
// Workgroup: 16 rows of W, four per wave; lane l works on row 4*wave + l/16
// and on LW-byte slices of K strided by 16*LW.  Each lane keeps MT running
// sums (rows of A past M are clamped and not stored); the 16 lanes of a row
// are summed with DPP rotations within their 16-lane row at the end.
constexpr int kDotUnroll = 4;

template <int LW>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t rs, uint32_t off, int policy_nt, int (&x)[LW / 4]) {
  if constexpr (LW == 16) {
    const v4i v = policy_nt ? __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0u, kWPolicy)
                            : __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0u, 0);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
    x[0] = policy_nt ? (int)__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0u, kWPolicy)
                     : (int)__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0u, 0);
  }
}

__device__ __forceinline__ int row16_sum(int v) {
  // row_ror:8, 4, 2, 1 inside each 16-lane row: every lane ends with the row's sum.
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x122, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x121, 0xf, 0xf, false);
  return v;
}

template <int LW, int MT>
__global__ __launch_bounds__(kThreads) void dot_t_sdot4_kernel(DotArgs p) {
  constexpr int NW = LW / 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int n = blockIdx.x * 16 + 4 * wave + (lane >> 4);
  const int m0 = blockIdx.y * MT;
  const __amdgpu_buffer_rsrc_t w_rs = dot_rsrc(p.W, (uint32_t)p.N * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t a_rs = dot_rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K);
  const uint32_t wrow = (uint32_t)min(n, p.N - 1) * (uint32_t)p.K;
  uint32_t arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) arow[t] = (uint32_t)min(m0 + t, p.M - 1) * (uint32_t)p.K;

  int acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0;

  constexpr int kStep = 16 * LW;  // bytes of K per row per step
  for (int k0 = 0; k0 < p.K; k0 += kStep * kDotUnroll) {
    int w[kDotUnroll][NW], a[kDotUnroll][MT][NW];
#pragma unroll
    for (int u = 0; u < kDotUnroll; ++u) {
      const int k = k0 + u * kStep + LW * c;
      const bool ok = k + LW <= p.K;  // K % LW == 0 on this path; a slice past K reads zeros
      load_words<LW>(w_rs, ok ? wrow + (uint32_t)k : kOutside, 1, w[u]);
#pragma unroll
      for (int t = 0; t < MT; ++t) load_words<LW>(a_rs, ok ? arow[t] + (uint32_t)k : kOutside, 0, a[u][t]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kDotUnroll; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < NW; ++j) acc[t] = __builtin_amdgcn_sdot4(a[u][t][j], w[u][j], acc[t], false);
  }

#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int s = row16_sum(acc[t]);
    if (c == 0 && n < p.N && m0 + t < p.M) p.C[(size_t)(m0 + t) * p.N + n] = s;
  }
}

// ---------------------------------------------------------------- scalar path

__global__ __launch_bounds__(kThreads) void dot_t_scalar_kernel(DotArgs p) {
  const size_t total = (size_t)p.M * p.N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / p.N);
    const int n = (int)(i - (size_t)m * p.N);
    const int8_t *a = p.A + (size_t)m * p.K;
    const int8_t *w = p.W + (size_t)n * p.K;
    uint32_t s = 0;  // modular sum
    for (int k = 0; k < p.K; ++k) s += (uint32_t)((int)a[k] * (int)w[k]);
    p.C[i] = (int32_t)s;
  }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

template <int LW>
hipError_t launch_sdot4(const DotArgs &a, hipStream_t stream) {
  const int mt = a.M <= 1 ? 1 : a.M <= 2 ? 2 : a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
  const dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + mt - 1) / mt));
  switch (mt) {
    case 1: hipLaunchKernelGGL((dot_t_sdot4_kernel<LW, 1>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((dot_t_sdot4_kernel<LW, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((dot_t_sdot4_kernel<LW, 4>), grid, dim3(kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((dot_t_sdot4_kernel<LW, 8>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((dot_t_sdot4_kernel<LW, 16>), grid, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

int dot_t_path(int M, int K, const void *A, const void *W) {
  if (M >= 16 && K % 16 == 0 && aligned16(A) && aligned16(W)) return 2;
  if (K % 4 == 0 && aligned4(A) && aligned4(W)) return 1;
  return 0;
}

hipError_t launch_dot_t(const DotArgs &a, hipStream_t stream) {
  switch (dot_t_path(a.M, a.K, a.A, a.W)) {
    case 2: {
      // Two 16-row tiles of A per pass when M allows, else one.
      if (a.M >= 32) {
        const dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + 31) / 32));
        hipLaunchKernelGGL(dot_t_mfma_kernel<2>, grid, dim3(kThreads), 0, stream, a);
      } else {
        const dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + 15) / 16));
        hipLaunchKernelGGL(dot_t_mfma_kernel<1>, grid, dim3(kThreads), 0, stream, a);
      }
      return hipGetLastError();
    }
    case 1:
      return (a.K % 16 == 0 && aligned16(a.A) && aligned16(a.W)) ? launch_sdot4<16>(a, stream)
                                                                  : launch_sdot4<4>(a, stream);
    default: {
      size_t blocks = ((size_t)a.M * a.N + kThreads - 1) / kThreads;
      if (blocks > 4096) blocks = 4096;
      hipLaunchKernelGGL(dot_t_scalar_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
}

}  // namespace q8
