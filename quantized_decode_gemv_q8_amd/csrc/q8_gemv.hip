// Q8_0 matvec for gfx950: C[m,n] = sum_k A[m,k] * W[k,n] * S[k/32, n].
//
// Operation: "Q8_0 matvec" page, sections "The tensors" (definition and
// layouts), "Factoring out the scale" (one scale multiply per block and
// column, applied to the block's unscaled partial) and "Bounds" (ragged N is
// masked; the K loop is whole blocks plus one masked remainder).
//
// Work decomposition (a CDNA design, not the pages' 64-column CTA tile):
//   * A workgroup is four wave64s.  It owns a column tile of 64*VEC columns and
//     a contiguous range of K blocks (its "split"); the four waves take the
//     range's blocks round-robin, so together they stream 4 consecutive
//     32-row blocks of the tile at a time.
//   * Lane l of a wave owns columns [tile*64*VEC + l*VEC, +VEC) and reads every
//     one of the 32 rows of a block for them: one VEC-byte load per row, so a
//     wave instruction reads 64*VEC contiguous bytes of one W row.  The block's
//     unscaled partial is therefore complete inside the lane, and the scale is
//     applied exactly once per block and column, with no cross-lane traffic.
//   * The activations of the workgroup's K range are staged once in LDS, with
//     the pitch padding rule of "@padstage" ("Which tiles it reaches"); every
//     lane of a wave reads the same activation (an LDS broadcast).
//   * Loads are software-pipelined: the next chunk of rows is in flight while
//     the current one is converted and multiplied.
//   * The four waves' sums are combined through LDS in a fixed tree.  With
//     more than one split per tile, each workgroup writes its partial; the last
//     workgroup to arrive (agent-scope release/acquire on a counter) sums the
//     partials in split order, writes C and re-arms the counter.  The result
//     does not depend on arrival order: the kernel is deterministic.
#include <type_traits>

#include "q8_common.h"

namespace q8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Geometry of one kernel instance.
template <int VEC>
struct Geo {
  static constexpr int kWords = (VEC + 3) / 4;                    // 32-bit words per lane-row
  static constexpr int kChunkRows = VEC >= 8 ? 128 / VEC : 32;    // rows per pipelined chunk
  static constexpr int kChunksPerBlock = kBlock / kChunkRows;
  static constexpr int kTileCols = 64 * VEC;
};

// Activation values each thread stages into LDS: m_tile * bps * 32 <= 256 * kStageRegs.
constexpr int kStageRegs = 8;

// W and S are read with raw buffer loads: the lane's column byte offset is one
// VGPR shared by every row, and the row's byte offset is a wave-uniform SGPR
// (soffset), so no per-row address arithmetic runs on the vector ALUs.  The
// descriptors also bound every access to the tensor's extent.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Third descriptor word for raw (stride 0) buffers on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
}

template <int VEC>
__device__ __forceinline__ void load_w(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                       uint32_t (&w)[Geo<VEC>::kWords]) {
  if constexpr (VEC == 16) {
    const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (VEC == 8) {
    const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (VEC == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  } else if constexpr (VEC == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0);
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff, soff, 0);
  }
}

// Byte j of a lane-row as f32; exact, and a single sign-extending convert.
template <int VEC>
__device__ __forceinline__ float wbyte(const uint32_t (&w)[Geo<VEC>::kWords], int j) {
  return static_cast<float>(static_cast<int8_t>(w[j >> 2] >> (8 * (j & 3))));
}

template <int VEC>
__device__ __forceinline__ void load_s(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, float (&s)[VEC]) {
  if constexpr (VEC >= 4) {
#pragma unroll
    for (int i = 0; i < VEC / 4; ++i) {
      const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16u * i, soff, 0);
      s[4 * i] = __uint_as_float(x.x);
      s[4 * i + 1] = __uint_as_float(x.y);
      s[4 * i + 2] = __uint_as_float(x.z);
      s[4 * i + 3] = __uint_as_float(x.w);
    }
  } else if constexpr (VEC == 2) {
    const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    s[0] = __uint_as_float(x.x);
    s[1] = __uint_as_float(x.y);
  } else {
    s[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
  }
}

// Makes this wave's LDS writes visible to the workgroup, without waiting for
// its outstanding global loads (a plain __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Compile-time loop: calls f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F &&f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>{});
      StaticFor<B + 1, E>::run(f);
    }
  }
};

// Per-wave streaming state.  A wave's k-th chunk (CR rows of one block)
// lives in register buffer k % 2; its block is the wave's k / CPB-th block and
// its position in that block is k % CPB.  Buffer and position are template
// arguments so that the steady-state loop has no conditional loads (which
// would force conservative waits on the load counter).
template <int VEC, int MT>
struct WaveStream {
  using G = Geo<VEC>;
  static constexpr int CR = G::kChunkRows;
  static constexpr int CPB = G::kChunksPerBlock;
  static constexpr int NWD = G::kWords;
  static constexpr int kUnroll = CPB > 2 ? CPB : 2;  // chunks per steady-state iteration

  __amdgpu_buffer_rsrc_t w_rs, s_rs;
  uint32_t col_off;   // this lane's byte offset into a W row
  int K, N, pitch;
  int b_first;        // first block of this wave
  int lds_first;      // its offset in the LDS stage
  const float *a_lds;
  uint32_t w[2][CR][NWD];
  float s[2][VEC];
  float part[MT][VEC];
  float acc[MT][VEC];

  template <int BUF, int H>
  __device__ __forceinline__ void issue(int j) {
    const int b = b_first + kWaves * j;
    const int row0 = b * kBlock + H * CR;
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      // Rows of the K remainder block past K re-read row K-1: their staged
      // activation is zero, so they add nothing ("Bounds").
      const int row = min(row0 + i, K - 1);
      load_w<VEC>(w_rs, col_off, (uint32_t)row * (uint32_t)N, w[BUF][i]);
    }
    if constexpr (H == CPB - 1) load_s<VEC>(s_rs, col_off * 4u, (uint32_t)b * (uint32_t)N * 4u, s[BUF]);
  }

  template <int BUF, int H>
  __device__ __forceinline__ void consume(int j) {
    const int kl = lds_first + kWaves * kBlock * j + H * CR;
    if constexpr (H == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < VEC; ++v) part[m][v] = 0.f;
    }
#pragma unroll
    for (int i0 = 0; i0 < CR; i0 += 4) {
      v4f a4[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) a4[m] = *reinterpret_cast<const v4f *>(&a_lds[m * pitch + kl + i0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float wf = wbyte<VEC>(w[BUF][i0 + i], v);
#pragma unroll
          for (int m = 0; m < MT; ++m) part[m][v] = fmaf(a4[m][i], wf, part[m][v]);
        }
      }
    }
    // "Factoring out the scale": one multiply per block and column.
    if constexpr (H == CPB - 1) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[m][v] = fmaf(part[m][v], s[BUF][v], acc[m][v]);
    }
  }

  // Streams chunks [0, nchunk): chunk k+1 is in flight while chunk k is used.
  // The scheduling barriers keep the compiler from sinking the next chunk's
  // loads down to their uses (which it otherwise does to save registers).
  __device__ __forceinline__ void run(int nchunk) {
    int c0 = 0;
    for (; c0 + kUnroll < nchunk; c0 += kUnroll) {
      const int j0 = c0 / CPB;
      StaticFor<0, kUnroll>::run([&](auto u_) {
        constexpr int u = decltype(u_)::value;
        issue<(u + 1) % 2, (u + 1) % CPB>(j0 + (u + 1) / CPB);
        __builtin_amdgcn_sched_barrier(0);
        consume<u % 2, u % CPB>(j0 + u / CPB);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // Last group: 1 .. kUnroll chunks.
    const int j0 = c0 / CPB;
    StaticFor<0, kUnroll>::run([&](auto u_) {
      constexpr int u = decltype(u_)::value;
      if (c0 + u < nchunk) {
        if (c0 + u + 1 < nchunk) issue<(u + 1) % 2, (u + 1) % CPB>(j0 + (u + 1) / CPB);
        __builtin_amdgcn_sched_barrier(0);
        consume<u % 2, u % CPB>(j0 + u / CPB);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  }
};

template <int VEC, int MT>
__global__ __launch_bounds__(kThreads) void q8_gemv_kernel(GemvArgs p) {
  using G = Geo<VEC>;
  constexpr int TW = G::kTileCols;

  extern __shared__ __attribute__((aligned(16))) float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x % p.n_tiles;
  const int split = blockIdx.x / p.n_tiles;
  const int m0 = blockIdx.y * MT;
  const int b_begin = split * p.bps;
  const int b_end = min(p.KB, b_begin + p.bps);
  const int k_begin = b_begin * kBlock;
  const int ks = (b_end - b_begin) * kBlock;  // staged activations per row
  const int col = tile * TW + lane * VEC;

  WaveStream<VEC, MT> st;
  st.w_rs = buffer_rsrc(p.W, (uint32_t)p.K * (uint32_t)p.N);
  st.s_rs = buffer_rsrc(p.S, (uint32_t)p.KB * (uint32_t)p.N * 4u);
  // Columns past N (ragged last tile) load column 0 instead and are never stored.
  st.col_off = col < p.N ? (uint32_t)col : 0u;
  st.K = p.K;
  st.N = p.N;
  st.pitch = p.pitch;
  st.b_first = b_begin + wave;
  st.lds_first = wave * kBlock;
  st.a_lds = lds;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int v = 0; v < VEC; ++v) st.acc[m][v] = 0.f;

  // This wave's blocks are b_begin + wave + 4 j; each is CPB chunks.
  const int nblk = max(0, (b_end - b_begin - wave + kWaves - 1) / kWaves);
  const int nchunk = nblk * WaveStream<VEC, MT>::CPB;

  // Activations first (their loads complete before the W loads issued next),
  // so that waiting for them does not drain the first chunk of W.
  float stage[kStageRegs];
#pragma unroll
  for (int r = 0; r < kStageRegs; ++r) {
    const int idx = tid + kThreads * r;
    const int m = idx / ks;
    const int k = idx - m * ks;
    const bool ok = m < MT && m0 + m < p.M && k_begin + k < p.K;
    stage[r] = ok ? p.A[(size_t)(m0 + m) * p.K + k_begin + k] : 0.f;
  }
  if (nchunk > 0) st.template issue<0, 0>(0);
#pragma unroll
  for (int r = 0; r < kStageRegs; ++r) {
    const int idx = tid + kThreads * r;
    const int m = idx / ks;
    const int k = idx - m * ks;
    if (m < MT) lds[m * p.pitch + k] = stage[r];
  }
  lds_barrier();

  if (nchunk > 0) st.run(nchunk);

  // Combine the four waves: LDS is reused for [wave][m][column].
  lds_barrier();
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float *dst = &lds[(wave * MT + m) * TW + lane * VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) dst[v] = st.acc[m][v];
  }
  lds_barrier();

  const bool direct = p.splits == 1;
  float *out = direct ? p.C : p.partial + (size_t)split * p.M * p.N;
  for (int o = tid; o < MT * TW; o += kThreads) {
    const float x = (lds[o] + lds[MT * TW + o]) + (lds[2 * MT * TW + o] + lds[3 * MT * TW + o]);
    const int m = o / TW;
    const int n = tile * TW + (o - m * TW);
    if (n < p.N && m0 + m < p.M) out[(size_t)(m0 + m) * p.N + n] = x;
  }
  if (direct) return;

  // Split-K: publish this partial, count arrivals, the last arrival combines.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  __shared__ uint32_t is_last;
  uint32_t *ctr = &p.counters[blockIdx.y * p.n_tiles + tile];
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == (uint32_t)(p.splits - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  for (int o = tid; o < MT * TW; o += kThreads) {
    const int m = o / TW;
    const int n = tile * TW + (o - m * TW);
    if (n >= p.N || m0 + m >= p.M) continue;
    const float *src = p.partial + (size_t)(m0 + m) * p.N + n;
    const size_t stride = (size_t)p.M * p.N;
    // Fixed order: pairwise within groups of four splits, then group sums in order.
    float total = 0.f;
    int s = 0;
    for (; s + 4 <= p.splits; s += 4) {
      const float g = (src[s * stride] + src[(s + 1) * stride]) + (src[(s + 2) * stride] + src[(s + 3) * stride]);
      total += g;
    }
    for (; s < p.splits; ++s) total += src[s * stride];
    p.C[(size_t)(m0 + m) * p.N + n] = total;
  }
  if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_fill_kernel(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

typedef void (*GemvKernel)(GemvArgs);

template <int VEC, int MT>
constexpr GemvKernel instance() {
  if constexpr (MT * VEC <= 32) return q8_gemv_kernel<VEC, MT>;
  return nullptr;
}

template <int VEC>
GemvKernel pick_mt(int m_tile) {
  switch (m_tile) {
    case 1: return instance<VEC, 1>();
    case 2: return instance<VEC, 2>();
    case 4: return instance<VEC, 4>();
    case 8: return instance<VEC, 8>();
    default: return nullptr;
  }
}

GemvKernel pick(int vec, int m_tile) {
  switch (vec) {
    case 16: return pick_mt<16>(m_tile);
    case 8: return pick_mt<8>(m_tile);
    case 4: return pick_mt<4>(m_tile);
    case 2: return pick_mt<2>(m_tile);
    case 1: return pick_mt<1>(m_tile);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_gemv(int vec, int m_tile, const GemvArgs &args, int m_chunks, size_t lds_bytes,
                       hipStream_t stream) {
  GemvKernel k = pick(vec, m_tile);
  if (k == nullptr) return hipErrorInvalidValue;
  if ((size_t)m_tile * args.bps * kBlock > (size_t)kThreads * kStageRegs) return hipErrorInvalidValue;
  dim3 grid((unsigned)(args.n_tiles * args.splits), (unsigned)m_chunks, 1);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), lds_bytes, stream, args);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void *p, size_t n_words, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t *)p, n_words);
  return hipGetLastError();
}

}  // namespace q8
