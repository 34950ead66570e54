// Q8_0 matvec kernel template for gfx950: C[m,n] = sum_k A[m,k] * W[k,n] * S[k/32, n].
// Included by one translation unit per VEC (q8_gemv_v*.hip), which compile in parallel.
//
// Operation: "Q8_0 matvec" page, sections "The tensors" (definition and
// layouts), "Factoring out the scale" (one scale multiply per block and
// column, applied to the block's unscaled partial) and "Bounds" (ragged N is
// masked, and a K that is not a multiple of 32 ends in a short last block
// whose missing rows contribute nothing).
//
// Work decomposition (a CDNA design, not the pages' 64-column CTA tile):
//   * W is cut into column tiles of 64*VEC columns and, along K, into groups of
//     four 32-row blocks.  The (tile, group) units, tile-major, are dealt out
//     in contiguous runs of equal length (within one unit) to the grid's
//     workgroups, one per CU at the decode shapes: every CU gets the same
//     work.  (Rounding work to whole tiles leaves CUs with two workgroups
//     next to CUs with one; two workgroups per CU finish unevenly because the
//     older one wins issue arbitration.)  A run may end in one tile and
//     continue in the next: each piece is a "segment".
//   * A workgroup is four wave64s; wave w takes block w of each group of its
//     segment, so the workgroup streams 128 consecutive rows of the tile.
//   * Lane l of a wave owns columns [tile*64*VEC + l*VEC, +VEC) and reads all
//     32 rows of a block for them: one VEC-byte load per row, so a wave
//     instruction reads 64*VEC contiguous bytes of one W row.  The block's
//     unscaled partial is complete inside the lane, and the scale is applied
//     exactly once per block and column, with no cross-lane traffic.
//   * Each wave stages the activations of its own blocks in a private LDS
//     region whose row pitch follows the padding rule of "@padstage" ("Which
//     tiles it reaches").  Every lane reads the same activation (a broadcast),
//     and no barrier is needed: LDS accesses of one wave are ordered.
//   * Loads are software-pipelined: the next chunk of rows is in flight while
//     the current one is converted and multiplied.
//   * The four waves' sums are combined through LDS in a fixed tree.  A
//     segment that covers its whole tile stores C directly.  Otherwise its
//     workgroup publishes a partial with device-coherent stores, waits for
//     them to complete, and bumps the tile's counter; the last of the tile's
//     contributors reads the partials with device-coherent loads, sums them
//     in K order, writes C and re-arms the counter.  (Agent-scope release and
//     acquire fences would write back or invalidate the whole L2 of an XCD
//     every time.)  Nothing waits on another workgroup, and the result does
//     not depend on arrival order.
#pragma once

#include <type_traits>

#include "q8_common.h"
#include "q8_sum.h"
#include "q8_xcd.h"

namespace q8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Column pieces per lane at VEC 16: two pieces of eight columns, 512 columns
// apart, so that each W load instruction of a wave reads 512 contiguous bytes
// of a row (eight per lane), as at VEC 8, and one workgroup reads both halves
// of each kilobyte of the row.
constexpr int kPiecesAt16 = 2;

// Geometry of one kernel instance.
template <int VEC>
struct Geo {
  static constexpr int kWords = (VEC + 3) / 4;                    // 32-bit words per lane-row
  static constexpr int kChunkRows = VEC >= 8 ? 128 / VEC : 32;    // rows per pipelined chunk
  static constexpr int kChunksPerBlock = kBlock / kChunkRows;
  static constexpr int kTileCols = 64 * VEC;
  // A lane owns kPieces runs of kPieceCols adjacent columns; piece p of lane l
  // starts at column 64 * kPieceCols * p + kPieceCols * l of the tile.
  static constexpr int kPieces = VEC == 16 ? kPiecesAt16 : 1;
  static constexpr int kPieceCols = VEC / kPieces;
  __device__ static constexpr int col(int lane, int v) {
    return 64 * kPieceCols * (v / kPieceCols) + kPieceCols * lane + v % kPieceCols;
  }
  // At VEC >= 8 a lane's scales (4*VEC contiguous bytes) would take VEC/4
  // 16-byte loads strided across the wave.  Instead the wave loads the S row
  // of its tile with fully coalesced 16-byte loads (lane l takes columns
  // 4l + 256i .. +3) and hands the values to their owners through a private
  // LDS area of 64*VEC floats.
  static constexpr bool kSwizzleScales = VEC >= 8;
  static constexpr int kScaleLoads = (VEC + 3) / 4;  // 16-byte S loads per lane and block
};


// W and S are read with raw buffer loads: the lane's column byte offset is one
// VGPR shared by every row, and the row's byte offset is a wave-uniform SGPR
// (soffset), so no per-row address arithmetic runs on the vector ALUs.  Every
// offset is clamped into the tensor before it is used.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Third descriptor word for raw (stride 0) buffers on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the streamed loads: non-temporal.  W and S are each read
// exactly once per call, so keeping them in the caches only evicts useful
// lines; measured on MI355X this streams 5-10% faster than the default policy.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
}

template <int VEC>
__device__ __forceinline__ void load_w(__amdgpu_buffer_rsrc_t rs, const uint32_t (&voff)[Geo<VEC>::kPieces],
                                       uint32_t soff, uint32_t (&w)[Geo<VEC>::kWords]) {
  constexpr int PC = Geo<VEC>::kPieceCols;
#pragma unroll
  for (int p = 0; p < Geo<VEC>::kPieces; ++p) {
    if constexpr (PC == 16) {
      const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[p], soff, kStreamPolicy);
      w[4 * p] = x.x; w[4 * p + 1] = x.y; w[4 * p + 2] = x.z; w[4 * p + 3] = x.w;
    } else if constexpr (PC == 8) {
      const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rs, voff[p], soff, kStreamPolicy);
      w[2 * p] = x.x; w[2 * p + 1] = x.y;
    } else if constexpr (PC == 4) {
      w[p] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff[p], soff, kStreamPolicy);
    } else if constexpr (PC == 2) {
      w[p] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff[p], soff, kStreamPolicy);
    } else {
      w[p] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff[p], soff, kStreamPolicy);
    }
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
      const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16u * i, soff, kStreamPolicy);
      s[4 * i] = __uint_as_float(x.x);
      s[4 * i + 1] = __uint_as_float(x.y);
      s[4 * i + 2] = __uint_as_float(x.z);
      s[4 * i + 3] = __uint_as_float(x.w);
    }
  } else if constexpr (VEC == 2) {
    const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kStreamPolicy);
    s[0] = __uint_as_float(x.x);
    s[1] = __uint_as_float(x.y);
  } else {
    s[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kStreamPolicy));
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

// Calls f(std::integral_constant<int, v>) for the run-time value v in [B, E)
// (one branch per value; v outside the range calls nothing).
template <int B, int E>
struct StaticSwitch {
  template <class F>
  __device__ __forceinline__ static void run(int v, F &&f) {
    if constexpr (B < E) {
      if (v == B) f(std::integral_constant<int, B>{});
      else StaticSwitch<B + 1, E>::run(v, f);
    }
  }
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Rows per pipelined chunk of instance (VEC, MT).  Instances wider than 16
// columns x rows per lane use half-size chunks so that their register ring
// of W fits beside the MT x VEC partial sums without spilling.
template <int VEC, int MT>
constexpr int kChunkRowsOf = VEC * MT > 16 ? Geo<VEC>::kChunkRows / 2 : Geo<VEC>::kChunkRows;

// Per-wave streaming state.  A workgroup's run of units is one stream: wave w
// takes block w of every group of the run, in order, so every wave of the
// workgroup has `count` blocks.  The wave's k-th chunk (CR rows of one block)
// lives in register buffer k % kDepth; its block is the wave's (k / CPB)-th
// and its position in that block is k % CPB.  kDepth - 1 chunks are in flight
// ahead of the one being used.  Buffer and position are template arguments,
// so no load is conditional in the steady state (a conditional load forces
// conservative waits on the load counter).  When a block ends a tile's share
// of the run, the wave parks its accumulators in an LDS slot and streams on.
template <int VEC, int MT, int DEPTH>
struct WaveStream {
  using G = Geo<VEC>;
  static constexpr int CR = kChunkRowsOf<VEC, MT>;
  static constexpr int CPB = kBlock / CR;
  static constexpr int NWD = G::kWords;
  static constexpr int TW = G::kTileCols;
  static constexpr int kDepth = DEPTH;  // register buffers (chunks) per wave
  // Chunks per steady-state iteration: cycles both the buffers and the blocks.
  static constexpr int kUnroll = DEPTH / gcd_c(DEPTH, CPB) * CPB;
  static_assert(DEPTH >= 2, "at least one chunk in flight");

  __amdgpu_buffer_rsrc_t w_rs, s_rs;  // descriptors of the sibling being issued
  const GemvArgs *args;
  int K, N, KB, groups, wave, pitch, last_chunk;
  const float *a_lds;  // the wave's activation stage: [MT][pitch], block j at 32 j
  float *s_lds;        // the wave's scale hand-over area: 64 * VEC floats (VEC >= 8)
  int lane;
  uint32_t s_off[G::kScaleLoads];  // coalesced S column offsets for the block being issued
  float *slots;        // parked sums: slot q at slots + q * 4 * MT * TW (+ wave * MT * TW)
  int it, ig;          // tile (over all siblings) and group of the next block to issue
  int isib, itile;     // that tile's sibling and its tile within the sibling
  int cg, cslot;       // group of the block being used, next free slot
  uint32_t col_off[G::kPieces];  // lane byte offsets (per piece) into a W row for the block being issued
  int b_issue;         // that block
  uint32_t w[kDepth][CR][NWD];
  float s[kDepth][VEC];
  float part[MT][VEC];
  float acc[MT][VEC];

  // Issues chunk c0 + U (c0 a multiple of kUnroll).
  template <int U>
  __device__ __forceinline__ void issue(int c0) {
    constexpr int BUF = U % kDepth, H = U % CPB;
    if constexpr (H == 0) {
      w_rs = buffer_rsrc(args->W[isib], (uint32_t)K * (uint32_t)N);
      s_rs = buffer_rsrc(args->S[isib], (uint32_t)KB * (uint32_t)N * 4u);
      // Columns past N (ragged last tile) load column 0 instead; blocks past
      // KB (in the last group of K) load row K-1 with zero activations.
#pragma unroll
      for (int q = 0; q < G::kPieces; ++q) {
        const int col = itile * TW + G::col(lane, q * G::kPieceCols);
        col_off[q] = col < N ? (uint32_t)col : 0u;
      }
      if constexpr (G::kSwizzleScales) {
#pragma unroll
        for (int i = 0; i < G::kScaleLoads; ++i) {
          const int c = itile * TW + 256 * i + 4 * lane;
          s_off[i] = c < N ? (uint32_t)c * 4u : 0u;
        }
      }
      b_issue = kWaves * ig + wave;
    }
    const int row0 = b_issue * kBlock + H * CR;
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      // Rows past K re-read row K-1: their staged activation is zero ("Bounds").
      const int row = min(row0 + i, K - 1);
      load_w<VEC>(w_rs, col_off, (uint32_t)row * (uint32_t)N, w[BUF][i]);
    }
    if constexpr (H == CPB - 1) {
      const uint32_t s_row = (uint32_t)min(b_issue, KB - 1) * (uint32_t)N * 4u;
      if constexpr (G::kSwizzleScales) {
#pragma unroll
        for (int i = 0; i < G::kScaleLoads; ++i) {
          const v4u x = __builtin_amdgcn_raw_buffer_load_b128(s_rs, s_off[i], s_row, kStreamPolicy);
          s[BUF][4 * i] = __uint_as_float(x.x);
          s[BUF][4 * i + 1] = __uint_as_float(x.y);
          s[BUF][4 * i + 2] = __uint_as_float(x.z);
          s[BUF][4 * i + 3] = __uint_as_float(x.w);
        }
      } else {
        load_s<VEC>(s_rs, col_off[0] * 4u, s_row, s[BUF]);
      }
      if (++ig == groups) {
        ig = 0;
        ++it;
        if (++itile == args->tiles_per) {
          itile = 0;
          ++isib;
        }
      }
    }
  }

  // Converts and accumulates chunk c0 + U.
  template <int U>
  __device__ __forceinline__ void consume(int c0) {
    constexpr int BUF = U % kDepth, H = U % CPB;
    const int kl = kBlock * ((c0 + U) / CPB) + H * CR;
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
      // Keep converts next to their FMAs: hoisted, a chunk's converted bytes
      // would all be live at once.
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (H == CPB - 1) {
      float sc[VEC];
      if constexpr (G::kSwizzleScales) {
        // Coalesced layout -> owner layout, through the wave's LDS area.
#pragma unroll
        for (int i = 0; i < G::kScaleLoads; ++i)
          *reinterpret_cast<v4f *>(&s_lds[256 * i + 4 * lane]) =
              v4f{s[BUF][4 * i], s[BUF][4 * i + 1], s[BUF][4 * i + 2], s[BUF][4 * i + 3]};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
          const v4f x = *reinterpret_cast<const v4f *>(&s_lds[G::col(lane, 4 * i)]);
          sc[4 * i] = x.x;
          sc[4 * i + 1] = x.y;
          sc[4 * i + 2] = x.z;
          sc[4 * i + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) sc[v] = s[BUF][v];
      }
      // "Factoring out the scale": one multiply per block and column.
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[m][v] = fmaf(part[m][v], sc[v], acc[m][v]);
      // End of this tile's share of the run (or of the run): park the sums.
      if (++cg == groups || c0 + U == last_chunk) {
        cg = 0;
        float *dst = slots + (size_t)cslot * (kWaves * MT * TW) + wave * (MT * TW);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            dst[m * TW + G::col(lane, v)] = acc[m][v];
            acc[m][v] = 0.f;
          }
        ++cslot;
      }
    }
  }

  // Step U of a group of R chunks starting at c0: chunk c0 + U + kDepth - 1
  // goes in flight (if it is one of the R), chunk c0 + U is used.  The
  // scheduling barriers keep the compiler from sinking the loads down to their
  // uses (which it otherwise does to save registers).
  template <int U, int R>
  __device__ __forceinline__ void step(int c0) {
    if constexpr (U + kDepth - 1 < R) issue<U + kDepth - 1>(c0);
    __builtin_amdgcn_sched_barrier(0);
    consume<U>(c0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Uses chunks c0 .. c0+R-1 (the first kDepth-1 of them already issued).
  template <int R>
  __device__ __forceinline__ void finish(int c0) {
    StaticFor<0, R>::run([&](auto u_) { step<decltype(u_)::value, R>(c0); });
  }

  // All R chunks of a short run: issue them all, stage, use them.
  template <int R, class Stage>
  __device__ __forceinline__ void whole(Stage &&stage) {
    StaticFor<0, R>::run([&](auto u_) { issue<decltype(u_)::value>(0); });
    stage();
    __builtin_amdgcn_sched_barrier(0);
    StaticFor<0, R>::run([&](auto u_) { consume<decltype(u_)::value>(0); });
  }

  // Streams chunks [0, nchunk) when nchunk = kDepth - 1 + REM (mod kUnroll).
  template <int REM, class Stage>
  __device__ __forceinline__ void run_rem(int nchunk, Stage &&stage) {
    StaticFor<0, kDepth - 1>::run([&](auto u_) { issue<decltype(u_)::value>(0); });
    stage();
    int c0 = 0;
    for (; c0 + kUnroll + kDepth - 2 < nchunk; c0 += kUnroll)
      StaticFor<0, kUnroll>::run([&](auto u_) { step<decltype(u_)::value, kUnroll + kDepth>(c0); });
    finish<kDepth - 1 + REM>(c0);  // exactly kDepth - 1 + REM chunks remain
  }

  // Streams chunks [0, nchunk), nchunk >= 1.  `stage` writes the wave's
  // activations to LDS; it runs after the first loads of W are issued (their
  // values were loaded into registers before, so waiting for them does not
  // drain W).  The kUnroll remainder classes are separate paths chosen before
  // any load is issued: a branch taken after the loop, with loads in flight,
  // makes the register allocator keep every path's buffers apart.
  template <class Stage>
  __device__ __forceinline__ void run(int nchunk, Stage &&stage) {
    last_chunk = nchunk - 1;
    if (nchunk < kDepth - 1) {
      StaticSwitch<1, kDepth - 1>::run(nchunk, [&](auto r_) { whole<decltype(r_)::value>(stage); });
      return;
    }
    StaticSwitch<0, kUnroll>::run((nchunk - (kDepth - 1)) % kUnroll,
                                  [&](auto r_) { run_rem<decltype(r_)::value>(nchunk, stage); });
  }
};

// Chunks per wave in the load pipeline (kDepth - 1 of them in flight).
template <int VEC, int MT>
constexpr int kStreamDepth = 4;

// Stores outputs 4*o4 .. 4*o4+3 of row chunk m0's tile (sibling sib, tile
// tis within the sibling), [MT][TW] in tile order, through the epilogue of
// "dot and tensor cores", section "The fused epilogue": each output x is
// written as y = alpha * x + corr[row] * C[row, n] (the second term only with
// row factors), so with alpha 1 and no row factors it is a plain store of x.
// Columns past N and rows past M are not stored.  The arguments are read
// once into registers: read per element, the compiler reloads them after
// every store (it cannot rule out that a store changes them).
template <int TW>
__device__ __forceinline__ void store_quad(const GemvArgs &p, int sib, int tis, int m0, int o4, v4f x) {
  float *const cs = p.C[sib];
  const float alpha = p.alpha;
  const float *const corr = p.corr;
  const int N = p.N, M = p.M;
  const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int o = 4 * o4 + e;
    const int m = o / TW;
    const int n = tis * TW + (o - m * TW);
    if (n < N && m0 + m < M) {
      float *c = cs + (size_t)(m0 + m) * N + n;
      float y = alpha * xs[e];
      if (corr != nullptr) y = fmaf(corr[m0 + m], *c, y);
      *c = y;
    }
  }
}

// Cache policy of the split-K partials' stores and loads: device-coherent
// (sc1), as for agent-scope atomic loads and stores.  A store is acknowledged
// once it is performed at the device's coherence point; a load misses in the
// per-XCD caches and reads that point.
constexpr int kDeviceCoherent = 16;
// When all contributors of a tile run on one XCD: stores with the default
// policy (acknowledged once they are in the XCD's L2) and loads with sc0
// (they miss in the CU's L1 and read the L2).
constexpr int kXcdStore = 0;
constexpr int kXcdLoad = 1;
// Contributors summed by one pairwise tree in a split-K combine.
constexpr int kCombineGroup = 8;
// Outputs 4*o4 .. 4*o4+3 of contributor c's partial (stride `per` floats).
template <int AUX>
__device__ __forceinline__ v4f load_partial_quad(__amdgpu_buffer_rsrc_t rs, int c, int o4, int per) {
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rs, ((uint32_t)c * (uint32_t)per + 4u * (uint32_t)o4) * 4u, 0, AUX);
  return v4f{__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
}

// Workgroup that owns unit u when units are dealt in runs of upw (+1 for the
// first rem workgroups).
__device__ __forceinline__ int wg_of_unit(int u, int upw, int rem) {
  const int big = rem * (upw + 1);
  return u < big ? u / (upw + 1) : rem + (u - big) / upw;
}

// The run (in tile-major order) that workgroup b streams.  The dispatcher
// sends workgroup b to XCD b % 8 (kXcds).  With band_runs > 0 (every tile cut
// into band_runs runs, one per workgroup), the runs are taken K-range-major
// and each XCD gets a contiguous stretch of that order: its workgroups read
// neighbouring column tiles of the same rows together, so the 128-byte lines
// that two tiles share when a row is not a multiple of 128 bytes are fetched
// into one L2 once.  Which run a workgroup takes never changes a result.
//
// With xcd_runs > 0 (every tile cut into xcd_runs runs, and the number of
// tiles a multiple of 8), all runs of tile t go to the workgroups b with
// b % 8 == t % 8, which the dispatcher places on one XCD: a tile's partials
// are then written and read in that XCD's L2.
__device__ __forceinline__ int run_of_block(const GemvArgs &p, int b) {
  if (p.xcd_runs > 0) {
    const int R = p.xcd_runs, x = b % kXcds, k = b / kXcds;
    return (kXcds * (k / R) + x) * R + k % R;
  }
  if (p.band_runs <= 0) return b;
  const int x = b % kXcds, k = b / kXcds;
  const int q = p.n_wg / kXcds, rr = p.n_wg % kXcds;
  const int i = x * q + min(x, rr) + k;
  const int r = i / p.n_tiles, t = i - r * p.n_tiles;
  return t * p.band_runs + r;
}

// The combine of the tiles this workgroup completed (bit q of last_mask:
// segment q), reading the partials with cache policy AUX.  A tile in
// stray_mask gets NaN outputs.  Re-arms the counters.
template <int VEC, int MT, int AUX>
__device__ __forceinline__ void combine_tiles(const GemvArgs &p, uint32_t last_mask, uint32_t stray_mask, const int *seg_lo,
                                              const int *seg_hi, int nseg, int t_first, int mc, int m0, int tid) {
  using G = Geo<VEC>;
  constexpr int TW = G::kTileCols;
  constexpr int kQuads = MT * TW / 4;
  auto rearm = [&](int t) {
    if (tid != 0) return;
    uint32_t *cnt = &p.counters[(mc * p.n_tiles + t) * kCounterStride];
    if constexpr (AUX == kXcdLoad)
      __hip_atomic_store(reinterpret_cast<uint64_t *>(cnt), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int q = 0; q < nseg; ++q) {
    if (!(last_mask & (1u << q))) continue;
    const int t = t_first + q;
    const int i0 = seg_lo[q];
    const int contributors = seg_hi[q] - i0 + 1;
    const int sib = t / p.tiles_per;
    if (stray_mask & (1u << q)) {
      const float nan = __builtin_nanf("");
      for (int o4 = tid; o4 < kQuads; o4 += kThreads) store_quad<TW>(p, sib, t - sib * p.tiles_per, m0, o4, v4f{nan, nan, nan, nan});
      rearm(t);
      continue;
    }
    // Each thread owns four adjacent outputs.  The summation order is the
    // same for every instance: a pairwise tree over each group of eight
    // contributors (absent ones are zero), then the group sums in K order
    // through a cascade (SumCascade).  The partials are read with 16-byte
    // device-coherent loads, two groups per round trip; the descriptor ends
    // at the last contributor, so reads past it return zero.
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.partial + (size_t)(mc * p.n_tiles + t) * p.cmax * (MT * TW),
                                                  (uint32_t)contributors * (MT * TW * 4));
    if constexpr (VEC >= 8) {
      // Up to four contributors (the large decode shapes at these widths):
      // one pairwise tree, plus the zero of the absent half of the group of
      // eight and of the cascade's empty levels, which is what the general
      // path below returns for them, bit for bit (-0 comes out +0).  Only
      // the wide instances carry this path; the narrow ones keep their code
      // as it was, which measured faster for them.
      if (contributors <= 4) {
        for (int o4 = tid; o4 < kQuads; o4 += kThreads) {
          v4f v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = load_partial_quad<AUX>(rs, i, o4, MT * TW);
          store_quad<TW>(p, sib, t - sib * p.tiles_per, m0, o4, ((v[0] + v[1]) + (v[2] + v[3])) + 0.f);
        }
        rearm(t);
        continue;
      }
    }
    for (int o4 = tid; o4 < kQuads; o4 += kThreads) {
      SumCascade<float, 4> total;
      for (int c = 0; c < contributors; c += 2 * kCombineGroup) {
        v4f v[2 * kCombineGroup];
#pragma unroll
        for (int i = 0; i < kCombineGroup; ++i) v[i] = load_partial_quad<AUX>(rs, c + i, o4, MT * TW);
        const bool second = contributors - c > kCombineGroup;
        if (second) {
#pragma unroll
          for (int i = kCombineGroup; i < 2 * kCombineGroup; ++i) v[i] = load_partial_quad<AUX>(rs, c + i, o4, MT * TW);
        }
#pragma unroll
        for (int g = 0; g < (second ? 2 : 1) * kCombineGroup; g += kCombineGroup) {
          const v4f *y = &v[g];
          const v4f s = ((y[0] + y[1]) + (y[2] + y[3])) + ((y[4] + y[5]) + (y[6] + y[7]));
          const float x[4] = {s.x, s.y, s.z, s.w};
          total.add(x);
        }
      }
      float sum[4];
      total.result(sum);
      store_quad<TW>(p, sib, t - sib * p.tiles_per, m0, o4, v4f{sum[0], sum[1], sum[2], sum[3]});
    }
    rearm(t);
  }
}

template <int VEC, int MT>
__global__ __launch_bounds__(kThreads) void q8_gemv_kernel(GemvArgs p) {
  using G = Geo<VEC>;
  constexpr int TW = G::kTileCols;
  constexpr int CPB = kBlock / kChunkRowsOf<VEC, MT>;

  extern __shared__ __attribute__((aligned(16))) float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = run_of_block(p, blockIdx.x);
  const int mc = blockIdx.y;
  const int m0 = mc * MT;
  const int u_begin = wg * p.upw + min(wg, p.rem);
  const int count = p.upw + (wg < p.rem ? 1 : 0);  // blocks per wave
  const int t_first = u_begin / p.groups;
  const int g_first = u_begin - t_first * p.groups;
  const int t_last = (u_begin + count - 1) / p.groups;
  float *stage = lds + wave * MT * p.pitch;           // this wave's activations
  float *s_area = lds + kWaves * MT * p.pitch;        // [wave][64 * VEC] scale hand-over (VEC >= 8)
  float *slots = s_area + (G::kSwizzleScales ? kWaves * 64 * VEC : 0);  // [segment][wave][m][column] sums
  __shared__ uint32_t last_mask;

  WaveStream<VEC, MT, kStreamDepth<VEC, MT>> st;
  st.args = &p;
  st.K = p.K;
  st.N = p.N;
  st.KB = p.KB;
  st.groups = p.groups;
  st.wave = wave;
  st.pitch = p.pitch;
  st.a_lds = stage;
  st.slots = slots;
  st.s_lds = s_area + wave * 64 * VEC;
  st.lane = lane;
  st.it = t_first;
  st.isib = t_first / p.tiles_per;
  st.itile = t_first - st.isib * p.tiles_per;
  st.ig = g_first;
  st.cg = g_first;
  st.cslot = 0;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int v = 0; v < VEC; ++v) st.acc[m][v] = 0.f;

  // Activations of this wave's blocks: element e = (m * count + j) * 32 + r of
  // the stage is A[m0 + m, 32 * b_j + r] with b_j = 4 * g_j + wave, g_j the
  // group of unit u_begin + j; zero past K or M.  Loaded before the first W
  // chunks so that waiting for them does not drain W.
  const int per_m = count * kBlock;
  float sv[kStageRegs];
#pragma unroll
  for (int q = 0; q < kStageRegs; ++q) {
    const int e = lane + 64 * q;
    const int m = e / per_m;
    const int rr = e - m * per_m;
    const int u = u_begin + (rr >> 5);
    const int g = u - (u / p.groups) * p.groups;
    const int k = kBlock * (kWaves * g + wave) + (rr & 31);
    const bool ok = m < MT && m0 + m < p.M && k < p.K;
    sv[q] = ok ? p.A[(size_t)(m0 + m) * p.K + k] : 0.f;
  }
  // Contributors [seg_lo, seg_hi] (workgroups) of each tile the run touches,
  // worked out by wave 0 while its first loads are in flight: the epilogue
  // then starts without integer divisions.
  __shared__ int seg_lo[kMaxSegments], seg_hi[kMaxSegments];
  const int nseg = t_last - t_first + 1;
  st.run(count * CPB, [&]() {
#pragma unroll
    for (int q = 0; q < kStageRegs; ++q) {
      const int e = lane + 64 * q;
      const int m = e / per_m;
      if (m < MT) stage[m * p.pitch + (e - m * per_m)] = sv[q];
    }
    if (wave == 0 && lane < nseg) {
      const int t = t_first + lane;
      seg_lo[lane] = wg_of_unit(t * p.groups, p.upw, p.rem);
      seg_hi[lane] = wg_of_unit(t * p.groups + p.groups - 1, p.upw, p.rem);
    }
  });
  lds_barrier();

  // Finish every tile of the run: the four waves' sums, four adjacent outputs
  // per thread, then a direct store (the run owns the whole tile) or a
  // published partial (one 16-byte store per thread: device-coherent, or
  // into the XCD's L2 when the tile's runs are all on this XCD).
  constexpr int kQuads = MT * TW / 4;
  const bool local = p.xcd_runs > 0;
  bool any_partial = false;
  for (int q = 0; q < nseg; ++q) {
    const int t = t_first + q;
    const int i0 = seg_lo[q], i1 = seg_hi[q];
    const v4f *sl = reinterpret_cast<const v4f *>(slots + (size_t)q * (kWaves * MT * TW));
    any_partial |= i0 != i1;
    if (i0 == i1) {
      const int sib = t / p.tiles_per;
      for (int o4 = tid; o4 < kQuads; o4 += kThreads) {
        const v4f x = (sl[o4] + sl[kQuads + o4]) + (sl[2 * kQuads + o4] + sl[3 * kQuads + o4]);
        store_quad<TW>(p, sib, t - sib * p.tiles_per, m0, o4, x);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc(p.partial + ((size_t)(mc * p.n_tiles + t) * p.cmax + (wg - i0)) * (MT * TW), MT * TW * 4);
      for (int o4 = tid; o4 < kQuads; o4 += kThreads) {
        const v4f x = (sl[o4] + sl[kQuads + o4]) + (sl[2 * kQuads + o4] + sl[3 * kQuads + o4]);
        const v4u u = v4u{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)};
        if (local)
          __builtin_amdgcn_raw_buffer_store_b128(u, rs, (uint32_t)o4 * 16u, 0, kXcdStore);
        else
          __builtin_amdgcn_raw_buffer_store_b128(u, rs, (uint32_t)o4 * 16u, 0, kDeviceCoherent);
      }
    }
  }
  if (!any_partial) return;

  // Count each shared tile's contribution once this workgroup's partials are
  // performed where the reader will look (s_waitcnt: device-coherent stores
  // are acknowledged only once they have reached the device's coherence
  // point, the others once they are in the XCD's L2): lane q of wave 0 bumps
  // segment q's counter, all in one go.  The last of a tile's contributors
  // combines it.  With the tile's runs on one XCD the counter also records
  // where each contributor ran; a tile with a contributor on another XCD (the
  // dispatcher did not place the workgroups as expected) cannot be read from
  // this L2, and its outputs are written as NaN instead of a wrong sum.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ uint32_t stray_mask;
  if (wave == 0) {
    bool last = false, stray = false;
    if (lane < nseg) {
      const int t = t_first + lane;
      const int i0 = seg_lo[lane], i1 = seg_hi[lane];
      if (i0 != i1) {
        uint32_t *cnt = &p.counters[(mc * p.n_tiles + t) * kCounterStride];
        if (local) {
          const uint32_t x = xcd_id() ^ (p.xcc_skew != 0 ? (uint32_t)(blockIdx.x / kXcds) & 1u : 0u);
          const uint64_t inc = xcd_increment(x);
          const uint64_t prev = __hip_atomic_fetch_add(reinterpret_cast<uint64_t *>(cnt), inc, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t n = (uint64_t)(i1 - i0 + 1);
          last = xcd_count_done(prev, n);
          stray = last && !xcd_all_here(prev, x, n);
        } else {
          const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = prev == (uint32_t)(i1 - i0);
        }
      }
    }
    const uint64_t mask = __ballot(last);
    const uint64_t smask = __ballot(stray);
    if (lane == 0) {
      last_mask = (uint32_t)mask;
      stray_mask = (uint32_t)smask;
    }
  }
  __syncthreads();
  if (last_mask == 0) return;
  if (local)
    combine_tiles<VEC, MT, kXcdLoad>(p, last_mask, stray_mask, seg_lo, seg_hi, nseg, t_first, mc, m0, tid);
  else
    combine_tiles<VEC, MT, kDeviceCoherent>(p, last_mask, stray_mask, seg_lo, seg_hi, nseg, t_first, mc, m0, tid);
}

typedef void (*GemvKernel)(GemvArgs);

// The instance (VEC, m_tile), or nullptr if it is not compiled (VEC * m_tile > 32).
template <int VEC>
GemvKernel pick_m_tile(int m_tile) {
  auto inst = [](auto mt_) -> GemvKernel {
    constexpr int MT = decltype(mt_)::value;
    if constexpr (MT * VEC <= 32) return q8_gemv_kernel<VEC, MT>;
    return nullptr;
  };
  switch (m_tile) {
    case 1: return inst(std::integral_constant<int, 1>{});
    case 2: return inst(std::integral_constant<int, 2>{});
    case 4: return inst(std::integral_constant<int, 4>{});
    case 8: return inst(std::integral_constant<int, 8>{});
    default: return nullptr;
  }
}

}  // namespace

// Per-VEC instance tables, one translation unit each.
GemvKernel gemv_kernel_v16(int m_tile);
GemvKernel gemv_kernel_v8(int m_tile);
GemvKernel gemv_kernel_v4(int m_tile);
GemvKernel gemv_kernel_v2(int m_tile);
GemvKernel gemv_kernel_v1(int m_tile);

}  // namespace q8
