// Q8_0 product for a few activation rows (2 <= M <= 64) on the matrix cores:
// C[m,n] = sum_k A[m,k] * W[k,n] * S[k/32, n], reading W and S once for all
// rows.
//
// Operation: "Q8_0 matvec" page, sections "The tensors" (definition),
// "Factoring out the scale" (the scale multiplies each block's unscaled
// partial once per block and column) and "Bounds" (ragged N and K are
// masked).  At M rows the per-row FMA path costs M multiply-adds per weight
// and runs out of vector ALU well before HBM bandwidth; here the contraction
// goes to v_mfma_f32_16x16x32_bf16, whose k-slice of 32 is exactly one Q8_0
// block, so the block's unscaled partial comes out of the matrix core and is
// scaled once per block and column, as the page prescribes.
//
// Precision.  "dot and tensor cores" (section "Hardware paths") notes that
// tensor-core f32 paths round their operands to 16 bits; that alone would
// miss a 1e-5 relative bound.  W is exact in bf16 (|w| <= 128 has at most 8
// significant bits).  A is split exactly into three bf16 parts,
// a = hi + mid + lo + r with |r| <= 2^-24 |a| (each part takes the rounding
// of the remainder so far; every subtraction is exact in f32), and every
// block takes three MFMAs, one per part, into the same f32 accumulator.
//
// Work decomposition:
//   * A workgroup (eight wave64s) owns a tile of 512 columns and a
//     contiguous range of K blocks (a split); the splits of a tile are
//     combined as in the matvec: device-coherent partials, an arrival
//     counter, and the last arrival sums the splits in K order.
//   * Per block the workgroup loads W[32 rows, 512 columns] into LDS, two
//     blocks ahead in registers, with 16-byte loads (a wave instruction reads
//     two whole 512-byte row segments).  When N or W's address is not a
//     multiple of 16 ("Bounds": N need not fill the tiles) the loads are 8
//     bytes (one 512-byte row segment per instruction) or 4 bytes (half a
//     segment), whichever both allow.  A's block (M x 32) is split into
//     its three bf16 parts in LDS once per workgroup.
//   * Wave w computes columns [64w, 64w + 64) as four 16x16 output tiles per
//     16 rows of A.  For the B operand a lane needs eight consecutive k of one
//     column; it reads four columns x eight rows as dwords from LDS and
//     converts the bytes straight into bf16 pairs in k order (a byte-selecting
//     convert and a byte permute), so the transpose costs nothing extra.
//     Lane l of tile i supplies column 4(l%16) + i of the wave's 64, which is
//     the column its outputs belong to.
//   * Eight waves of at most 128 registers (up to 16 rows) let two
//     workgroups share a CU with four waves per SIMD, so one wave's convert
//     or wait overlaps another's matrix ops.
#include <type_traits>

#include "q8_common.h"
#include "q8_sum.h"
#include "q8_xcd.h"

namespace q8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));

constexpr int kGemmCols = kGemmTileCols;   // columns per workgroup tile
constexpr int kGW = kGemmWaves;            // waves per workgroup
constexpr int kGThreads = 64 * kGW;
constexpr int kWaveCols = kGemmCols / kGW; // columns per wave (64)
constexpr int kWaveTiles = kWaveCols / 16; // 16-column output tiles per wave
constexpr int kWaveGroups = kWaveCols / 64;  // groups of 64 columns per wave
constexpr int kWPitch = kGemmCols + 16;    // LDS row pitch of a W block, bytes (16-byte aligned rows)
// LDS row pitch of an A block part, bf16 (96 bytes).  Measured with
// SQ_LDS_BANK_CONFLICT at 64 rows: 8.7 M conflict cycles per launch at 80
// bytes, 112 and 144 bytes, 3.2 M at 96 bytes (the pitch the dense kernels'
// part tiles also use).
constexpr int kAPitch = 48;
constexpr int kDepthG = 2;                 // W blocks held in registers ahead of the one in LDS
constexpr int kStreamPolicyG = 2;          // non-temporal: W and S are read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even bf16 of (x, y) packed into one dword, x in the low
// half (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, y}, bf16x2));
}

// Two signed bytes (byte `i` of words x0 and x1) as a pair of bf16 in one
// dword, x0's in the low half.  Exact: the f32 of a byte has 16 zero low bits.
__device__ __forceinline__ uint32_t byte_pair_bf16(uint32_t x0, uint32_t x1, int i) {
  const float f0 = static_cast<float>(static_cast<int8_t>(x0 >> (8 * i)));
  const float f1 = static_cast<float>(static_cast<int8_t>(x1 >> (8 * i)));
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// Makes this workgroup's LDS writes visible to its other waves without
// waiting for outstanding global loads (a plain __syncthreads would drain the
// prefetch ring every block).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int B, int E>
struct SFor {
  template <class F>
  __device__ __forceinline__ static void run(F &&f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>{});
      SFor<B + 1, E>::run(f);
    }
  }
};

// RT: 16-row tiles of A (M <= 16 * RT).
// WW: bytes per W load (16, 8 or 4); N and W's address are multiples of it.
template <int RT, int WW>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(RT == 1 ? 4 : 2))) void q8_gemm_kernel(GemmArgs p) {
  static_assert(WW == 16 || WW == 8 || WW == 4, "16-, 8- or 4-byte W loads");
  using WVec = std::conditional_t<WW == 16, u4, std::conditional_t<WW == 8, u2, uint32_t>>;
  // A tile row of W is kGemmCols / WW lanes' pieces.  One load instruction of
  // a wave covers kRowsPerLoad rows (two for 16-byte loads) or 64 lanes'
  // pieces of one row; kSides loads cover a row side by side (two for 4-byte
  // loads).  kWLoads loads per lane bring in the wave's rows of a block.
  constexpr int kLanesPerRow = kGemmCols / WW;
  constexpr int kPieceLanes = kLanesPerRow < 64 ? kLanesPerRow : 64;
  constexpr int kSides = kLanesPerRow / kPieceLanes;
  constexpr int kRowsPerLoad = 64 / kPieceLanes;
  constexpr int kWaveRows = kBlock / kGW;  // rows of a block per wave
  constexpr int kWLoads = kWaveRows * kSides / kRowsPerLoad;
  // Two LDS buffers: block j is staged in buffer j & 1, so staging the next
  // block never overwrites the one other waves may still be reading, and one
  // barrier per block suffices.
  __shared__ __attribute__((aligned(16))) int8_t w_lds_buf[2][kBlock * kWPitch];
  __shared__ __attribute__((aligned(16))) uint16_t a_lds_buf[2][3][16 * RT * kAPitch];
  __shared__ uint32_t last_flag, stray_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Rows beyond 16*RT would run as further passes (grid z), each with its own
  // rows of A and C, partials and counters, reading W again; with RT chosen
  // by gemm_row_tiles every launch up to kGemmMaxRows rows is one pass.
  constexpr int kTileElems = 16 * RT * kGemmCols;
  {
    const int pass = blockIdx.z;
    p.A += (size_t)pass * 16 * RT * p.K;
    p.C += (size_t)pass * 16 * RT * p.N;
    p.M = min(16 * RT, p.M - pass * 16 * RT);
    p.partial += (size_t)pass * p.n_tiles * p.splits * kTileElems;
    p.counters += pass * p.n_tiles * kCounterStride;
  }
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int n0 = tile * kGemmCols;
  const int b_begin = split * p.bps;
  const int b_end = min(p.KB, b_begin + p.bps);
  const int nb = b_end - b_begin;  // >= 1 (the host never launches an empty split)

  // Every prefetch is issued unconditionally (a conditional load makes the
  // compiler wait for all outstanding loads); the ones past this split's last
  // block go through descriptors with no records, which return zeros without
  // touching memory.
  const uint32_t w_bytes = (uint32_t)p.K * (uint32_t)p.N;
  const uint32_t s_bytes = (uint32_t)p.KB * (uint32_t)p.N * 4u;
  const uint32_t a_bytes = (uint32_t)p.M * (uint32_t)p.K * 4u;

  // This thread's WW-byte piece of a W block in load i: row kWaveRows*wave
  // + kRowsPerLoad*(i/kSides) + lrow of the block, columns n0 + w_col(i % kSides)
  // .. +WW-1.  The load's first row goes into the wave-uniform scalar offset,
  // clamped to K - 1; with 16-byte loads the upper half-wave steps one row
  // further per lane, only while that row exists.  Columns past N (the
  // ragged last tile; N is a multiple of WW) read column 0, rows past K
  // re-read a row of W; their activations are zero, and outputs past N are
  // not stored.
  const int lrow = lane / kPieceLanes;  // 0, or 1 for the upper half-wave of 16-byte loads
  auto w_col = [&](int side) { return WW * (kPieceLanes * side + lane % kPieceLanes); };
  uint32_t w_voff[kSides];
#pragma unroll
  for (int v = 0; v < kSides; ++v) {
    const int wcol = n0 + w_col(v);
    w_voff[v] = wcol < p.N ? (uint32_t)wcol : 0u;
  }
  auto load_w = [&](int b, bool live, WVec (&x)[kWLoads]) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(p.W, live ? w_bytes : 0u);
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
      const int r = min(b * kBlock + kWaveRows * wave + kRowsPerLoad * (i / kSides), p.K - 1);
      const uint32_t voff = w_voff[i % kSides] + (lrow != 0 && r + 1 < p.K ? (uint32_t)p.N : 0u);
      const uint32_t soff = (uint32_t)r * (uint32_t)p.N;
      if constexpr (WW == 16)
        x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kStreamPolicyG);
      else if constexpr (WW == 8)
        x[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kStreamPolicyG);
      else
        x[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kStreamPolicyG);
    }
  };

  // Scales of this lane's output columns: group q of the wave, columns
  // 64q + 4(l%16) .. +3 of the wave's 128.
  const int c16 = lane & 15;
  const int g4 = lane >> 4;
  uint32_t s_voff[kWaveGroups];
#pragma unroll
  for (int q = 0; q < kWaveGroups; ++q) {
    const int c = n0 + kWaveCols * wave + 64 * q + 4 * c16;
    s_voff[q] = c < p.N ? (uint32_t)c * 4u : 0u;
  }

  // Activation block b: pairs of adjacent k, pair i = tid + kGThreads * j of
  // the 16*RT x 32 block (16 pairs per row), so that one convert rounds two
  // elements.  With 16 rows there are 256 pairs: waves 4-7 stage none.
  constexpr int kAPairs = (16 * RT * kBlock / 2 + kGThreads - 1) / kGThreads;  // per thread
  constexpr int kAElems = 2 * kAPairs;
  const bool a_stager = 16 * RT * kBlock / 2 >= kGThreads || tid < 16 * RT * kBlock / 2;
  // Element h of pair j: row i/16, k = 2 (i % 16) + h.  Elements past M or K
  // load element 0; they are replaced by zero when the block is staged (not
  // here, which would wait for the load at once).  The row test and the row's
  // offset are fixed for the whole loop; the tests combine with & so that
  // they stay selects (a short-circuit test became branches around the loads).
  bool a_row_ok[kAPairs];
  int a_kk[kAPairs];
  uint32_t a_row_off[kAPairs];
#pragma unroll
  for (int j = 0; j < kAPairs; ++j) {
    const int i = tid + kGThreads * j;
    a_row_ok[j] = a_stager & ((i >> 4) < p.M);
    a_kk[j] = 2 * (i & 15);
    a_row_off[j] = (uint32_t)(i >> 4) * (uint32_t)p.K + (uint32_t)a_kk[j];
  }
  auto a_ok = [&](int b, int j, int h) { return a_row_ok[j] & (b * kBlock + a_kk[j] + h < p.K); };
  auto load_a = [&](int b, bool live, float (&v)[kAElems]) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(p.A, live ? a_bytes : 0u);
#pragma unroll
    for (int j = 0; j < kAPairs; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = a_ok(b, j, h) ? (a_row_off[j] + (uint32_t)(b * kBlock + h)) * 4u : 0u;
        v[2 * j + h] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0u, 0));
      }
  };

  f4 acc[kWaveTiles][RT];
#pragma unroll
  for (int t = 0; t < kWaveTiles; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = f4{0.f, 0.f, 0.f, 0.f};

  auto load_s = [&](int b, bool live, u4 (&sv)[kWaveGroups]) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(p.S, live ? s_bytes : 0u);
    const uint32_t soff = (uint32_t)min(b, p.KB - 1) * (uint32_t)p.N * 4u;
#pragma unroll
    for (int q = 0; q < kWaveGroups; ++q) sv[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, s_voff[q], soff, kStreamPolicyG);
  };

  // Register ring: W, A and S of blocks b_begin + j for j < kDepthG are in flight.
  WVec wring[kDepthG][kWLoads];
  float aring[kDepthG][kAElems];
  u4 sring[kDepthG][kWaveGroups];
#pragma unroll
  for (int d = 0; d < kDepthG; ++d) {
    load_w(b_begin + d, d < nb, wring[d]);
    load_a(b_begin + d, d < nb, aring[d]);
    load_s(b_begin + d, d < nb, sring[d]);
  }

  // Block j from ring slot D: stage it in LDS, refill the slot, multiply.
  auto process = [&](auto d_, auto refill_, int j) {
    constexpr int D = decltype(d_)::value;
    constexpr bool REFILL = decltype(refill_)::value;
      const int b = b_begin + j;
      // Scales of this block for the lane's eight output columns.
      const u4 (&sv)[kWaveGroups] = sring[D];
      // Block j into its LDS buffer.  The last reader of that buffer was block
      // j - 2, which every wave finished before the barrier of block j - 1.
      int8_t *w_lds = w_lds_buf[j & 1];
      uint16_t(*a_lds)[16 * RT * kAPitch] = a_lds_buf[j & 1];
#pragma unroll
      for (int i = 0; i < kWLoads; ++i) {
        const int row = kWaveRows * wave + kRowsPerLoad * (i / kSides) + lrow;
        *reinterpret_cast<WVec *>(&w_lds[row * kWPitch + w_col(i % kSides)]) = wring[D][i];
      }
      // A's three parts: each part is the rounding of what the parts before
      // left, and each remainder is exact in f32.
      if (a_stager) {
#pragma unroll
        for (int jj = 0; jj < kAPairs; ++jj) {
          const int i = tid + kGThreads * jj;
          const int m = i >> 4;
          const int k = 2 * (i & 15);
          float x = a_ok(b, jj, 0) ? aring[D][2 * jj] : 0.f;
          float y = a_ok(b, jj, 1) ? aring[D][2 * jj + 1] : 0.f;
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const uint32_t u = pk_bf16(x, y);
            *reinterpret_cast<uint32_t *>(&a_lds[q][m * kAPitch + k]) = u;
            if (q < 2) {
              x -= __uint_as_float(u << 16);
              y -= __uint_as_float(u & 0xffff0000u);
            }
          }
        }
      }
      lds_barrier();
      // Refill this ring slot with block j + kDepthG (past the split's end:
      // loads that return zeros, issued anyway to keep the pattern fixed).
      if constexpr (REFILL) {
        load_w(b + kDepthG, j + kDepthG < nb, wring[D]);
        load_a(b + kDepthG, j + kDepthG < nb, aring[D]);
      }
      // A operands: row 16r + l%16, k = 8*(l/16) .. +7, for each part.
      bf16x8 aop[3][RT];
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int r = 0; r < RT; ++r)
          aop[part][r] = *reinterpret_cast<const bf16x8 *>(&a_lds[part][(16 * r + c16) * kAPitch + 8 * g4]);
      // B operands of the wave's eight column tiles: four columns x eight
      // rows of W per lane and column group, as bf16 pairs in k order.
      bf16x8 bop[kWaveTiles];
#pragma unroll
      for (int q = 0; q < kWaveGroups; ++q) {
        uint32_t x[8];
        const int cb = kWaveCols * wave + 64 * q + 4 * c16;
#pragma unroll
        for (int jr = 0; jr < 8; ++jr) x[jr] = *reinterpret_cast<const uint32_t *>(&w_lds[(8 * g4 + jr) * kWPitch + cb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u4 bw;
          bw.x = byte_pair_bf16(x[0], x[1], i);
          bw.y = byte_pair_bf16(x[2], x[3], i);
          bw.z = byte_pair_bf16(x[4], x[5], i);
          bw.w = byte_pair_bf16(x[6], x[7], i);
          bop[4 * q + i] = __builtin_bit_cast(bf16x8, bw);
        }
      }
      // The block's unscaled partial of every tile: one MFMA per part of A,
      // part-major so that consecutive MFMAs are independent.
      f4 part[kWaveTiles][RT];
#pragma unroll
      for (int t = 0; t < kWaveTiles; ++t)
#pragma unroll
        for (int r = 0; r < RT; ++r) part[t][r] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pa = 0; pa < 3; ++pa)
#pragma unroll
        for (int t = 0; t < kWaveTiles; ++t)
#pragma unroll
          for (int r = 0; r < RT; ++r)
            part[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[pa][r], bop[t], part[t][r], 0, 0, 0);
      // "Factoring out the scale": one multiply per block and column.
#pragma unroll
      for (int t = 0; t < kWaveTiles; ++t) {
        const float s = reinterpret_cast<const float *>(&sv[t >> 2])[t & 3];
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[t][r] = f4{fmaf(part[t][r].x, s, acc[t][r].x), fmaf(part[t][r].y, s, acc[t][r].y),
                         fmaf(part[t][r].z, s, acc[t][r].z), fmaf(part[t][r].w, s, acc[t][r].w)};
      }
    // The scales were used above: refill their slot now.
    if constexpr (REFILL) load_s(b + kDepthG, j + kDepthG < nb, sring[D]);
  };

  // Whole rounds of kDepthG blocks with a fixed load pattern, then the last
  // nb % kDepthG blocks from the ring without refills.
  const int rounds = nb / kDepthG;
  for (int r = 0; r < rounds; ++r) {
    SFor<0, kDepthG>::run([&](auto d_) { process(d_, std::true_type{}, r * kDepthG + decltype(d_)::value); });
  }
  const int tail = nb - rounds * kDepthG;
  SFor<0, kDepthG - 1>::run([&](auto d_) {
    if (decltype(d_)::value < tail) process(d_, std::false_type{}, rounds * kDepthG + decltype(d_)::value);
  });

  // Lane l of tile (q, i) holds rows 16r + 4(l/16) .. +3 of column
  // 64q + 4(l%16) + i of the wave's 128.
  auto out_index = [&](int t, int r, int e, int &m, int &col) {
    const int q = t >> 2, i = t & 3;
    m = 16 * r + 4 * g4 + e;
    col = kWaveCols * wave + 64 * q + 4 * c16 + i;
  };
  if (p.splits == 1) {
#pragma unroll
    for (int t = 0; t < kWaveTiles; ++t)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int m, col;
          out_index(t, r, e, m, col);
          if (m < p.M && n0 + col < p.N) p.C[(size_t)m * p.N + n0 + col] = acc[t][r][e];
        }
    return;
  }

  // Split-K: publish this split's partial with device-coherent (sc1) 16-byte
  // stores, count it, and let the last split of the tile sum them in K order.
  // The partial keeps the lanes' register layout: piece ((w*8 + t)*RT + r)*64
  // + l holds lane l's four values of tile (t, r) of wave w, so each store
  // instruction of a wave writes 1 KB contiguously.
  // With xcd_local every split of this tile runs on this XCD (the tile is
  // blockIdx.x, the split blockIdx.y, and the number of tiles is a multiple
  // of 8, so the dispatcher's turn-by-turn placement puts them together): the
  // partials are then stored into the XCD's L2 (acknowledged there) and read
  // back from it with sc0, and the counter records each split's XCD; if a
  // split ran elsewhere the tile's outputs are written as NaN.
  constexpr int kPieces = kTileElems / 4;
  constexpr int kCoherent = 16;  // cache policy: sc1, written through to the device's coherence point
  constexpr int kL2Load = 1;     // sc0: past the CU's L1, from the XCD's L2
  const bool local = p.xcd_local != 0;
  // A lane's four rows of row tile r are 16r + 4(l/16) .. +3.  When they all
  // lie past M (few rows: their partials are zero and never stored), the
  // lane's partial store and load take an offset past the descriptor's
  // records, so they move no data, without a branch; the rows that exist
  // are published and summed as before.
  auto past_m = [&](int r) { return 16 * r + 4 * g4 < p.M ? 0u : 0x80000000u; };
  const __amdgpu_buffer_rsrc_t part_rs =
      rsrc(p.partial + (size_t)tile * p.splits * kTileElems, (uint32_t)p.splits * kTileElems * 4u);
#pragma unroll
  for (int t = 0; t < kWaveTiles; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t piece = (uint32_t)(((wave * kWaveTiles + t) * RT + r) * 64 + lane);
      const u4 v = __builtin_bit_cast(u4, acc[t][r]);
      const uint32_t off = ((uint32_t)split * kPieces + piece) * 16u + past_m(r);
      if (local)
        __builtin_amdgcn_raw_buffer_store_b128(v, part_rs, off, 0u, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b128(v, part_rs, off, 0u, kCoherent);
    }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t *cnt = &p.counters[tile * kCounterStride];
  if (tid == 0) {
    if (local) {
      const uint32_t x = xcd_id() ^ (p.xcc_skew != 0 ? (uint32_t)split & 1u : 0u);
      const uint64_t prev = __hip_atomic_fetch_add(reinterpret_cast<uint64_t *>(cnt), xcd_increment(x), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      const bool last = xcd_count_done(prev, (uint64_t)p.splits);
      last_flag = last;
      stray_flag = last && !xcd_all_here(prev, x, (uint64_t)p.splits);
    } else {
      const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = prev == (uint32_t)(p.splits - 1);
      stray_flag = 0;
    }
  }
  __syncthreads();
  if (!last_flag) return;
  auto rearm = [&]() {
    if (tid != 0) return;
    if (local)
      __hip_atomic_store(reinterpret_cast<uint64_t *>(cnt), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (stray_flag) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < kWaveTiles; ++t)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int m, col;
          out_index(t, r, e, m, col);
          if (m < p.M && n0 + col < p.N) p.C[(size_t)m * p.N + n0 + col] = nan;
        }
    rearm();
    return;
  }
  // Sum the splits in K order: pairwise over groups of eight, then the groups
  // in order through the cascade of the matvec's combine (SumCascade).
  // Thread (wave, lane) sums the pieces of its own accumulator tiles, BATCH
  // at a time with every load of a batch in flight: its own split is still in
  // its registers, and only the other splits are read back.  A descriptor
  // without records stands in for its own split and for the empty places of
  // the last group of eight; its loads return zeros without a memory access.
  // Up to 64 splits (eight groups) the cascade is the plain sequential sum, so
  // that case keeps one level and two pieces in flight; more splits take the
  // full cascade one piece at a time, within the 16-row instance's registers.
  const __amdgpu_buffer_rsrc_t none_rs = rsrc(p.partial, 0u);
  constexpr int kOwn = kWaveTiles * RT;  // pieces per thread
  auto combine = [&](auto batch_, auto levels_, auto aux_) {
    constexpr int BATCH = decltype(batch_)::value, LEVELS = decltype(levels_)::value, AUX = decltype(aux_)::value;
    static_assert(kOwn % BATCH == 0, "whole batches of pieces");
#pragma unroll
    for (int j0 = 0; j0 < kOwn; j0 += BATCH) {
      SumCascade<f4, BATCH, LEVELS> total;
      for (int c = 0; c < p.splits; c += 8) {
        f4 v[BATCH][8];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int t = (j0 + i) / RT, r = (j0 + i) % RT;
          const uint32_t piece = (uint32_t)(((wave * kWaveTiles + t) * RT + r) * 64 + lane);
#pragma unroll
          for (int sp = 0; sp < 8; ++sp) {
            const int sj = c + sp;
            const bool remote = sj < p.splits && sj != split;
            const uint32_t off = ((uint32_t)min(sj, p.splits - 1) * kPieces + piece) * 16u + past_m(r);
            const f4 x = __builtin_bit_cast(
                f4, __builtin_amdgcn_raw_buffer_load_b128(remote ? part_rs : none_rs, off, 0u, AUX));
            v[i][sp] = sj == split ? acc[t][r] : x;
          }
        }
        f4 x[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          x[i] = ((v[i][0] + v[i][1]) + (v[i][2] + v[i][3])) + ((v[i][4] + v[i][5]) + (v[i][6] + v[i][7]));
        total.add(x);
      }
      f4 sum[BATCH];
      total.result(sum);
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int t = (j0 + i) / RT, r = (j0 + i) % RT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int m, col;
          out_index(t, r, e, m, col);
          if (m < p.M && n0 + col < p.N) p.C[(size_t)m * p.N + n0 + col] = sum[i][e];
        }
      }
    }
  };
  if (p.splits <= 64) {
    if (local)
      combine(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, kL2Load>{});
    else
      combine(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, kCoherent>{});
  } else {
    combine(std::integral_constant<int, 1>{}, std::integral_constant<int, 6>{}, std::integral_constant<int, kCoherent>{});
  }
  rearm();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream) {
  if (a.M < 1 || a.M > kGemmMaxRows) return hipErrorInvalidValue;
  const int rt = gemm_row_tiles(a.M);
  if (a.w_width != 16 && a.w_width != 8 && a.w_width != 4) return hipErrorInvalidValue;
  if (a.N % a.w_width != 0 || (reinterpret_cast<uintptr_t>(a.W) % a.w_width) != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.n_tiles, (unsigned)a.splits, (unsigned)((a.M + 16 * rt - 1) / (16 * rt)));
  auto go = [&](auto rt_) {
    constexpr int R = decltype(rt_)::value;
    if (a.w_width == 16)
      hipLaunchKernelGGL((q8_gemm_kernel<R, 16>), grid, dim3(kGThreads), 0, stream, a);
    else if (a.w_width == 8)
      hipLaunchKernelGGL((q8_gemm_kernel<R, 8>), grid, dim3(kGThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((q8_gemm_kernel<R, 4>), grid, dim3(kGThreads), 0, stream, a);
  };
  if (rt == 1)
    go(std::integral_constant<int, 1>{});
  else if (rt == 2)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, 4>{});
  return hipGetLastError();
}

}  // namespace q8
