// Dense f32 products on the matrix cores: dot (C = A B with B [K,N]) and
// dot_t (C = A B^T with B [N,K]), through the fused epilogue
// y = alpha * P + corr[m] * C_old.
//
// Operation: "dot and tensor cores" page, table of built-ins (dot(a, b) is
// a @ b, dot_t(a, b) is a @ b^T), section "The k loop" (a workgroup owns an
// output tile and adds the product of one panel of A and one of B per step of
// K; under pipelining the copy of the next panel overlaps the math on the
// current one) and section "The fused epilogue" (the product is scaled, and
// optionally added to row-scaled old contents, as it is written).
//
// Precision.  Section "Hardware paths" gives f32 operands an f32 accumulator
// on FMA units.  v_mfma_f32_32x32x2_f32 multiplies full f32 operands into an
// f32 accumulator (no operand rounding), so it keeps that contract; it is
// also the only way to reach the chip's f32 matrix rate, since vector FMA
// without packed instructions gets half of it.
//
// Work decomposition (gfx950):
//   * A workgroup of four wave64s owns a 128 x 128 tile of C; wave w owns the
//     64 x 64 quarter (w / 2, w % 2) as 2 x 2 MFMA tiles of 32 x 32 (64
//     accumulator registers per lane).
//   * K is walked in panels of 32.  Panel p + 1 is loaded from global memory
//     into registers while panel p is multiplied out of LDS; the registers
//     are then written to the other LDS buffer and one barrier per panel
//     separates the two (two LDS buffers).
//   * Within a panel, MFMA step s (0..15) takes k = s from lanes 0..31 and
//     k = 16 + s from lanes 32..63 (the contraction is a sum, so any pairing
//     of k with MFMA slots that both operands share is the same product up to
//     rounding order).  A lane therefore reads 16 consecutive k of its row of
//     a [row][k] tile as four 16-byte LDS reads.
//   * LDS tiles: A and dot_t's B as [128 rows][32 k] with a row pitch of 36
//     floats (8 consecutive rows of 144 bytes start on distinct 4-bank groups,
//     so 16-byte reads of 8 lanes never share a bank); dot's B as [32 k][128
//     columns] with a pitch of 132 floats, read one dword per lane (32 lanes
//     read 128 contiguous bytes).
//   * Tiles are dealt to the eight XCDs in contiguous ranges (the dispatcher
//     sends workgroup i to XCD i mod 8), and inside a range in groups of
//     eight tile rows, column by column, so that the workgroups resident on
//     one XCD share panels of A and B in its L2.
//   * Ragged M and N are masked at the store; a ragged last panel of K is
//     zero-filled before it reaches LDS.  Rows and columns past the operands
//     are read through bounded buffer descriptors (reads past the end return
//     zero, nothing faults).
#include <type_traits>

#include "q8_common.h"

namespace q8 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 128;            // rows of C per workgroup
constexpr int kTN = 128;            // columns of C per workgroup
constexpr int kTK = 32;             // K per panel
constexpr int kPitchK = kTK + 4;    // [row][k] tile pitch, floats
constexpr int kPitchN = kTN + 4;    // [k][column] tile pitch, floats
constexpr int kRowTile = kTM * kPitchK;  // floats of one [128][32] tile
constexpr int kGroupRows = 8;       // tile rows per group of the tile order

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

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

// Registers of one thread's share of a 128 x 32 panel (4096 floats over 256
// threads): four 16-byte chunks at VEC 4, sixteen dwords at VEC 1.
struct Panel {
  f4 v[4];
};

// Loads this thread's share of a k-contiguous panel: rows row0..row0+127 of
// a [rows][K] matrix (row pitch K floats), columns k0..k0+31.
//   VEC 4: chunk c = tid + 256 i is row c / 8, k 4 (c % 8).
//   VEC 1: element e = tid + 256 j is row e / 32, k e % 32.
template <int VEC>
__device__ __forceinline__ void load_rows(Panel &pn, __amdgpu_buffer_rsrc_t rs, int tid, int row0, int K, int k0) {
  if constexpr (VEC == 4) {
    const uint32_t base = ((uint32_t)(row0 + tid / 8) * (uint32_t)K + (uint32_t)(k0 + 4 * (tid % 8))) * 4u;
    const uint32_t step = 32u * (uint32_t)K * 4u;
    SFor<0, 4>::run([&](auto i) {
      pn.v[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + i * step, 0u, 0));
    });
  } else {
    const uint32_t base = ((uint32_t)(row0 + tid / 32) * (uint32_t)K + (uint32_t)(k0 + tid % 32)) * 4u;
    const uint32_t step = 8u * (uint32_t)K * 4u;
    SFor<0, 16>::run([&](auto j) {
      pn.v[j / 4][j % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, base + j * step, 0u, 0));
    });
  }
}

// Writes a k-contiguous panel to a [128][kPitchK] LDS tile, zeroing k >= kv.
template <int VEC>
__device__ __forceinline__ void store_rows(float *t, const Panel &pn, int tid, int kv) {
  if constexpr (VEC == 4) {
    const int kc = 4 * (tid % 8);
    const bool live = kc < kv;  // K % 4 == 0 at VEC 4: a chunk is all in or all out
    SFor<0, 4>::run([&](auto i) {
      const f4 x = live ? pn.v[i] : f4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f4 *>(t + (tid / 8 + 32 * i) * kPitchK + kc) = x;
    });
  } else {
    const int k = tid % 32;
    const bool live = k < kv;
    SFor<0, 16>::run([&](auto j) {
      t[(tid / 32 + 8 * j) * kPitchK + k] = live ? pn.v[j / 4][j % 4] : 0.f;
    });
  }
}

// Loads this thread's share of a [32 k][128 columns] panel of dot's B [K,N].
//   VEC 4: chunk c = tid + 256 i is k c / 32, column 4 (c % 32).
//   VEC 1: element e = tid + 256 j is k e / 128, column e % 128.
template <int VEC>
__device__ __forceinline__ void load_cols(Panel &pn, __amdgpu_buffer_rsrc_t rs, int tid, int k0, int N, int n0) {
  if constexpr (VEC == 4) {
    const uint32_t base = ((uint32_t)(k0 + tid / 32) * (uint32_t)N + (uint32_t)(n0 + 4 * (tid % 32))) * 4u;
    const uint32_t step = 8u * (uint32_t)N * 4u;
    SFor<0, 4>::run([&](auto i) {
      pn.v[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + i * step, 0u, 0));
    });
  } else {
    const uint32_t base = ((uint32_t)(k0 + tid / 128) * (uint32_t)N + (uint32_t)(n0 + tid % 128)) * 4u;
    const uint32_t step = 2u * (uint32_t)N * 4u;
    SFor<0, 16>::run([&](auto j) {
      pn.v[j / 4][j % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, base + j * step, 0u, 0));
    });
  }
}

// Writes dot's B panel to a [32][kPitchN] LDS tile, zeroing k >= kv.
template <int VEC>
__device__ __forceinline__ void store_cols(float *t, const Panel &pn, int tid, int kv) {
  if constexpr (VEC == 4) {
    SFor<0, 4>::run([&](auto i) {
      const int k = tid / 32 + 8 * i;
      const f4 x = k < kv ? pn.v[i] : f4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f4 *>(t + k * kPitchN + 4 * (tid % 32)) = x;
    });
  } else {
    SFor<0, 16>::run([&](auto j) {
      const int k = tid / 128 + 2 * j;
      t[k * kPitchN + tid % 128] = k < kv ? pn.v[j / 4][j % 4] : 0.f;
    });
  }
}

// Tile of this workgroup: XCD-contiguous ranges, then groups of kGroupRows
// tile rows walked column by column.
__device__ __forceinline__ void tile_of(int wg, int n_wg, int tiles_m, int tiles_n, int *tm, int *tn) {
  const int x = wg % 8, slot = wg / 8;
  const int q = n_wg / 8, rem = n_wg % 8;
  const int t = (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + slot;
  const int per_group = kGroupRows * tiles_n;
  const int g = t / per_group, r = t % per_group;
  const int first = g * kGroupRows;
  const int rows = min(kGroupRows, tiles_m - first);
  *tm = first + r % rows;
  *tn = r / rows;
}

// TRANS_B: dot_t (B [N,K]); otherwise dot (B [K,N]).  VEC: 4 when every row
// of A and B starts 16-byte aligned, else 1.
template <bool TRANS_B, int VEC>
__global__ __launch_bounds__(kThreads) void dense_f32_kernel(DenseArgs p) {
  __shared__ __attribute__((aligned(16))) float a_lds[2][kRowTile];
  __shared__ __attribute__((aligned(16))) float b_lds[2][TRANS_B ? kRowTile : kTK * kPitchN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, half = lane >> 5;
  const int tiles_m = (p.M + kTM - 1) / kTM, tiles_n = (p.N + kTN - 1) / kTN;
  int tm, tn;
  tile_of(blockIdx.x, (int)gridDim.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * kTM, n0 = tn * kTN;

  const __amdgpu_buffer_rsrc_t a_rs = rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K * 4u);
  const __amdgpu_buffer_rsrc_t b_rs = rsrc(p.B, (uint32_t)p.N * (uint32_t)p.K * 4u);
  const int np = (p.K + kTK - 1) / kTK;

  auto load = [&](Panel &pa, Panel &pb, int kt) {
    load_rows<VEC>(pa, a_rs, tid, m0, p.K, kt);
    if constexpr (TRANS_B) {
      load_rows<VEC>(pb, b_rs, tid, n0, p.K, kt);
    } else {
      load_cols<VEC>(pb, b_rs, tid, kt, p.N, n0);
    }
  };
  auto store = [&](const Panel &pa, const Panel &pb, int buf, int kt) {
    const int kv = p.K - kt;
    store_rows<VEC>(a_lds[buf], pa, tid, kv);
    if constexpr (TRANS_B) {
      store_rows<VEC>(b_lds[buf], pb, tid, kv);
    } else {
      store_cols<VEC>(b_lds[buf], pb, tid, kv);
    }
  };

  f16v acc[2][2];
  SFor<0, 2>::run([&](auto i) { SFor<0, 2>::run([&](auto j) { acc[i][j] = f16v{}; }); });

  Panel pa, pb;
  load(pa, pb, 0);
  store(pa, pb, 0, 0);
  lds_barrier();

  for (int pnl = 0; pnl < np; ++pnl) {
    const int buf = pnl & 1;
    const bool more = pnl + 1 < np;
    if (more) load(pa, pb, (pnl + 1) * kTK);

    // Operands of this panel: lane (r32, half) holds k = 16 half + s, s = 0..15.
    f4 af[2][4], bf[2][4];
    SFor<0, 2>::run([&](auto i) {
      const float *src = a_lds[buf] + (64 * wm + 32 * i + r32) * kPitchK + 16 * half;
      SFor<0, 4>::run([&](auto q) { af[i][q] = *reinterpret_cast<const f4 *>(src + 4 * q); });
    });
    SFor<0, 2>::run([&](auto j) {
      if constexpr (TRANS_B) {
        const float *src = b_lds[buf] + (64 * wn + 32 * j + r32) * kPitchK + 16 * half;
        SFor<0, 4>::run([&](auto q) { bf[j][q] = *reinterpret_cast<const f4 *>(src + 4 * q); });
      } else {
        const float *src = b_lds[buf] + (16 * half) * kPitchN + 64 * wn + 32 * j + r32;
        SFor<0, 16>::run([&](auto s) { bf[j][s / 4][s % 4] = src[s * kPitchN]; });
      }
    });
    SFor<0, 16>::run([&](auto s) {
      SFor<0, 2>::run([&](auto i) {
        SFor<0, 2>::run([&](auto j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s / 4][s % 4], bf[j][s / 4][s % 4], acc[i][j], 0,
                                                           0, 0);
        });
      });
    });

    if (more) {
      store(pa, pb, buf ^ 1, (pnl + 1) * kTK);
      lds_barrier();
    }
  }

  // Epilogue.  Accumulator register r of lane (r32, half) in tile (i, j) is
  // row 8 (r / 4) + 4 half + r % 4 and column r32 of that 32 x 32 tile.  A
  // tile wholly inside C and an epilogue without row factors (both uniform
  // over the workgroup) take straight-line stores.
  const bool whole = m0 + kTM <= p.M && n0 + kTN <= p.N;
  const int m_w = m0 + 64 * wm + 4 * half, n_w = n0 + 64 * wn + r32;
  if (whole && p.corr == nullptr) {
    float *base = p.C + (size_t)m_w * p.N + n_w;
    SFor<0, 2>::run([&](auto i) {
      SFor<0, 2>::run([&](auto j) {
        SFor<0, 16>::run([&](auto r) {
          base[(size_t)(32 * i + 8 * (r / 4) + r % 4) * p.N + 32 * j] = p.alpha * acc[i][j][(int)r];
        });
      });
    });
    return;
  }
  SFor<0, 2>::run([&](auto i) {
    SFor<0, 2>::run([&](auto j) {
      const int n = n_w + 32 * j;
      SFor<0, 16>::run([&](auto r) {
        const int m = m_w + 32 * i + 8 * (r / 4) + r % 4;
        if (m < p.M && n < p.N) {
          float *c = p.C + (size_t)m * p.N + n;
          float y = p.alpha * acc[i][j][(int)r];
          if (p.corr) y = fmaf(p.corr[m], *c, y);
          *c = y;
        }
      });
    });
  });
}

}  // namespace

hipError_t launch_dense_f32(const DenseArgs &a, bool trans_b, int vec, hipStream_t stream) {
  const int tiles = ((a.M + kTM - 1) / kTM) * ((a.N + kTN - 1) / kTN);
  const dim3 grid((unsigned)tiles), block(kThreads);
  if (vec == 4) {
    if (trans_b) {
      hipLaunchKernelGGL((dense_f32_kernel<true, 4>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((dense_f32_kernel<false, 4>), grid, block, 0, stream, a);
    }
  } else if (vec == 1) {
    if (trans_b) {
      hipLaunchKernelGGL((dense_f32_kernel<true, 1>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((dense_f32_kernel<false, 1>), grid, block, 0, stream, a);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q8
