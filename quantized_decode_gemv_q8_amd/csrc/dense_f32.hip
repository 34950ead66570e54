// Dense f32 products on the matrix cores: dot (C = A B with B [K,N]) and
// dot_t (C = A B^T with B [N,K]), through the fused epilogue
// y = alpha * P + corr[m] * C_old.
//
// Operation: "dot and tensor cores" page, table of built-ins (dot(a, b) is
// a @ b, dot_t(a, b) is a @ b^T), section "The k loop" (a workgroup owns an
// output tile and adds the product of one panel of A and one of B per step of
// K, the copy of the next panel overlapping the math on the current one) and
// section "The fused epilogue" (the product is scaled, and optionally added to
// row-scaled old contents, as it is written).
//
// Precision.  Section "Hardware paths" gives f32 operands an f32 accumulator;
// tensor-core paths that round the operands to 16 bits would miss that.  Here
// every f32 operand is split exactly into three bf16 parts, x = x0 + x1 + x2
// (each part the round-to-nearest bf16 of what the previous ones leave; the
// subtractions are exact and 3 x 8 significant bits hold all 24 of an f32),
// and of the nine part products the six with p + q <= 2 are accumulated in
// f32 by v_mfma_f32_16x16x32_bf16.  The three dropped products are below
// 2^-24 |a b| together, so every product keeps f32 accuracy while the work
// runs on the bf16 matrix cores: six bf16 MFMAs per f32 product still beat
// the f32 matrix rate (measured 199 against 129 TFLOP/s of f32 products on
// a 4096^3 product).
//
// Work decomposition (gfx950):
//   * A workgroup of four wave64s owns a 128 x 128 tile of C; wave w owns the
//     64 x 64 quarter (w / 2, w % 2) as 4 x 4 MFMA tiles of 16 x 16 (64
//     accumulator registers per lane).  K goes in panels of 32, one MFMA
//     k-slice.  With more tiles than two per CU the grid stops at two
//     workgroups per CU and each takes several tiles in turn, loading the
//     next tile's first panel while it multiplies the current one's last.
//   * Each thread loads its share of the next panel (A, and B) into registers
//     while the current one is multiplied; the panel is split as it is
//     written to LDS, as three bf16 part tiles [row][k].  One LDS buffer
//     (60 KB) lets two workgroups share a CU, with two barriers per panel;
//     the MFMA block runs at raised wave priority so the other workgroup's
//     staging fills its gaps.
//   * LDS padding ("@padstage"): the part tiles are read by column (the 16
//     lanes of a read pass take 16 rows at the same k), so rows are padded
//     from 64 to 96 bytes.  Measured against the unpadded tile, the padding
//     takes the 4096^3 product from 832 to 678 us; a pad of 16 bytes (the
//     pages' 8 elements) gives 690.
//   * Loads keep a per-lane offset fixed for the whole K loop; the panel's k
//     offset and every row step are scalar offsets.  dot's B [K,N] is read
//     with dword loads so that each thread holds four consecutive k of one
//     column (its [column][k] part tiles are then written 8 bytes at a time).
//   * Tiles are dealt to the eight XCDs in contiguous ranges (the dispatcher
//     sends workgroup i to XCD i mod 8), and inside a range in groups of
//     eight tile rows, column by column, so that the workgroups resident on
//     one XCD share panels of A and B in its L2.
//   * Ragged M and N are masked at the store; a ragged last panel of K is
//     zero-filled as it is staged.  Rows and columns past the operands are
//     read through bounded buffer descriptors (reads past the end return
//     zero, nothing faults).
#include <type_traits>

#include "q8_common.h"

namespace q8 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 128;            // rows of C per workgroup
constexpr int kTN = 128;            // columns of C per workgroup
constexpr int kTK = 32;             // K per panel (one MFMA k-slice)
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
// threads).
struct Panel {
  f4 v[4];
};

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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));

constexpr int kSP = kTK + 16;              // bf16 pitch of a [row][k] part tile (96 bytes)
constexpr int kPartTile = 128 * kSP;       // bf16 elements of one part tile

// Round-to-nearest-even bf16 of (x, y) packed into one dword, x in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, y}, bf16x2));
}

// Splits four f32 into three bf16 parts each, as packed pairs: part q of
// elements (2h, 2h+1) is dword h of out[q].  Each remainder is exact.
__device__ __forceinline__ void split3(f4 x, u2 (&out)[3]) {
  SFor<0, 2>::run([&](auto h) {
    float a = x[2 * (int)h], b = x[2 * (int)h + 1];
    SFor<0, 3>::run([&](auto q) {
      const uint32_t u = pk_bf16(a, b);
      out[q][(int)h] = u;
      if constexpr (q < 2) {
        a -= __uint_as_float(u << 16);
        b -= __uint_as_float(u & 0xffff0000u);
      }
    });
  });
}

// Loads of the split kernel: the per-lane part of each address is fixed for
// the whole K loop, and the panel's k offset and each row step go into the
// scalar offset.
//   rows  (A, and dot_t's B): VEC 4: chunk i is row tid/8 + 32 i, k 4 (tid % 8);
//         VEC 1: element j is row tid/32 + 8 j, k tid % 32.
//   cols  (dot's B [K,N]): element (j, e) is column tid % 128, k 4 (tid/128 + 2 j) + e.
template <int VEC>
__device__ __forceinline__ uint32_t rows_voff(int tid, int row0, int K) {
  return VEC == 4 ? ((uint32_t)(row0 + tid / 8) * (uint32_t)K + 4u * (uint32_t)(tid % 8)) * 4u
                  : ((uint32_t)(row0 + tid / 32) * (uint32_t)K + (uint32_t)(tid % 32)) * 4u;
}
template <int VEC>
__device__ __forceinline__ void sload_rows(Panel &pn, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int K, int k0) {
  if constexpr (VEC == 4) {
    SFor<0, 4>::run([&](auto i) {
      const uint32_t so = (uint32_t)k0 * 4u + (uint32_t)(32 * i) * (uint32_t)K * 4u;
      pn.v[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, so, 0));
    });
  } else {
    SFor<0, 16>::run([&](auto j) {
      const uint32_t so = (uint32_t)k0 * 4u + (uint32_t)(8 * j) * (uint32_t)K * 4u;
      pn.v[j / 4][j % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, so, 0));
    });
  }
}
__device__ __forceinline__ uint32_t cols_voff(int tid, int n0, int N) {
  return ((uint32_t)(4 * (tid / 128)) * (uint32_t)N + (uint32_t)(n0 + tid % 128)) * 4u;
}
__device__ __forceinline__ void sload_cols(Panel &pn, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int N, int k0) {
  SFor<0, 4>::run([&](auto j) {
    SFor<0, 4>::run([&](auto e) {
      const uint32_t so = (uint32_t)(k0 + 8 * j + e) * (uint32_t)N * 4u;
      pn.v[j][(int)e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, so, 0));
    });
  });
}

// Writes a rows panel as three [128][kSP] part tiles.  MASK zeroes k >= kv
// (only the ragged last panel needs it).
template <int VEC, bool MASK>
__device__ __forceinline__ void stage_rows_split(__bf16 *t, const Panel &pn, int tid, int kv) {
  if constexpr (VEC == 4) {
    const int kc = 4 * (tid % 8);
    SFor<0, 4>::run([&](auto i) {
      u2 q[3];
      split3(MASK && kc >= kv ? f4{0.f, 0.f, 0.f, 0.f} : pn.v[i], q);
      const int off = (tid / 8 + 32 * i) * kSP + kc;
      SFor<0, 3>::run([&](auto pp) { *reinterpret_cast<u2 *>(t + pp * kPartTile + off) = q[pp]; });
    });
  } else {
    const int k = tid % 32;
    SFor<0, 4>::run([&](auto i) {
      u2 q[3];
      split3(MASK && k >= kv ? f4{0.f, 0.f, 0.f, 0.f} : pn.v[i], q);
      SFor<0, 4>::run([&](auto e) {
        const int off = (tid / 32 + 8 * (4 * i + e)) * kSP + k;
        SFor<0, 3>::run([&](auto pp) {
          const uint32_t w = q[pp][(int)e / 2];
          reinterpret_cast<uint16_t *>(t)[pp * kPartTile + off] = (uint16_t)(e % 2 ? w >> 16 : w);
        });
      });
    });
  }
}

// Writes dot's B panel (cols layout) as three [128 columns][kSP] part tiles.
template <bool MASK>
__device__ __forceinline__ void stage_cols_split(__bf16 *t, const Panel &pn, int tid, int kv) {
  SFor<0, 4>::run([&](auto j) {
    const int kq = 4 * (tid / 128 + 2 * j);
    f4 x = pn.v[j];
    if constexpr (MASK) {
      SFor<0, 4>::run([&](auto e) { x[(int)e] = kq + (int)e < kv ? x[(int)e] : 0.f; });
    }
    u2 q[3];
    split3(x, q);
    const int off = (tid % 128) * kSP + kq;
    SFor<0, 3>::run([&](auto pp) { *reinterpret_cast<u2 *>(t + pp * kPartTile + off) = q[pp]; });
  });
}

template <bool TRANS_B, int VEC>
__global__ __launch_bounds__(kThreads) void dense_split_kernel(DenseArgs p) {
  __shared__ __attribute__((aligned(16))) __bf16 a_lds[3 * kPartTile];
  __shared__ __attribute__((aligned(16))) __bf16 b_lds[3 * kPartTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int tiles_m = (p.M + kTM - 1) / kTM, tiles_n = (p.N + kTN - 1) / kTN;
  const int tiles = tiles_m * tiles_n;

  const __amdgpu_buffer_rsrc_t a_rs = rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K * 4u);
  const __amdgpu_buffer_rsrc_t b_rs = rsrc(p.B, (uint32_t)p.N * (uint32_t)p.K * 4u);
  const int np = (p.K + kTK - 1) / kTK;

  // The workgroup takes tiles v = blockIdx.x + i * gridDim.x in turn (with
  // the grid a multiple of eight, all of them in its XCD's range).  The first
  // panel of the next tile is loaded while the last panel of the current one
  // is multiplied, so its latency overlaps that multiply and the stores.
  int v = blockIdx.x;
  int tm, tn;
  tile_of(v, tiles, tiles_m, tiles_n, &tm, &tn);
  uint32_t a_voff = rows_voff<VEC>(tid, tm * kTM, p.K);
  uint32_t b_voff = TRANS_B ? rows_voff<VEC>(tid, tn * kTN, p.K) : cols_voff(tid, tn * kTN, p.N);
  auto load = [&](Panel &pa, Panel &pb, int kt) {
    sload_rows<VEC>(pa, a_rs, a_voff, p.K, kt);
    if constexpr (TRANS_B) {
      sload_rows<VEC>(pb, b_rs, b_voff, p.K, kt);
    } else {
      sload_cols(pb, b_rs, b_voff, p.N, kt);
    }
  };
  auto stage = [&](auto mask_, const Panel &pa, const Panel &pb, int kv) {
    constexpr bool MASK = decltype(mask_)::value;
    stage_rows_split<VEC, MASK>(a_lds, pa, tid, kv);
    if constexpr (TRANS_B) {
      stage_rows_split<VEC, MASK>(b_lds, pb, tid, kv);
    } else {
      stage_cols_split<MASK>(b_lds, pb, tid, kv);
    }
  };

  Panel pa, pb;
  load(pa, pb, 0);
  for (bool first = true;; first = false) {
    const int m0 = tm * kTM, n0 = tn * kTN;
    const int v_next = v + (int)gridDim.x;
    const bool more = v_next < tiles;
    f4 acc[4][4];
    SFor<0, 4>::run([&](auto i) { SFor<0, 4>::run([&](auto j) { acc[i][j] = f4{0.f, 0.f, 0.f, 0.f}; }); });

    for (int pnl = 0; pnl < np; ++pnl) {
      const int kt = pnl * kTK;
      if (pnl > 0 || !first) lds_barrier();  // every wave has finished reading the previous panel
      if (p.K - kt >= kTK) {
        stage(std::false_type{}, pa, pb, kTK);
      } else {
        stage(std::true_type{}, pa, pb, p.K - kt);
      }
      lds_barrier();
      if (pnl + 1 < np) {
        load(pa, pb, kt + kTK);
      } else if (more) {
        tile_of(v_next, tiles, tiles_m, tiles_n, &tm, &tn);
        a_voff = rows_voff<VEC>(tid, tm * kTM, p.K);
        b_voff = TRANS_B ? rows_voff<VEC>(tid, tn * kTN, p.K) : cols_voff(tid, tn * kTN, p.N);
        load(pa, pb, 0);
      }

      // Lane l of MFMA tile (i, j) supplies row / column 16 i + l % 16 and
      // k = 8 (l / 16) .. +7 of each part.
      bf16x8 af[4][3], bf[4][3];
      SFor<0, 4>::run([&](auto i) {
        SFor<0, 3>::run([&](auto pp) {
          af[i][pp] = *reinterpret_cast<const bf16x8 *>(a_lds + pp * kPartTile + (64 * wm + 16 * i + c16) * kSP + 8 * g4);
          bf[i][pp] = *reinterpret_cast<const bf16x8 *>(b_lds + pp * kPartTile + (64 * wn + 16 * i + c16) * kSP + 8 * g4);
        });
      });
      // Part products with p + q <= 2, smallest first, at raised wave priority
      // so that the other workgroup's staging fills the gaps rather than delays them.
      __builtin_amdgcn_s_setprio(1);
      SFor<0, 6>::run([&](auto t) {
        constexpr int kP[6] = {2, 1, 0, 1, 0, 0};
        constexpr int kQ[6] = {0, 1, 2, 0, 1, 0};
        SFor<0, 4>::run([&](auto i) {
          SFor<0, 4>::run([&](auto j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i][kP[t]], bf[j][kQ[t]], acc[i][j], 0, 0, 0);
          });
        });
      });
      __builtin_amdgcn_s_setprio(0);
    }

    // Lane l of tile (i, j) holds rows 16 i + 4 (l / 16) + e, column 16 j + l % 16.
    // A tile wholly inside C without row factors (both uniform over the
    // workgroup) takes straight-line stores.
    const bool whole = m0 + kTM <= p.M && n0 + kTN <= p.N;
    const int m_w = m0 + 64 * wm + 4 * g4, n_w = n0 + 64 * wn + c16;
    if (whole && p.corr == nullptr) {
      float *base = p.C + (size_t)m_w * p.N + n_w;
      SFor<0, 4>::run([&](auto i) {
        SFor<0, 4>::run([&](auto j) {
          SFor<0, 4>::run([&](auto e) {
            base[(size_t)(16 * i + e) * p.N + 16 * j] = p.alpha * acc[i][j][(int)e];
          });
        });
      });
    } else {
      SFor<0, 4>::run([&](auto i) {
        SFor<0, 4>::run([&](auto j) {
          const int n = n_w + 16 * j;
          SFor<0, 4>::run([&](auto e) {
            const int m = m_w + 16 * i + e;
            if (m < p.M && n < p.N) {
              float *c = p.C + (size_t)m * p.N + n;
              float y = p.alpha * acc[i][j][(int)e];
              if (p.corr) y = fmaf(p.corr[m], *c, y);
              *c = y;
            }
          });
        });
      });
    }
    if (!more) break;
    v = v_next;
  }
}

}  // namespace

hipError_t launch_dense_f32(const DenseArgs &a, bool trans_b, int vec, int max_wgs, hipStream_t stream) {
  // One workgroup per tile up to max_wgs; beyond that a grid of max_wgs
  // (rounded down to a multiple of eight) whose workgroups take several tiles.
  const int tiles = ((a.M + kTM - 1) / kTM) * ((a.N + kTN - 1) / kTN);
  const int cap = max_wgs >= 8 ? max_wgs / 8 * 8 : 8;
  const dim3 grid((unsigned)(tiles <= cap ? tiles : cap)), block(kThreads);
  if (vec == 4) {
    if (trans_b) {
      hipLaunchKernelGGL((dense_split_kernel<true, 4>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((dense_split_kernel<false, 4>), grid, block, 0, stream, a);
    }
  } else if (vec == 1) {
    if (trans_b) {
      hipLaunchKernelGGL((dense_split_kernel<true, 1>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((dense_split_kernel<false, 1>), grid, block, 0, stream, a);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q8
