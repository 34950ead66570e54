// Ordered summation shared by the split-K combines of the Q8_0 kernels.
#pragma once

namespace q8 {

// An ordered sum of many terms (the per-group sums of a split-K combine),
// taken as a cascade of short sequential sums: level 0 adds up to eight
// terms in order, and every eighth term it hands its sum on to level 1, which
// adds up to eight such sums, and so on; the last level adds whatever reaches
// it.  The result is the levels' sums, highest first.  With at most eight
// terms it equals the plain sequential sum bit for bit; in general each term
// passes through at most kLevels short sums, so the rounding grows with the
// number of levels instead of the number of terms.  The order depends only on
// the number of terms, so the result is deterministic.  T is float or a float
// vector.  With L = 1 it is the plain sequential sum.
template <class T, int W, int L = 6>
struct SumCascade {
  static constexpr int kLevels = L;  // at 6: 8^5 terms before the last level sums in order
  T lvl[kLevels][W];
  int n = 0;  // terms added so far (wave-uniform)
  __device__ __forceinline__ SumCascade() {
#pragma unroll
    for (int l = 0; l < kLevels; ++l)
#pragma unroll
      for (int j = 0; j < W; ++j) lvl[l][j] = T{};
  }
  __device__ __forceinline__ void add(const T (&x)[W]) {
#pragma unroll
    for (int j = 0; j < W; ++j) lvl[0][j] += x[j];
    int q = ++n;
#pragma unroll
    for (int l = 0; l + 1 < kLevels; ++l) {
      if (q & 7) break;
      q >>= 3;
#pragma unroll
      for (int j = 0; j < W; ++j) {
        lvl[l + 1][j] += lvl[l][j];
        lvl[l][j] = T{};
      }
    }
  }
  __device__ __forceinline__ void result(T (&out)[W]) const {
#pragma unroll
    for (int j = 0; j < W; ++j) {
      T r = lvl[kLevels - 1][j];
#pragma unroll
      for (int l = kLevels - 2; l >= 0; --l) r += lvl[l][j];
      out[j] = r;
    }
  }
};

}  // namespace q8
