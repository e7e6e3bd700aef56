// e2f_dense.hip -- the channel-wise tensor product h (x) R(r) as a dense
// Clebsch-Gordan contraction: the baseline that the E2Former-V2 write-up
// (stapisi.com, section 2.2, Fig. 3) measures EAAS against, and that the
// gist.science summary (technical summary 2.1) prices at O(L^6) against
// EAAS's O(L^3).
//
// For every path (li, lf, lo) the real coupling tensor C_p[mi, mf, mo] is
// applied in full, zeros included:
//
//   y[lo, mo] += sum_{mi, mf} w_p C_p[mi, mf, mo] h[li, mi] R_lf(r)[mf]
//
// with R_lf the real solid harmonics |r|^lf C_lf(r_hat) (Racah normalisation)
// as polynomials of the vector's components.  At lmax = 2 that is 615
// multiply-adds per channel plus the 81 products h[si] R[sf]; EAAS needs about
// 95.  The coefficients (weights folded in) arrive from the host in the order
// path, mi, mf, mo, and are read through the scalar unit; one group of
// 2^lane_log lanes serves one vector, each lane V adjacent channels (4 when C
// allows it, else 1: the unrolled contraction is long, and each width is
// compiled separately).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {
namespace {

constexpr int kDenseWaves = 4;

// Offset of path (li, lf, lo)'s tensor in the flat table: paths in
// lexicographic order, each (2li+1)(2lf+1)(2lo+1) entries.
__host__ __device__ constexpr int dense_offset(int lmax, int li_, int lf_, int lo_) {
  int off = 0;
  for (int li = 0; li <= lmax; ++li)
    for (int lf = 0; lf <= lmax; ++lf)
      for (int lo = 0; lo <= lmax; ++lo) {
        if (lo < (li > lf ? li - lf : lf - li) || lo > li + lf) continue;
        if (li == li_ && lf == lf_ && lo == lo_) return off;
        off += (2 * li + 1) * (2 * lf + 1) * (2 * lo + 1);
      }
  return -1;
}

// Real solid harmonics R_l(r) = |r|^l C_l(r_hat), l <= LMAX, components
// m = -l..l at flat index l^2 + l + m:
//   l = 1: (y, z, x)
//   l = 2: (sqrt3 xy, sqrt3 yz, (3z^2 - r^2)/2, sqrt3 xz, sqrt3/2 (x^2 - y^2))
template <int LMAX>
__device__ inline void solid_harmonics(float x, float y, float z, float* R) {
  R[0] = 1.0f;
  if constexpr (LMAX >= 1) {
    R[1] = y;
    R[2] = z;
    R[3] = x;
  }
  if constexpr (LMAX >= 2) {
    const float k3 = 1.7320508075688772f;
    const float r2 = x * x + y * y + z * z;
    R[4] = k3 * x * y;
    R[5] = k3 * y * z;
    R[6] = 0.5f * (3.0f * z * z - r2);
    R[7] = k3 * x * z;
    R[8] = 0.5f * k3 * (x * x - y * y);
  }
}

// The non-zero-sized (si, sf, so) triples of the contraction in table order,
// with their coefficient index: every path's full tensor, zeros included.
struct Term {
  int si, sf, so, ci;
};

constexpr int dense_terms_count(int lmax) {
  int n = 0;
  for (int li = 0; li <= lmax; ++li)
    for (int lf = 0; lf <= lmax; ++lf)
      for (int lo = 0; lo <= lmax; ++lo)
        if (lo >= (li > lf ? li - lf : lf - li) && lo <= li + lf)
          n += (2 * li + 1) * (2 * lf + 1) * (2 * lo + 1);
  return n;
}

template <int LMAX>
struct DenseTerms {
  static constexpr int n = dense_terms_count(LMAX);
  Term t[n];
  // ordered by (li, lf), then (mi, mf), then lo and mo, so that consecutive terms
  // share the product h[si] R[sf]
  constexpr DenseTerms() : t() {
    int k = 0;
    for (int li = 0; li <= LMAX; ++li)
      for (int lf = 0; lf <= LMAX; ++lf)
        for (int mi = 0; mi < 2 * li + 1; ++mi)
          for (int mf = 0; mf < 2 * lf + 1; ++mf)
            for (int lo = 0; lo <= LMAX; ++lo) {
              if (lo < (li > lf ? li - lf : lf - li) || lo > li + lf) continue;
              for (int mo = 0; mo < 2 * lo + 1; ++mo) {
                t[k].si = li * li + mi;
                t[k].sf = lf * lf + mf;
                t[k].so = lo * lo + mo;
                t[k].ci = dense_offset(LMAX, li, lf, lo) +
                          (mi * (2 * lf + 1) + mf) * (2 * lo + 1) + mo;
                ++k;
              }
            }
  }
};

template <int LMAX>
struct DenseTable {
  static constexpr DenseTerms<LMAX> tab{};   // evaluated once per degree
};

// y[so] += c[ci] (x[si] R[sf]) for terms I.., indices fixed at compile time
// (the product x[si] R[sf] of consecutive terms is the same value, computed once)
template <int LMAX, int V, int I>
__device__ __forceinline__ void dense_apply(const float (&x)[ncomp(LMAX)][V], const float (&R)[ncomp(LMAX)],
                                            const DenseCoef& cf, float (&y)[ncomp(LMAX)][V]) {
  constexpr Term tm = DenseTable<LMAX>::tab.t[I];
  const float c = cf.c[tm.ci];
#pragma unroll
  for (int v = 0; v < V; ++v) y[tm.so][v] = fmaf(c, x[tm.si][v] * R[tm.sf], y[tm.so][v]);
  if constexpr (I + 1 < DenseTerms<LMAX>::n) dense_apply<LMAX, V, I + 1>(x, R, cf, y);
}

template <int LMAX, int V, typename T>
__global__ __launch_bounds__(64 * kDenseWaves) void k_dense_tp(EaasArgs a, DenseCoef cf) {
  constexpr int S = ncomp(LMAX);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lg = a.lane_log;
  const int sub = lane >> lg;
  const int gl = lane & ((1 << lg) - 1);
  const int64_t atom = ((int64_t)blockIdx.x * kDenseWaves + w) * (64 >> lg) + sub;
  if (atom >= a.n) return;
  const int C = a.C;
  float R[S];
  solid_harmonics<LMAX>(a.r[3 * atom], a.r[3 * atom + 1], a.r[3 * atom + 2], R);
  const T* src = static_cast<const T*>(a.h_in) + atom * (int64_t)S * C;
  T* dst = static_cast<T*>(a.h_out) + atom * (int64_t)S * C;
  for (int c0 = gl * V; c0 < C; c0 += V << lg) {
    float x[S][V];
#pragma unroll
    for (int s = 0; s < S; ++s) VecIO<T, V>::load(src + s * C + c0, x[s]);
    float y[S][V];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int v = 0; v < V; ++v) y[s][v] = 0.0f;
    dense_apply<LMAX, V, 0>(x, R, cf, y);
#pragma unroll
    for (int s = 0; s < S; ++s) VecIO<T, V>::store(dst + s * C + c0, y[s]);
  }
}

template <int L, typename T>
int dense_go(int V, const EaasArgs& a, const DenseCoef& cf, hipStream_t s) {
  const int64_t per_block = (int64_t)kDenseWaves * (64 >> a.lane_log);
  const dim3 grid((unsigned)((a.n + per_block - 1) / per_block));
  const dim3 blk(64 * kDenseWaves);
  (void)hipGetLastError();
  switch (V) {
    case 1: hipLaunchKernelGGL((k_dense_tp<L, 1, T>), grid, blk, 0, s, a, cf); break;
    case 4: hipLaunchKernelGGL((k_dense_tp<L, 4, T>), grid, blk, 0, s, a, cf); break;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

template <typename T>
int dense_l(int lmax, int V, const EaasArgs& a, const DenseCoef& cf, hipStream_t s) {
  switch (lmax) {
    case 0: return dense_go<0, T>(V, a, cf, s);
    case 1: return dense_go<1, T>(V, a, cf, s);
    case 2: return dense_go<2, T>(V, a, cf, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

static_assert(dense_offset(2, 2, 2, 2) + 125 == kDenseCoefs, "615 entries at lmax = 2");

}  // namespace

int launch_dense(int lmax, int dtype, int V, const EaasArgs& a, const DenseCoef& cf,
                 hipStream_t s) {
  return dtype == 0 ? dense_l<float>(lmax, V, a, cf, s) : dense_l<uint16_t>(lmax, V, a, cf, s);
}

}  // namespace e2f
