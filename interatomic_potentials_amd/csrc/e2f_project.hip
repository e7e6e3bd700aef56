// e2f_project.hip -- learned projections fused with the EAAS pre-coupling.
//
// Queries and keys are invariant scalar projections of the l = 0 row
// (gist.science summary of arXiv 2601.16622, technical summary 2.2, Eq. 6):
//   q_i = h_i[l=0] W_Q,   k_i = h_i[l=0] W_K,
// and the values mix channels within each degree, the rotation-equivariant
// linear map of irrep features, before the pre-coupling of the write-up's
// section 2 (EAAS) and section 3.1 (step 1):
//   v_i[l] = h_i[l] W_V[l],   h'_i = v_i (x) R(r_i).
// Everything lands in the attention workspace: row 0 = k, rows 1..S = h',
// and q in the query rows.
//
// The projections are the only dense contraction of the path and run on the
// matrix cores: v_mfma_f32_16x16x4_f32 for fp32 storage and
// v_mfma_f32_16x16x32_bf16 for bf16 storage, accumulating in fp32.
//
// One workgroup = C/16 waves; wave w owns output channels [16 w, 16 w + 16)
// and holds its slices of all weight matrices in registers for the whole
// launch.  Workgroups are persistent and loop over tiles of 16 atoms:
//  1. the tile's h rows (16 consecutive atoms: one contiguous block) are
//     copied into LDS, padded by 16 bytes per atom so that the 16 operand
//     rows of one MFMA read fall into different LDS banks;
//  2. each wave runs the products with the tile as the A operand (row =
//     atom) and its weight slices as B, for all S rows and for q and k;
//  3. q and k go to memory from the accumulators; the value rows go back
//     to LDS as fp32;
//  4. every thread takes (atom, channel) pairs, applies EAAS to the pair's S
//     components and stores the h' rows, consecutive threads on consecutive
//     channels.
// The contraction index is split over the four 16-lane groups of a wave:
// group g covers k in [g C/4, (g+1) C/4).  Any split is valid as long as the
// A and B operands use the same one; this one makes every operand read a
// contiguous, aligned 16-byte access.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Operand fragments of one 16x16 MFMA: KPL contraction values per lane.
template <typename T>
struct Mma;

template <>
struct Mma<float> {
  static constexpr int KPL = 1;
  using Frag = float;
  __device__ static v4f mma(Frag a, Frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  // KPL values starting at p (16-byte aligned when used in groups of four)
  __device__ static Frag load(const float* p) { return *p; }
  __device__ static Frag gather(const float* w, int /*stride*/) { return w[0]; }
};

template <>
struct Mma<uint16_t> {
  static constexpr int KPL = 8;
  using Frag = v8bf;
  __device__ static v4f mma(Frag a, Frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static Frag load(const uint16_t* p) {
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(p));
  }
  // eight values of one weight column, rows stride apart
  __device__ static Frag gather(const uint16_t* w, int stride) {
    v4u u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      u[e] = uint32_t(w[(2 * e) * stride]) | (uint32_t(w[(2 * e + 1) * stride]) << 16);
    return __builtin_bit_cast(v8bf, u);
  }
};

// a wave-uniform value moved to a scalar register
__device__ inline float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ inline void store_elem(float* p, float v) { *p = v; }
__device__ inline void store_elem(uint16_t* p, float v) { *p = f32_to_bf16(v); }

template <int LMAX, typename T, int C>
__global__ __launch_bounds__(C / 16 * 64) void k_proj_eaas(ProjArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  constexpr int NT = C / 16 * 64;           // threads per workgroup
  constexpr int KG = C / 4;                 // contraction values per lane group
  constexpr int KPL = Mma<T>::KPL;
  constexpr int NI = KG / KPL;              // MFMAs per (row, matrix)
  constexpr int NM = 3 + LMAX;              // W_Q, W_K, W_V[0..LMAX]
  constexpr int TA = kProjTileAtoms;
  constexpr int PA = S * C + 16 / (int)sizeof(T);   // LDS pitch of an h row block (elements)
  constexpr int PV = S * C + 4;                     // LDS pitch of a value row block (floats)
  constexpr int CPA = S * C * (int)sizeof(T) / 16;  // 16-byte chunks per atom
  constexpr int PER = (TA * CPA + NT - 1) / NT;     // chunks per thread
  static_assert(KG % KPL == 0, "channel count does not fit the MFMA shape");
  using Frag = typename Mma<T>::Frag;

  __shared__ __align__(16) T sa[TA * PA];
  __shared__ __align__(16) float sv[TA * PV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 15;                // B column / A row (atom of the tile)
  const int g = lane >> 4;                  // lane group: contraction range, output rows 4g..4g+3
  const int c0 = (tid >> 6) * 16;           // this wave's output channels

  // weight slices: wf[m][t] holds W_m[g KG + t KPL + e][c0 + col], e < KPL
  Frag wf[NM][NI];
  {
    const T* wq = static_cast<const T*>(a.w_q);
    const T* wk = static_cast<const T*>(a.w_k);
    const T* wv = static_cast<const T*>(a.w_v);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const T* w = m == 0 ? wq : (m == 1 ? wk : wv + (size_t)(m - 2) * C * C);
#pragma unroll
      for (int t = 0; t < NI; ++t)
        wf[m][t] = Mma<T>::gather(w + (size_t)(g * KG + t * KPL) * C + c0 + col, C);
    }
  }

  const T* h = static_cast<const T*>(a.h);
  T* ws = static_cast<T*>(a.ws);
  T* qo = static_cast<T*>(a.q_out);
  const int64_t ntiles = (a.n + TA - 1) / TA;
  // A tile's rows are loaded into registers one tile ahead: issued after the
  // previous tile's products (when their accumulators are free), they arrive
  // during its EAAS and stores.  Not at fp32 with C = 128, whose weight slices
  // leave no registers for it: there the loads are issued at the tile's start.
  // The buffer range ends at the tile's last atom, so reads past it (a partial
  // last tile) return zeros without a branch.
  constexpr bool AHEAD = !(sizeof(T) == 4 && C >= 128);
  v4u buf[PER];
  auto fetch = [&](int64_t t) {
    const int64_t b0 = t * TA;
    const int nb = (int)(a.n - b0 < TA ? a.n - b0 : TA);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(h + b0 * (int64_t)(S * C), (uint32_t)(nb * CPA * 16));
#pragma unroll
    for (int p = 0; p < PER; ++p)
      buf[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + p * NT) * 16, 0, 0);
  };
  if (AHEAD && (int64_t)blockIdx.x < ntiles) fetch(blockIdx.x);
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t a0 = tile * TA;
    const int na = (int)(a.n - a0 < TA ? a.n - a0 : TA);

    // 1. stage the tile's rows in LDS
    {
      if (!AHEAD) fetch(tile);
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int q = tid + p * NT;
        if (PER * NT == TA * CPA || q < TA * CPA)
          *reinterpret_cast<v4u*>(reinterpret_cast<char*>(sa) + (q / CPA) * (PA * (int)sizeof(T)) +
                                  (q % CPA) * 16) = buf[p];
      }
    }
    __syncthreads();

    // 2. products: acc[s] = v rows, acc[S] = q, acc[S + 1] = k
    v4f acc[S + 2];
#pragma unroll
    for (int s = 0; s < S + 2; ++s) acc[s] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int l = s < 1 ? 0 : (s < 4 ? 1 : 2);
      const T* arow = sa + col * PA + s * C + g * KG;
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        const Frag af = Mma<T>::load(arow + t * KPL);
        acc[s] = Mma<T>::mma(af, wf[2 + l][t], acc[s]);
        if (s == 0) {
          acc[S] = Mma<T>::mma(af, wf[0][t], acc[S]);
          acc[S + 1] = Mma<T>::mma(af, wf[1][t], acc[S + 1]);
        }
      }
    }

    // 3. q and k straight out; value rows to LDS (fp32).  sv was last read in
    //    step 4 of the previous tile, before this tile's barrier.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;              // output row = atom of the tile
      if (i < na) {
        const int64_t atom = a0 + i;
        store_elem(qo + atom * C + c0 + col, acc[S][r]);
        store_elem(ws + atom * (int64_t)((S + 1) * C) + c0 + col, acc[S + 1][r]);
      }
#pragma unroll
      for (int s = 0; s < S; ++s) sv[i * PV + s * C + c0 + col] = acc[s][r];
    }
    if (AHEAD && tile + gridDim.x < ntiles) fetch(tile + gridDim.x);
    __syncthreads();

    // 4. EAAS per (atom, channel); stores coalesced along the channels
    for (int p = tid; p < TA * C; p += NT) {
      const int i = p / C;
      const int c = p - i * C;
      if (i >= na) break;
      const int64_t atom = a0 + i;
      Frame f = make_frame(a.r[3 * atom], a.r[3 * atom + 1], a.r[3 * atom + 2]);
      Dy2 d = make_dy2(f);
      Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
      if constexpr (C % 64 == 0) {
        // the wave's 64 lanes share one atom: hold its frame and reindex
        // weights in scalar registers (the weight slices fill the vector file)
        f.ct = uni(f.ct); f.st = uni(f.st); f.c1 = uni(f.c1); f.s1 = uni(f.s1);
        f.c2 = uni(f.c2); f.s2 = uni(f.s2); f.r1 = uni(f.r1); f.r2 = uni(f.r2);
        d.d00 = uni(d.d00); d.d01 = uni(d.d01); d.d02 = uni(d.d02);
        d.d11 = uni(d.d11); d.d12 = uni(d.d12); d.d22 = uni(d.d22);
#pragma unroll
        for (int q = 0; q < kMaxPaths; ++q)
#pragma unroll
          for (int m = 0; m <= LMAX; ++m) R.k[q][m] = uni(R.k[q][m]);
      }
      float x[S], y[S];
#pragma unroll
      for (int s = 0; s < S; ++s) x[s] = sv[i * PV + s * C + c];
      eaas_channel<LMAX>(x, y, f, d, R);
      T* dst = ws + atom * (int64_t)((S + 1) * C) + C + c;
#pragma unroll
      for (int s = 0; s < S; ++s) store_elem(dst + s * C, y[s]);
    }
    // the next tile's step 1 overwrites sa, last read in step 2 above (before
    // the barrier that preceded step 4), so no further barrier is needed here
  }
}

template <int LMAX, typename T, int C>
int go(const ProjArgs& a, const EaasCoef& cf, hipStream_t s) {
  const int64_t ntiles = (a.n + kProjTileAtoms - 1) / kProjTileAtoms;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_proj_eaas<LMAX, T, C>, C / 16 * 64,
                                                   0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int64_t cap = (int64_t)cus * per_cu;
  const unsigned grid = (unsigned)(ntiles < cap ? ntiles : cap);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_proj_eaas<LMAX, T, C>), dim3(grid), dim3(C / 16 * 64), 0, s, a, cf);
  return (int)hipGetLastError();
}

template <int LMAX, typename T>
int go_c(int C, const ProjArgs& a, const EaasCoef& cf, hipStream_t s) {
  switch (C) {
    case 16:
      if constexpr (sizeof(T) == 4) return go<LMAX, T, 16>(a, cf, s);
      return (int)hipErrorInvalidValue;
    case 32: return go<LMAX, T, 32>(a, cf, s);
    case 64: return go<LMAX, T, 64>(a, cf, s);
    case 128: return go<LMAX, T, 128>(a, cf, s);
    default: return (int)hipErrorInvalidValue;
  }
}

template <typename T>
int go_l(int lmax, int C, const ProjArgs& a, const EaasCoef& cf, hipStream_t s) {
  switch (lmax) {
    case 0: return go_c<0, T>(C, a, cf, s);
    case 1: return go_c<1, T>(C, a, cf, s);
    default: return go_c<2, T>(C, a, cf, s);
  }
}

}  // namespace

bool proj_supported(int C, int dtype) {
  if (dtype == 0) return C == 16 || C == 32 || C == 64 || C == 128;
  return C == 32 || C == 64 || C == 128;
}

int launch_proj(int lmax, int dtype, int C, const ProjArgs& a, const EaasCoef& cf,
                hipStream_t s) {
  if (a.n == 0) return 0;
  return dtype == 0 ? go_l<float>(lmax, C, a, cf, s) : go_l<uint16_t>(lmax, C, a, cf, s);
}

}  // namespace e2f
