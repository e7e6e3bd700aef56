// e2f_project_bwd.hip -- gradients through the learned projections (fp32).
//
// The projections of the layer (gist.science summary of arXiv 2601.16622,
// technical summary 2.2, Eq. 6, with the values mixed per degree):
//   q_i = h_i[0] W_Q,   k_i = h_i[0] W_K,   v_i[l] = h_i[l] W_V[l].
// The attention's backward passes deliver dq, dk ([N, C]) and dv ([N, S, C],
// the adjoint of the pre-coupling applied to dh').  Through the projections:
//   dh_i[l = 0] = dv_i[0] W_V[0]^T + dq_i W_Q^T + dk_i W_K^T
//   dh_i[l > 0] = dv_i[l] W_V[l]^T                       (per component m)
//   dW_Q = sum_i h_i[0]^T dq_i,   dW_K = sum_i h_i[0]^T dk_i,
//   dW_V[l] = sum_i sum_m h_i[l, m]^T dv_i[l, m].
// The value rows v themselves are recomputed here too: the position gradient
// of the pre-coupling needs them.
//
// Row products (k_rows_w): the layout of the forward's projection kernel.
// One workgroup = C/16 waves, wave w owns output channels [16 w, 16 w + 16)
// and holds its slices of the weight matrices (W, or W^T for the gradient)
// in registers; workgroups are persistent over tiles of 16 atoms whose input
// rows are staged in LDS and form the A operand of v_mfma_f32_16x16x4_f32.
//
// Weight gradients (k_dw): a plain reduction over rows, one wave per
// (matrix, 64x64 output tile, chunk of rows), the rows read straight from
// memory, 4 rows per MFMA.  Lane (c, g) loads 4 consecutive columns of row
// g of the step (16-byte loads), so MFMA block e covers the columns 4 i + e:
// a permutation of the output tile, undone at the store.  Every chunk writes
// its own partial matrix, and k_dw_reduce sums the chunks in order: the
// result is the same bit for bit from run to run.
//
// Channel counts without a matrix-core build take plain vector-ALU kernels
// with the same partial layout and the same reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ inline v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline void put(float* p, float v) { *p = v; }
__device__ inline void put(uint16_t* p, float v) { *p = f32_to_bf16(v); }

constexpr int kRowTile = 16;   // atoms per tile of the row products

// ------------------------------------------------------------ row products

// GRAD = false: out[i, s] = x[i, s] W_V[l(s)]                       (values)
// GRAD = true:  out[i, s] = x[i, s] W_V[l(s)]^T, and for s = 0 also
//               + dq_i W_Q^T + dk_i W_K^T                           (dL/dh)
template <int LMAX, int C, bool GRAD, typename TO>
__global__ __launch_bounds__(C / 16 * 64) void k_rows_w(RowsArgs a) {
  constexpr int S = ncomp(LMAX);
  constexpr int NT = C / 16 * 64;
  constexpr int KG = C / 4;                     // contraction values per lane group
  constexpr int NR = GRAD ? S + 2 : S;          // staged rows per atom: x, then dq and dk
  constexpr int NM = GRAD ? LMAX + 3 : LMAX + 1;   // W_V[0..LMAX], then W_Q and W_K
  constexpr int TA = kRowTile;
  constexpr int PA = NR * C + 4;                // LDS pitch of an atom (floats)
  constexpr int CPA = NR * C / 4;               // 16-byte chunks per atom
  __shared__ __align__(16) float sa[TA * PA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 15;                    // A row (atom of the tile) / B column
  const int g = lane >> 4;                      // contraction range, output rows 4g..4g+3
  const int c0 = (tid >> 6) * 16;               // this wave's output channels

  // wf[m][t] = B_m[g KG + t][c0 + col], B = W (values) or W^T (gradients)
  float wf[NM][KG];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const float* w = m <= LMAX ? a.w_v + (size_t)m * C * C : (m == LMAX + 1 ? a.w_q : a.w_k);
#pragma unroll
    for (int t = 0; t < KG; ++t)
      wf[m][t] = GRAD ? w[(size_t)(c0 + col) * C + g * KG + t] : w[(size_t)(g * KG + t) * C + c0 + col];
  }

  const int64_t ntiles = (a.n + TA - 1) / TA;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t a0 = tile * TA;
    const int na = (int)(a.n - a0 < TA ? a.n - a0 : TA);
    // 1. stage the tile's rows (zeros past the last atom)
    for (int q = tid; q < TA * CPA; q += NT) {
      const int i = q / CPA;
      const int e = q - i * CPA;
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (i < na) {
        const int64_t atom = a0 + i;
        if (e < S * C / 4)
          v = *reinterpret_cast<const float4*>(a.x + atom * (int64_t)(S * C) + 4 * e);
        else if (e < (S + 1) * C / 4)
          v = *reinterpret_cast<const float4*>(a.dq + atom * C + 4 * (e - S * C / 4));
        else
          v = *reinterpret_cast<const float4*>(a.dk + atom * C + 4 * (e - (S + 1) * C / 4));
      }
      *reinterpret_cast<float4*>(sa + i * PA + 4 * e) = v;
    }
    __syncthreads();

    // 2. products
    v4f acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) acc[s] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int l = s < 1 ? 0 : (s < 4 ? 1 : 2);
      const float* arow = sa + col * PA + s * C + g * KG;
#pragma unroll
      for (int t = 0; t < KG; ++t) acc[s] = mfma4(arow[t], wf[l][t], acc[s]);
    }
    if constexpr (GRAD) {
      const float* qrow = sa + col * PA + S * C + g * KG;
      const float* krow = qrow + C;
#pragma unroll
      for (int t = 0; t < KG; ++t) {
        acc[0] = mfma4(qrow[t], wf[LMAX + 1][t], acc[0]);
        acc[0] = mfma4(krow[t], wf[LMAX + 2][t], acc[0]);
      }
    }

    // 3. results straight from the accumulators
    TO* out = static_cast<TO*>(a.out);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      if (i < na) {
        TO* dst = out + (a0 + i) * (int64_t)(S * C) + c0 + col;
#pragma unroll
        for (int s = 0; s < S; ++s) put(dst + s * C, acc[s][r]);
      }
    }
    __syncthreads();   // every read of sa is done before the next tile is staged
  }
}

// Any C: one workgroup per atom, thread c computes output channel c, input
// channels summed in order.
template <int LMAX, bool GRAD, typename TO>
__global__ __launch_bounds__(256) void k_rows_generic(RowsArgs a, int C) {
  constexpr int S = ncomp(LMAX);
  constexpr int NR = GRAD ? S + 2 : S;
  extern __shared__ float s_x[];   // [NR, C] of this atom
  const int64_t atom = blockIdx.x;
  if (atom >= a.n) return;
  for (int e = threadIdx.x; e < NR * C; e += blockDim.x) {
    float v;
    if (e < S * C)
      v = a.x[atom * (int64_t)(S * C) + e];
    else if (e < (S + 1) * C)
      v = a.dq[atom * C + e - S * C];
    else
      v = a.dk[atom * C + e - (S + 1) * C];
    s_x[e] = v;
  }
  __syncthreads();
  TO* dst = static_cast<TO*>(a.out) + atom * (int64_t)(S * C);
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float y[S];
#pragma unroll
    for (int s = 0; s < S; ++s) y[s] = 0.0f;
#pragma unroll
    for (int l = 0; l <= LMAX; ++l) {
      const float* w = a.w_v + (size_t)l * C * C;
      for (int i = 0; i < C; ++i) {
        const float b = GRAD ? w[(size_t)c * C + i] : w[(size_t)i * C + c];
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m) y[l * l + m] = fmaf(s_x[(l * l + m) * C + i], b, y[l * l + m]);
      }
    }
    if constexpr (GRAD) {
      for (int i = 0; i < C; ++i) {
        y[0] = fmaf(s_x[S * C + i], a.w_q[(size_t)c * C + i], y[0]);
        y[0] = fmaf(s_x[(S + 1) * C + i], a.w_k[(size_t)c * C + i], y[0]);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) put(dst + s * C + c, y[s]);
  }
}

// ------------------------------------------------------- weight gradients

// the job and chunk of partial-matrix slot `unit`, and the output tile
__device__ inline bool dw_locate(const DwArgs& a, int64_t unit, int tiles2, int& jb, int64_t& chunk,
                                 int& tile) {
  for (jb = 0; jb < a.njobs; ++jb) {
    const int64_t n = (int64_t)a.job[jb].chunks * tiles2;
    if (unit < n) {
      chunk = unit / tiles2;
      tile = (int)(unit - chunk * tiles2);
      return true;
    }
    unit -= n;
  }
  return false;
}

// row r of a job: atom r / mult, component r % mult of the job's degree
__device__ inline int64_t dw_row(const DwJob& j, int64_t r, int64_t stride) {
  const int64_t n = r / j.mult;
  return n * stride + (r - n * j.mult) * j.C;
}

constexpr int kDwAhead = 4;   // row steps in flight per wave

// TM x TM output tile a wave (TM = min(C, 64)), 4 rows per MFMA
template <int C>
__global__ __launch_bounds__(256) void k_dw(DwArgs a) {
  constexpr int TM = C < 64 ? C : 64;
  constexpr int TPD = C / TM;                   // tiles per dimension
  constexpr int FB = TM / 16;                   // 16-column blocks per tile side
  constexpr int VW = TM / 16;                   // consecutive columns a lane loads (FB of them)
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int jb, tile;
  int64_t chunk;
  if (!dw_locate(a, unit, TPD * TPD, jb, chunk, tile)) return;   // whole wave
  const DwJob& J = a.job[jb];
  const int ta = tile / TPD, tb = tile - ta * TPD;
  const int a0 = ta * TM + VW * col;            // this lane's first column of X
  const int b0 = tb * TM + VW * col;            // and of dY
  const int64_t r_begin = chunk * J.chunk_rows;
  const int64_t r_end = r_begin + J.chunk_rows < J.rows ? r_begin + J.chunk_rows : J.rows;

  v4f acc[FB][FB];
#pragma unroll
  for (int e = 0; e < FB; ++e)
#pragma unroll
    for (int f = 0; f < FB; ++f) acc[e][f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // The next row this lane fetches, r = (atom n, component m), advanced 4 rows a step
  // without a division: the row offsets move by 4 C inside an atom and by the atom
  // stride less mult C at each wrap (at most four wraps a step, at mult = 1).
  int64_t r = r_begin + g;
  int64_t n = r / J.mult;
  int m = (int)(r - n * J.mult);
  int64_t ox = n * J.xs + (int64_t)m * J.C + a0;
  int64_t oy = n * J.ys + (int64_t)m * J.C + b0;
  const int64_t wx = J.xs - (int64_t)J.mult * J.C, wy = J.ys - (int64_t)J.mult * J.C;
  auto fetch = [&](float (&xa)[VW], float (&yb)[VW]) {
    if (r < r_end) {
      VecIO<float, VW>::load(J.x + ox, xa);
      VecIO<float, VW>::load(J.dy + oy, yb);
    } else {
#pragma unroll
      for (int e = 0; e < VW; ++e) xa[e] = yb[e] = 0.0f;
    }
    r += 4;
    m += 4;
    ox += 4 * J.C;
    oy += 4 * J.C;
    while (m >= J.mult) {
      m -= J.mult;
      ox += wx;
      oy += wy;
    }
  };
  // kDwAhead steps of 4 rows in flight: step p of a group is used, then refilled with the
  // step kDwAhead later
  float xa[kDwAhead][VW], yb[kDwAhead][VW];
#pragma unroll
  for (int p = 0; p < kDwAhead; ++p) fetch(xa[p], yb[p]);
  for (int64_t r0 = r_begin; r0 < r_end; r0 += 4 * kDwAhead) {
#pragma unroll
    for (int p = 0; p < kDwAhead; ++p) {
#pragma unroll
      for (int e = 0; e < FB; ++e)
#pragma unroll
        for (int f = 0; f < FB; ++f) acc[e][f] = mfma4(xa[p][e], yb[p][f], acc[e][f]);
      fetch(xa[p], yb[p]);
    }
  }
  // block (e, f), element r of lane (col, g): row 4g + r of block e is column
  // VW (4g + r) + e of the tile's X side; column col of block f is VW col + f
  float* P = a.partial + (J.part_off + chunk) * (int64_t)(C * C);
#pragma unroll
  for (int e = 0; e < FB; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ia = ta * TM + VW * (4 * g + r) + e;
      float v[VW];
#pragma unroll
      for (int f = 0; f < FB; ++f) v[f] = acc[e][f][r];
      VecIO<float, VW>::store(P + (int64_t)ia * C + b0, v);
    }
}

// Any C: 16x16 output tile per workgroup, thread (ia, ib), rows of the chunk in order.
__global__ __launch_bounds__(256) void k_dw_generic(DwArgs a, int C) {
  const int tpd = (C + 15) / 16;
  int jb, tile;
  int64_t chunk;
  if (!dw_locate(a, blockIdx.x, tpd * tpd, jb, chunk, tile)) return;
  const DwJob& J = a.job[jb];
  const int ia = (tile / tpd) * 16 + (threadIdx.x >> 4);
  const int ib = (tile % tpd) * 16 + (threadIdx.x & 15);
  const int64_t r_begin = chunk * J.chunk_rows;
  const int64_t r_end = r_begin + J.chunk_rows < J.rows ? r_begin + J.chunk_rows : J.rows;
  if (ia >= C || ib >= C) return;
  float acc = 0.0f;
  for (int64_t r = r_begin; r < r_end; ++r)
    acc = fmaf(J.x[dw_row(J, r, J.xs) + ia], J.dy[dw_row(J, r, J.ys) + ib], acc);
  a.partial[(J.part_off + chunk) * (int64_t)C * C + (int64_t)ia * C + ib] = acc;
}

// out_j[e] = sum over the job's chunks, in order
__global__ __launch_bounds__(256) void k_dw_reduce(DwArgs a) {
  const int64_t cc = (int64_t)a.C * a.C;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int jb = blockIdx.y;
  if (e >= cc || jb >= a.njobs) return;
  const DwJob& J = a.job[jb];
  const float* p = a.partial + J.part_off * cc + e;
  // eight loads in flight, added in chunk order
  float s = 0.0f;
  int c = 0;
  for (; c + 8 <= J.chunks; c += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[(int64_t)(c + k) * cc];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; c < J.chunks; ++c) s += p[(int64_t)c * cc];
  J.out[e] = s;
}

int persistent_grid(const void* fn, int threads, int64_t tiles) {
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int64_t cap = (int64_t)cus * per_cu;
  return (int)(tiles < cap ? tiles : cap);
}

template <int LMAX, int C, bool GRAD, typename TO>
int rows_go(const RowsArgs& a, hipStream_t s) {
  const int64_t ntiles = (a.n + kRowTile - 1) / kRowTile;
  const void* fn = reinterpret_cast<const void*>(&k_rows_w<LMAX, C, GRAD, TO>);
  const int grid = persistent_grid(fn, C / 16 * 64, ntiles);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_rows_w<LMAX, C, GRAD, TO>), dim3(grid), dim3(C / 16 * 64), 0, s, a);
  return (int)hipGetLastError();
}

template <int LMAX, bool GRAD, typename TO>
int rows_c(int C, const RowsArgs& a, hipStream_t s) {
  switch (C) {
    case 16: return rows_go<LMAX, 16, GRAD, TO>(a, s);
    case 32: return rows_go<LMAX, 32, GRAD, TO>(a, s);
    case 64: return rows_go<LMAX, 64, GRAD, TO>(a, s);
    case 128: return rows_go<LMAX, 128, GRAD, TO>(a, s);
    default: break;
  }
  const int threads = C < 256 ? (C + 63) / 64 * 64 : 256;
  const size_t lds = (size_t)(GRAD ? ncomp(LMAX) + 2 : ncomp(LMAX)) * C * sizeof(float);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_rows_generic<LMAX, GRAD, TO>), dim3((unsigned)a.n), dim3(threads), lds, s,
                     a, C);
  return (int)hipGetLastError();
}

template <bool GRAD, typename TO>
int rows_l(int lmax, int C, const RowsArgs& a, hipStream_t s) {
  switch (lmax) {
    case 0: return rows_c<0, GRAD, TO>(C, a, s);
    case 1: return rows_c<1, GRAD, TO>(C, a, s);
    case 2: return rows_c<2, GRAD, TO>(C, a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

bool rows_mfma(int C) { return C == 16 || C == 32 || C == 64 || C == 128; }

int launch_value_rows(int lmax, int C, const RowsArgs& a, hipStream_t s) {
  if (a.n == 0) return 0;
  return rows_l<false, float>(lmax, C, a, s);
}

int launch_grad_rows(int lmax, int C, int dtype, const RowsArgs& a, hipStream_t s) {
  if (a.n == 0) return 0;
  return dtype == 0 ? rows_l<true, float>(lmax, C, a, s) : rows_l<true, uint16_t>(lmax, C, a, s);
}

int launch_weight_grads(const DwArgs& a, hipStream_t s) {
  int64_t units = 0;
  const int C = a.C;
  const bool mfma = rows_mfma(C);
  const int tpd = mfma ? (C < 64 ? 1 : C / 64) : (C + 15) / 16;
  for (int j = 0; j < a.njobs; ++j) units += (int64_t)a.job[j].chunks * tpd * tpd;
  (void)hipGetLastError();
  if (mfma) {
    const dim3 grid((unsigned)((units + 3) / 4));
    switch (C) {
      case 16: hipLaunchKernelGGL((k_dw<16>), grid, dim3(256), 0, s, a); break;
      case 32: hipLaunchKernelGGL((k_dw<32>), grid, dim3(256), 0, s, a); break;
      case 64: hipLaunchKernelGGL((k_dw<64>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((k_dw<128>), grid, dim3(256), 0, s, a); break;
    }
  } else {
    hipLaunchKernelGGL(k_dw_generic, dim3((unsigned)units), dim3(256), 0, s, a, C);
  }
  int st = (int)hipGetLastError();
  if (st != 0) return st;
  const int64_t cc = (int64_t)C * C;
  hipLaunchKernelGGL(k_dw_reduce, dim3((unsigned)((cc + 255) / 256), (unsigned)a.njobs), dim3(256),
                     0, s, a);
  return (int)hipGetLastError();
}

}  // namespace e2f
