// e2f_neighbours.hip -- padded neighbour lists on the GPU (cell list), and
// the atoms grouped by cell in Morton order.
//
// The attention takes each target's neighbours as a padded index row plus a
// mask (E2Former-V2 write-up, section 3.2) within the edge cutoff (section
// 5.1).  Definition, shared with the float64 CPU reference: the neighbours
// of i are the j != i with
//   d2 = ((dx*dx + dy*dy) + dz*dz) < rc*rc      (float64, one rounding per
//   operation, d_ = p_i - p_j formed from the float32 positions),
// listed by increasing (d2, j), the first K kept; the rest of the row holds
// index -1 and mask 0; n_within counts all of them.
//
// Passes:
//  1. bounding box: block partials, then one block that lays out a grid of
//     cells no smaller than rc (times 1 + 2^-20) per axis and at most
//     2^bmax per axis, so every pair closer than rc lies in the same or
//     adjacent cells; cells are numbered by their Morton code;
//  2. per atom its cell, counted with an atomic add;
//  3. exclusive scan of the counts: cell starts;
//  4. scatter: atoms grouped by cell, positions copied beside them so the
//     candidate loop reads them contiguously;
//  5. one wavefront per target, targets in the grouped order (neighbouring
//     waves share cells in cache): the 27 cells around the target's cell are
//     flattened into one stream of candidates, read 64 at a time (the next 64
//     in flight while the current ones are tested); accepted (d2, j) pairs are compacted into
//     LDS with a ballot; when the LDS batch is full, and at the end, the kept
//     pairs and the batch are sorted by (d2, j) with a bitonic network and the
//     first K are kept.  The result does not depend on the order of atoms
//     within a cell (which the atomic scatter leaves open).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "e2f_internal.hpp"

namespace e2f {
namespace {

struct NlGrid {
  double lo[3];     // bounding-box minimum
  double side[3];   // cell side per axis (>= rc)
  int dims[3];      // cells per axis
  int bits;         // Morton bits per axis
};

// One target (wave) a workgroup: candidate counts vary, and a workgroup's LDS
// is freed only when its last wave ends (Large 0.35 -> 0.32 ms against four).
constexpr int kNlWaves = 1;   // targets per workgroup
constexpr int kNlAhead = 3;   // candidate batches in flight per wave

__device__ inline uint32_t spread3(uint32_t v) {  // bits b -> 3b
  v &= 0x3ffu;
  v = (v | (v << 16)) & 0x030000ffu;
  v = (v | (v << 8)) & 0x0300f00fu;
  v = (v | (v << 4)) & 0x030c30c3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}

__device__ inline uint32_t compact3(uint32_t v) {  // 3b -> b
  v &= 0x09249249u;
  v = (v | (v >> 2)) & 0x030c30c3u;
  v = (v | (v >> 4)) & 0x0300f00fu;
  v = (v | (v >> 8)) & 0x030000ffu;
  v = (v | (v >> 16)) & 0x3ffu;
  return v;
}

__device__ inline int32_t morton(int x, int y, int z) {
  return (int32_t)(spread3((uint32_t)x) | (spread3((uint32_t)y) << 1) | (spread3((uint32_t)z) << 2));
}

__device__ inline void nl_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(256) void k_nl_fill(int64_t n, int32_t* p, int32_t v) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = v;
}

// 1a. per-block (min, max) of the positions
__global__ __launch_bounds__(256) void k_nl_bbox(int64_t n, const float* pos, float* partial) {
  __shared__ float red[6][256];
  const int t = threadIdx.x;
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int64_t i = (int64_t)blockIdx.x * 256 + t; i < n; i += (int64_t)gridDim.x * 256) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float v = pos[3 * i + d];
      mn[d] = fminf(mn[d], v);
      mx[d] = fmaxf(mx[d], v);
    }
  }
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    red[d][t] = mn[d];
    red[3 + d][t] = mx[d];
  }
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) {
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        red[d][t] = fminf(red[d][t], red[d][t + o]);
        red[3 + d][t] = fmaxf(red[3 + d][t], red[3 + d][t + o]);
      }
    }
    __syncthreads();
  }
  if (t < 6) partial[blockIdx.x * 6 + t] = red[t][0];
}

// 1b. reduce the partials and lay out the grid (one block)
__global__ __launch_bounds__(256) void k_nl_grid(int nparts, const float* partial, double rc,
                                                 int bmax, NlGrid* grid) {
  __shared__ float red[6][256];
  const int t = threadIdx.x;
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int b = t; b < nparts; b += 256) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      mn[d] = fminf(mn[d], partial[b * 6 + d]);
      mx[d] = fmaxf(mx[d], partial[b * 6 + 3 + d]);
    }
  }
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    red[d][t] = mn[d];
    red[3 + d][t] = mx[d];
  }
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) {
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        red[d][t] = fminf(red[d][t], red[d][t + o]);
        red[3 + d][t] = fmaxf(red[3 + d][t], red[3 + d][t + o]);
      }
    }
    __syncthreads();
  }
  if (t == 0) {
    const double side_min = rc * (1.0 + 1.0 / 1048576.0);   // margin over rounding in step 2
    int dmax = 1;
    for (int d = 0; d < 3; ++d) {
      const double lo = (double)red[d][0], ext = (double)red[3 + d][0] - lo;
      double nc = floor(ext / side_min);
      const double cap = (double)(1 << bmax);
      nc = nc < 1.0 ? 1.0 : (nc > cap ? cap : nc);
      grid->lo[d] = lo;
      grid->dims[d] = (int)nc;
      grid->side[d] = ext > 0.0 ? ext / nc : 1.0;
      dmax = grid->dims[d] > dmax ? grid->dims[d] : dmax;
    }
    int bits = 0;
    while ((1 << bits) < dmax) ++bits;
    grid->bits = bits;
  }
}

__device__ inline int cell_coord(float x, const NlGrid& g, int d) {
  int c = (int)floor(((double)x - g.lo[d]) / g.side[d]);
  return c < 0 ? 0 : (c >= g.dims[d] ? g.dims[d] - 1 : c);
}

// 2. cell of every atom, counted
__global__ __launch_bounds__(256) void k_nl_cells(int64_t n, const float* pos, const NlGrid* gp,
                                                  int32_t* cell, int32_t* counts) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const NlGrid g = *gp;
  const int32_t c = morton(cell_coord(pos[3 * i], g, 0), cell_coord(pos[3 * i + 1], g, 1),
                           cell_coord(pos[3 * i + 2], g, 2));
  cell[i] = c;
  atomicAdd(&counts[c], 1);
}

// 4. atoms grouped by cell; their positions beside them
__global__ __launch_bounds__(256) void k_nl_scatter(int64_t n, const float* pos,
                                                    const int32_t* cell, int32_t* cursor,
                                                    int32_t* sorted_idx, float4* sorted_pos) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t p = atomicAdd(&cursor[cell[i]], 1);
  sorted_idx[p] = (int32_t)i;
  sorted_pos[p] = make_float4(pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], 0.0f);
}

// (d2, j) order; padding entries carry the largest key
__device__ inline bool pair_less(uint64_t da, int32_t ja, uint64_t db, int32_t jb) {
  return da < db || (da == db && ja < jb);
}

// sort kd/kj[0, cnt) ascending by (d2, j): one wave, bitonic, LDS; each lane
// takes compare-exchange pairs (lo, lo + jj) directly, so no lane idles
__device__ inline void sort_pairs(uint64_t* kd, int32_t* kj, int cnt, int lane) {
  int n2 = 1;
  while (n2 < cnt) n2 <<= 1;
  for (int e = cnt + lane; e < n2; e += 64) {
    kd[e] = ~0ull;
    kj[e] = 0x7fffffff;
  }
  nl_wave_sync();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int e = lane; e < (n2 >> 1); e += 64) {
        const int lo = ((e & ~(jj - 1)) << 1) | (e & (jj - 1));
        const int hi = lo + jj;
        const uint64_t da = kd[lo], db = kd[hi];
        const int32_t ja = kj[lo], jb = kj[hi];
        const bool up = (lo & k) == 0;
        if (up ? pair_less(db, jb, da, ja) : pair_less(da, ja, db, jb)) {
          kd[lo] = db; kd[hi] = da;
          kj[lo] = jb; kj[hi] = ja;
        }
      }
      nl_wave_sync();
    }
  }
}

// 5. one wave per target
template <int LCAP>
__global__ __launch_bounds__(kNlWaves * 64) void k_nl_build(NlArgs a, const NlGrid* gp) {
#pragma clang fp contract(off)
  __shared__ uint64_t skd[kNlWaves][LCAP];
  __shared__ int32_t skj[kNlWaves][LCAP];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t slot = (int64_t)blockIdx.x * kNlWaves + w;
  if (slot >= a.N) return;
  const NlGrid g = *gp;
  uint64_t* kd = skd[w];
  int32_t* kj = skj[w];
  const int32_t i = a.sorted_idx[slot];
  const float4 pi = reinterpret_cast<const float4*>(a.sorted_pos)[slot];
  const double xi = (double)pi.x, yi = (double)pi.y, zi = (double)pi.z;
  const double rc2 = a.rc * a.rc;
  const int32_t ci = a.cell[i];
  const int cx = (int)compact3((uint32_t)ci), cy = (int)compact3((uint32_t)ci >> 1),
            cz = (int)compact3((uint32_t)ci >> 2);
  const int K = a.K;
  int kept = 0;     // sorted pairs at [0, kept)
  int nb = 0;       // unsorted batch at [kept, kept + nb)
  int total = 0;    // all accepted

  // The 27 surrounding cells' ranges, flattened into one candidate stream: lane
  // c < 27 holds cell c's start and its offset in the stream, so every batch of
  // 64 candidates is full whatever the cell sizes.
  int cbeg = 0, clen = 0;
  if (lane < 27) {
    const int x = cx + lane % 3 - 1, y = cy + (lane / 3) % 3 - 1, z = cz + lane / 9 - 1;
    if (x >= 0 && x < g.dims[0] && y >= 0 && y < g.dims[1] && z >= 0 && z < g.dims[2]) {
      const int32_t c = morton(x, y, z);
      cbeg = a.starts[c];
      clen = a.starts[c + 1] - cbeg;
    }
  }
  int coff = clen;   // inclusive scan over the 27 lanes, then exclusive
  for (int o = 1; o < 32; o <<= 1) {
    const int v = __shfl_up(coff, o);
    if (lane >= o) coff += v;
  }
  const int ncand = __builtin_amdgcn_readfirstlane(__shfl(coff, 26));   // wave-uniform
  coff -= clen;
  // candidate e of the stream: its cell is the last c < 27 with offset <= e.
  // Every lane shuffles at every step (a lane that skips a shuffle does not
  // provide its own value to the others), so the source lane is clamped and
  // only the comparison is conditional.
  auto locate = [&](int e) -> int32_t {
    int c = 0;
#pragma unroll
    for (int k = 16; k > 0; k >>= 1) {
      const int t = c + k;
      const int ot = __shfl(coff, t < 27 ? t : 26);
      if (t < 27 && ot <= e) c = t;
    }
    return __shfl(cbeg, c) + (e - __shfl(coff, c));
  };
  // kNlAhead batches of loads in flight.  The loop is unrolled by kNlAhead so
  // that each register slot is tested and refilled in place (copying a slot
  // whose load is still in flight would wait for it).  locate() shuffles, so
  // every lane calls it.
  float4 qr[kNlAhead];
  int32_t jr[kNlAhead];
  auto fetch = [&](int B, float4& q, int32_t& j) {
    const int e = B + lane;
    const int32_t pidx = locate(e < ncand ? e : 0);
    if (e < ncand) {
      q = reinterpret_cast<const float4*>(a.sorted_pos)[pidx];
      j = a.sorted_idx[pidx];
    }
  };
#pragma unroll
  for (int d = 0; d < kNlAhead; ++d) {
    qr[d] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    jr[d] = -1;
    if (64 * d < ncand) fetch(64 * d, qr[d], jr[d]);
  }
  for (int b0 = 0; b0 < ncand; b0 += 64 * kNlAhead) {
#pragma unroll
    for (int d = 0; d < kNlAhead; ++d) {
      const int B = b0 + 64 * d;
      if (B >= ncand) break;
      const float4 q = qr[d];
      const int32_t j = jr[d];
      if (B + 64 * kNlAhead < ncand) fetch(B + 64 * kNlAhead, qr[d], jr[d]);
      bool ok = false;
      double d2 = 0.0;
      if (B + lane < ncand) {
        const double ex = xi - (double)q.x, ey = yi - (double)q.y, ez = zi - (double)q.z;
        d2 = (ex * ex + ey * ey) + ez * ez;
        ok = j != i && d2 < rc2;
      }
      const uint64_t bal = __ballot(ok);
      const int add = __popcll(bal);
      if (add != 0) {
        if (kept + nb + add > LCAP) {   // make room: keep the K nearest so far
          sort_pairs(kd, kj, kept + nb, lane);
          kept = kept + nb < K ? kept + nb : K;
          nb = 0;
        }
        if (ok) {
          const int at = kept + nb + __popcll(bal & ((1ull << lane) - 1ull));
          kd[at] = (uint64_t)__double_as_longlong(d2);
          kj[at] = j;
        }
        nb += add;
        total += add;
        nl_wave_sync();
      }
    }
  }
  sort_pairs(kd, kj, kept + nb, lane);
  kept = kept + nb < K ? kept + nb : K;
  int32_t* irow = a.idx + (int64_t)i * K;
  uint8_t* mrow = a.mask + (int64_t)i * K;
  for (int k = lane; k < K; k += 64) {
    irow[k] = k < kept ? kj[k] : -1;
    mrow[k] = k < kept ? 1 : 0;
  }
  if (a.n_within && lane == 0) a.n_within[i] = total;
}

int nl_err() { return static_cast<int>(hipGetLastError()); }

}  // namespace

int launch_neighbours(const NlArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  const int64_t cells = (int64_t)1 << (3 * a.bmax);
  const unsigned gn = (unsigned)((a.N + 255) / 256);
  NlGrid* grid = static_cast<NlGrid*>(a.grid);
  const int nparts = a.N < (int64_t)kBboxBlocks * 256 ? (int)((a.N + 255) / 256) : kBboxBlocks;
  hipLaunchKernelGGL(k_nl_bbox, dim3(nparts), dim3(256), 0, s, a.N, a.pos, a.partial);
  hipLaunchKernelGGL(k_nl_grid, dim3(1), dim3(256), 0, s, nparts, a.partial, a.rc, a.bmax, grid);
  hipLaunchKernelGGL(k_nl_fill, dim3((unsigned)((cells + 1 + 255) / 256)), dim3(256), 0, s,
                     cells + 1, a.starts, 0);
  hipLaunchKernelGGL(k_nl_cells, dim3(gn), dim3(256), 0, s, a.N, a.pos, grid, a.cell, a.starts);
  int st = launch_scan_exclusive(cells, a.starts, a.tile_sums, a.cursor, s);
  if (st != 0) return st;
  hipLaunchKernelGGL(k_nl_scatter, dim3(gn), dim3(256), 0, s, a.N, a.pos, a.cell, a.cursor,
                     a.sorted_idx, reinterpret_cast<float4*>(a.sorted_pos));
  const dim3 gb((unsigned)((a.N + kNlWaves - 1) / kNlWaves));
  if (a.K <= 448)
    hipLaunchKernelGGL(k_nl_build<512>, gb, dim3(kNlWaves * 64), 0, s, a, grid);
  else
    hipLaunchKernelGGL(k_nl_build<2048>, gb, dim3(kNlWaves * 64), 0, s, a, grid);
  if (a.order)
    (void)hipMemcpyAsync(a.order, a.sorted_idx, (size_t)a.N * 4, hipMemcpyDeviceToDevice, s);
  return nl_err();
}

}  // namespace e2f
