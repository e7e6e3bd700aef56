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
//  4. each atom's frame, Wigner blocks and reindex weights are computed once
//     (one thread per atom, during step 3) into an LDS table; every thread
//     then takes (atom, channel) pairs, applies EAAS to the pair's S
//     components and stores the h' rows, consecutive threads on consecutive
//     channels.  With C a multiple of 64 a wave takes whole atoms, and holds
//     the atom's table entry in scalar registers.
// Where the registers allow (every layout but fp32 with C = 128, whose weight
// slices fill the vector file), step 2 runs with the operands swapped,
// D = W^T h^T: each lane then ends with four consecutive output channels of
// one atom, all S components, so steps 3 and 4 run from the accumulators with
// the atom's table entry, without the value rows' trip through LDS.
// Channel counts this kernel is not built for (any other C up to kProjMaxC)
// take a plain vector-ALU kernel, k_proj_generic, with the same arithmetic
// order per output (input channels in order, fp32 accumulation).
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

// one atom's coupling data, computed once per tile and read by every channel
template <int LMAX>
struct __align__(16) AtomFrame {
  Frame f;
  Dy2 d;
  Reindex<LMAX> R;
};

template <int LMAX>
__device__ inline AtomFrame<LMAX> uni(const AtomFrame<LMAX>& e) {
  AtomFrame<LMAX> u;
  u.f.ct = uni(e.f.ct); u.f.st = uni(e.f.st); u.f.c1 = uni(e.f.c1); u.f.s1 = uni(e.f.s1);
  u.f.c2 = uni(e.f.c2); u.f.s2 = uni(e.f.s2); u.f.r1 = uni(e.f.r1); u.f.r2 = uni(e.f.r2);
  u.d.d00 = uni(e.d.d00); u.d.d01 = uni(e.d.d01); u.d.d02 = uni(e.d.d02);
  u.d.d11 = uni(e.d.d11); u.d.d12 = uni(e.d.d12); u.d.d22 = uni(e.d.d22);
#pragma unroll
  for (int q = 0; q < kMaxPaths; ++q)
#pragma unroll
    for (int m = 0; m <= LMAX; ++m) u.R.k[q][m] = uni(e.R.k[q][m]);
  return u;
}

// one element of q or k on the fp32 C = 128 path (the only one that stores element-wise)
__device__ inline void store_elem(float* p, float v) { *p = v; }

// Two waves a SIMD: the weight slices, accumulators and next-tile registers fit in 256
// registers, and the compiler is held to that (it would otherwise spill into AGPRs at C = 64).
template <int LMAX, typename T, int C>
__global__ __launch_bounds__(C / 16 * 64, 2) void k_proj_eaas(ProjArgs a, EaasCoef cf) {
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
  // Where registers allow (all but fp32 with C = 128, whose weight slices fill the vector
  // file), the products run transposed so that each lane ends with whole (atom, channel)
  // columns, and the coupling runs from registers; there the next tile's rows are loaded
  // ahead too.
  constexpr bool TRANS = !(sizeof(T) == 4 && C >= 128);
  constexpr int PER = (TA * CPA + NT - 1) / NT;     // chunks per thread
  static_assert(KG % KPL == 0, "channel count does not fit the MFMA shape");
  using Frag = typename Mma<T>::Frag;

  __shared__ __align__(16) T sa[TA * PA];
  // value rows through LDS on the path that keeps the original MFMA layout (fp32, C = 128)
  __shared__ __align__(16) float sv[TRANS ? 1 : TA * PV];
  // the transposed path's output tile at bf16 storage: per atom its S + 1 workspace
  // rows (k, h') and then its q row, in the storage type, POB bytes apart (32 bytes of
  // padding spread the atoms over the LDS banks).  It goes to memory as whole rows:
  // each wave instruction then writes 1 KB of consecutive bytes, where stores straight
  // from the accumulators would write 32-byte pieces of 16 different atoms' rows.  At
  // fp32 those pieces are 64 bytes and the tile's LDS and registers (the compiler
  // parks accumulators in AGPRs, one wave a SIMD) cost more than they save, so fp32
  // stores straight from the accumulators.
  constexpr bool OTILE = TRANS && sizeof(T) == 2;
  constexpr int CPW = (S + 1) * C * (int)sizeof(T) / 16;   // 16-byte chunks of an atom's rows
  constexpr int CPQ = C * (int)sizeof(T) / 16;             // 16-byte chunks of its q row
  constexpr int POB = (CPW + CPQ) * 16 + 32;
  static_assert(!OTILE || (C * (int)sizeof(T)) % 16 == 0, "rows of whole 16-byte chunks");
  __shared__ __align__(16) char so[OTILE ? TA * POB : 16];
  // frames of FB consecutive tiles of this workgroup: computed by one wave's lanes at
  // once every FB tiles (the computation is a long dependent chain, so 64 frames take
  // hardly longer than 16); two tiles where the tiles' own LDS is largest (fp32, C = 128)
  constexpr int FB = (sizeof(T) == 4 && C >= 128) ? 2 : 4;
  static_assert(FB * TA <= 64, "one wave computes a batch");
  __shared__ AtomFrame<LMAX> sf[FB * TA];

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
  constexpr bool AHEAD = TRANS;
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
  int kb = 0;   // this tile's place in its batch of FB frame tiles
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, kb = (kb + 1) % FB) {
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

    if constexpr (TRANS) {
      // 2. products with the operands swapped (D = W^T h^T): lane (col, g) ends with
      //    output channels c0 + 4g + r (r < 4) of atom col; acc[s] = value row s,
      //    acc[S] = q, acc[S + 1] = k
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
          acc[s] = Mma<T>::mma(wf[2 + l][t], af, acc[s]);
          if (s == 0) {
            acc[S] = Mma<T>::mma(wf[0][t], af, acc[S]);
            acc[S + 1] = Mma<T>::mma(wf[1][t], af, acc[S + 1]);
          }
        }
      }
      // the frames of this tile and the next FB - 1 of the workgroup, at the first tile
      // of each batch (sf was last read in step 4 of the previous tile, before this
      // tile's first barrier)
      if (kb == 0 && tid < FB * TA) {
        const int64_t ft = tile + (int64_t)(tid / TA) * gridDim.x;
        const int64_t atom = ft * TA + tid % TA;
        if (ft < ntiles && atom < a.n) {
          AtomFrame<LMAX> e;
          e.f = make_frame(a.r[3 * atom], a.r[3 * atom + 1], a.r[3 * atom + 2]);
          e.d = make_dy2(e.f);
          e.R = make_reindex<LMAX>(cf, e.f);
          sf[tid] = e;
        }
      }
      __syncthreads();   // sa is free for the next tile's rows; sf is written
      if (tile + gridDim.x < ntiles) fetch(tile + gridDim.x);
      if constexpr (OTILE) {
        // 3-4. q, k and EAAS straight from the accumulators: four consecutive channels of
        //      atom col a lane, into the output tile (so was last read before this
        //      tile's first barrier)
        {
          const int cl = c0 + 4 * g;
          T* orow = reinterpret_cast<T*>(so + col * POB) + cl;
          {
            float o[4] = {acc[S][0], acc[S][1], acc[S][2], acc[S][3]};
            VecIO<T, 4>::store(orow + (S + 1) * C, o);
            float kk[4] = {acc[S + 1][0], acc[S + 1][1], acc[S + 1][2], acc[S + 1][3]};
            VecIO<T, 4>::store(orow, kk);
          }
          const AtomFrame<LMAX> e = sf[kb * TA + col];
          float y[4][S];
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[S];
  #pragma unroll
            for (int s = 0; s < S; ++s) x[s] = acc[s][r];
            eaas_channel<LMAX>(x, y[r], e.f, e.d, e.R);
          }
  #pragma unroll
          for (int s = 0; s < S; ++s) {
            float o[4] = {y[0][s], y[1][s], y[2][s], y[3][s]};
            VecIO<T, 4>::store(orow + (s + 1) * C, o);
          }
        }
        __syncthreads();   // the output tile is complete
        // 5. the tile's rows to memory, 16 bytes a lane: the workspace rows of its
        //    na atoms are one contiguous block, and so are their q rows
        {
          char* wdst = reinterpret_cast<char*>(ws + a0 * (int64_t)((S + 1) * C));
          for (int q = tid; q < na * CPW; q += NT) {
            const int at = q / CPW;
            const int ch = q - at * CPW;
            *reinterpret_cast<v4u*>(wdst + (int64_t)q * 16) =
                *reinterpret_cast<const v4u*>(so + at * POB + ch * 16);
          }
          char* qdst = reinterpret_cast<char*>(qo + a0 * (int64_t)C);
          for (int q = tid; q < na * CPQ; q += NT) {
            const int at = q / CPQ;
            const int ch = q - at * CPQ;
            *reinterpret_cast<v4u*>(qdst + (int64_t)q * 16) =
                *reinterpret_cast<const v4u*>(so + at * POB + (CPW + ch) * 16);
          }
        }
      } else {
        // 3-4. q, k and EAAS straight from the accumulators: four consecutive channels
        //      of atom col a lane, one store of the four per row
        if (col < na) {
          const int64_t atom = a0 + col;
          const int cl = c0 + 4 * g;
          T* wrow = ws + atom * (int64_t)((S + 1) * C) + cl;
          {
            float o[4] = {acc[S][0], acc[S][1], acc[S][2], acc[S][3]};
            VecIO<T, 4>::store(qo + atom * C + cl, o);
            float kk[4] = {acc[S + 1][0], acc[S + 1][1], acc[S + 1][2], acc[S + 1][3]};
            VecIO<T, 4>::store(wrow, kk);
          }
          const AtomFrame<LMAX> e = sf[kb * TA + col];
          float y[4][S];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[S];
#pragma unroll
            for (int s = 0; s < S; ++s) x[s] = acc[s][r];
            eaas_channel<LMAX>(x, y[r], e.f, e.d, e.R);
          }
#pragma unroll
          for (int s = 0; s < S; ++s) {
            float o[4] = {y[0][s], y[1][s], y[2][s], y[3][s]};
            VecIO<T, 4>::store(wrow + (s + 1) * C, o);
          }
        }
      }
    } else {
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
      // the frames of this tile and the next FB - 1 of the workgroup, once per atom, at
      // the first tile of each batch (sf was last read in step 4 of the previous tile,
      // before this tile's first barrier)
      if (kb == 0 && tid < FB * TA) {
        const int64_t ft = tile + (int64_t)(tid / TA) * gridDim.x;
        const int64_t atom = ft * TA + tid % TA;
        if (ft < ntiles && atom < a.n) {
          AtomFrame<LMAX> e;
          e.f = make_frame(a.r[3 * atom], a.r[3 * atom + 1], a.r[3 * atom + 2]);
          e.d = make_dy2(e.f);
          e.R = make_reindex<LMAX>(cf, e.f);
          sf[tid] = e;
        }
      }
      __syncthreads();
      const AtomFrame<LMAX>* tf = sf + kb * TA;   // this tile's frames

      // 4. EAAS per (atom, channel); stores coalesced along the channels
      if constexpr (C % 64 == 0) {
        // a wave takes whole atoms: their table entries go to scalar registers
        // (the weight slices fill the vector file).  Lane l owns the VPL adjacent
        // channels VPL l .. VPL l + VPL - 1, so each component is one LDS read and
        // one store of VPL values a lane.
        constexpr int NW = NT / 64;
        constexpr int VPL = C / 64;
        static_assert(VPL == 1 || VPL == 2, "64 or 128 channels");
        const int c0 = lane * VPL;
        for (int i = tid >> 6; i < na; i += NW) {
          const AtomFrame<LMAX> e = uni<LMAX>(tf[i]);
          const int64_t atom = a0 + i;
          T* dst = ws + atom * (int64_t)((S + 1) * C) + C + c0;
          float x[VPL][S], y[VPL][S];
  #pragma unroll
          for (int s = 0; s < S; ++s) {
            const float* src = &sv[i * PV + s * C + c0];
            if constexpr (VPL == 2) {
              const float2 v = *reinterpret_cast<const float2*>(src);
              x[0][s] = v.x;
              x[1][s] = v.y;
            } else {
              x[0][s] = src[0];
            }
          }
  #pragma unroll
          for (int v = 0; v < VPL; ++v) eaas_channel<LMAX>(x[v], y[v], e.f, e.d, e.R);
  #pragma unroll
          for (int s = 0; s < S; ++s) {
            float o[VPL];
  #pragma unroll
            for (int v = 0; v < VPL; ++v) o[v] = y[v][s];
            VecIO<T, VPL>::store(dst + s * C, o);
          }
        }
      } else {
        for (int p = tid; p < TA * C; p += NT) {
          const int i = p / C;
          const int c = p - i * C;
          if (i >= na) break;
          const int64_t atom = a0 + i;
          const AtomFrame<LMAX> e = tf[i];
          float x[S], y[S];
  #pragma unroll
          for (int s = 0; s < S; ++s) x[s] = sv[i * PV + s * C + c];
          eaas_channel<LMAX>(x, y, e.f, e.d, e.R);
          T* dst = ws + atom * (int64_t)((S + 1) * C) + C + c;
  #pragma unroll
          for (int s = 0; s < S; ++s) store_elem(dst + s * C, y[s]);
        }
      }
    }
    // the next tile's step 1 overwrites sa, last read in step 2 above (before
    // the barrier that preceded step 4), so no further barrier is needed here
  }
}

// ---------------------------------------------------------- any C: vector ALU
//
// The same products and coupling for channel counts the matrix-core kernel is
// not built for (C not in its list, or too wide for its register-held weight
// slices).  One workgroup per atom: the atom's S rows are staged in LDS; thread
// c computes output channel c of q, k and every value row, summing over the
// input channels in order (fp32 accumulation), then applies EAAS to channel c.
template <int LMAX, typename T>
__global__ __launch_bounds__(256) void k_proj_generic(ProjArgs a, EaasCoef cf, int C) {
  constexpr int S = ncomp(LMAX);
  extern __shared__ float s_h[];   // [S, C] of this atom, widened to fp32
  const int64_t atom = blockIdx.x;
  if (atom >= a.n) return;
  const T* h = static_cast<const T*>(a.h) + atom * (int64_t)S * C;
  for (int e = threadIdx.x; e < S * C; e += blockDim.x) {
    float v;
    VecIO<T, 1>::load(h + e, &v);
    s_h[e] = v;
  }
  __syncthreads();
  const T* wq = static_cast<const T*>(a.w_q);
  const T* wk = static_cast<const T*>(a.w_k);
  const T* wv = static_cast<const T*>(a.w_v);
  const Frame f = make_frame(a.r[3 * atom], a.r[3 * atom + 1], a.r[3 * atom + 2]);
  const Dy2 d = make_dy2(f);
  const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
  T* ws = static_cast<T*>(a.ws) + atom * (int64_t)(S + 1) * C;
  T* qo = static_cast<T*>(a.q_out) + atom * (int64_t)C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float q = 0.0f, k = 0.0f, v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = 0.0f;
    for (int i = 0; i < C; ++i) {
      float w_q, w_k;
      VecIO<T, 1>::load(wq + (int64_t)i * C + c, &w_q);
      VecIO<T, 1>::load(wk + (int64_t)i * C + c, &w_k);
      q = fmaf(s_h[i], w_q, q);
      k = fmaf(s_h[i], w_k, k);
#pragma unroll
      for (int l = 0; l <= LMAX; ++l) {
        float w_v;
        VecIO<T, 1>::load(wv + ((int64_t)l * C + i) * C + c, &w_v);
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m) v[l * l + m] = fmaf(s_h[(l * l + m) * C + i], w_v, v[l * l + m]);
      }
    }
    VecIO<T, 1>::store(qo + c, &q);
    VecIO<T, 1>::store(ws + c, &k);
    float y[S];
    eaas_channel<LMAX>(v, y, f, d, R);
#pragma unroll
    for (int s = 0; s < S; ++s) VecIO<T, 1>::store(ws + (s + 1) * C + c, &y[s]);
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

template <int LMAX, typename T>
int go_generic(int C, const ProjArgs& a, const EaasCoef& cf, hipStream_t s) {
  const int threads = C < 256 ? (C + 63) / 64 * 64 : 256;
  const size_t lds = (size_t)ncomp(LMAX) * C * sizeof(float);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_proj_generic<LMAX, T>), dim3((unsigned)a.n), dim3(threads), lds, s, a, cf,
                     C);
  return (int)hipGetLastError();
}

// the matrix-core kernel's channel counts
bool proj_mfma(int C, int dtype) {
  if (dtype == 0) return C == 16 || C == 32 || C == 64 || C == 128;
  return C == 32 || C == 64 || C == 128;
}

template <typename T>
int go_l(int lmax, int C, const ProjArgs& a, const EaasCoef& cf, hipStream_t s) {
  const bool mfma = proj_mfma(C, sizeof(T) == 4 ? 0 : 1);
  switch (lmax) {
    case 0: return mfma ? go_c<0, T>(C, a, cf, s) : go_generic<0, T>(C, a, cf, s);
    case 1: return mfma ? go_c<1, T>(C, a, cf, s) : go_generic<1, T>(C, a, cf, s);
    default: return mfma ? go_c<2, T>(C, a, cf, s) : go_generic<2, T>(C, a, cf, s);
  }
}

}  // namespace

bool proj_supported(int C, int dtype) {
  (void)dtype;
  return C >= 1 && C <= kProjMaxC;
}

int launch_proj(int lmax, int dtype, int C, const ProjArgs& a, const EaasCoef& cf,
                hipStream_t s) {
  if (a.n == 0) return 0;
  return dtype == 0 ? go_l<float>(lmax, C, a, cf, s) : go_l<uint16_t>(lmax, C, a, cf, s);
}

}  // namespace e2f
