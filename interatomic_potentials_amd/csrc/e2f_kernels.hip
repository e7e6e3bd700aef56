// e2f_kernels.hip -- gfx950 kernels of libe2f.
//
// k_eaas       EAAS tensor product per atom (write-up section 2): one group of
//              2^lane_log lanes per atom, each lane owning V adjacent channels
//              of every irrep row; rows are read and written as one coalesced
//              vector access per lane.  In workspace mode it also copies the
//              l = 0 row (the key) in front of h', so that a neighbour's K and
//              V form one contiguous block for the stream below, and into the
//              query rows.
// k_aggregate  steps 2 and 3 (write-up section 3; gist.science summary 2.2):
//              one wavefront per target, targets taken in a spatial schedule.
//              The valid slots of the target's row are compacted into LDS
//              with a ballot and sorted by atom index; the wave then splits
//              into 64 / 2^lane_log subgroups that stream disjoint neighbours
//              (each neighbour's (S + 1) rows read once, coalesced), keep a
//              running max and normaliser per head (online softmax, base-2
//              with log2(e) folded into the scale) and fp32 accumulators in
//              registers, merge the subgroups with cross-lane exchanges, and
//              apply the target-side EAAS before the only store.
// k_frames     test hook: alignment rotation and Wigner-D blocks as built here.
// k_validate   flags a valid slot whose index lies outside [0, N).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the `hl` adjacent lanes of one head (hl a power of two, heads
// aligned to hl).  HL > 0 fixes the width at compile time; HL = 0 takes it
// from `hl` with uniform branches.  DPP within a 16-lane row.
__device__ inline float head_sum(float x, int hl);

// The values of x on the two lanes of the pair (lane, lane ^ o), the lower
// lane's first, on both lanes: o = 16 and 32 by a cross-row swap (VALU, no
// LDS), other o by a shuffle.
template <int O>
__device__ inline void pair_lohi(float x, int o, int lane, float& lo, float& hi) {
  if constexpr (O == 32) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    lo = __uint_as_float(sw[0]);   // lanes 0-31's value, on every lane
    hi = __uint_as_float(sw[1]);   // lanes 32-63's value
  } else if constexpr (O == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    lo = __uint_as_float(sw[0]);   // the even 16-lane row's value
    hi = __uint_as_float(sw[1]);   // the odd row's value
  } else {
    const float p = __shfl_xor(x, o);
    const bool upper = (lane & o) != 0;
    lo = upper ? p : x;
    hi = upper ? x : p;
  }
}

// One step of merging the online-softmax states (mu, z, acc) of the lane pairs
// (lane, lane ^ o): both lanes evaluate lo c_lo + hi c_hi from the same
// operands, so both end with the same bits.
template <int O, int S, int V>
__device__ inline void merge_state(float& mu, float& z, float (&acc)[S][V], int o, int lane) {
  float mlo, mhi, zlo, zhi;
  pair_lohi<O>(mu, o, lane, mlo, mhi);
  pair_lohi<O>(z, o, lane, zlo, zhi);
  const float mx = fmaxf(mlo, mhi);
  const float clo = exp2_fast(mlo - mx);
  const float chi = exp2_fast(mhi - mx);
  z = zlo * clo + zhi * chi;
#pragma unroll
  for (int r = 0; r < S; ++r)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float alo, ahi;
      pair_lohi<O>(acc[r][v], o, lane, alo, ahi);
      acc[r][v] = alo * clo + ahi * chi;
    }
  mu = mx;
}

// One halving step of a reduce-scatter of online-softmax states across the lane
// pairs (lane, lane ^ O), O = 16 or 32: of the 2W channels in `in`, the lower
// lane of each pair keeps channels [0, W) and the upper lane [W, 2W), merged,
// in `out`.  One swap hands each lane both copies of the channel it keeps, the
// lower lane's first, so both lanes merge from the same operands.
template <int O, int S, int W>
__device__ inline void merge_halve(float& mu, float& z, const float (&in)[S][2 * W],
                                   float (&out)[S][W], int lane) {
  float mlo, mhi, zlo, zhi;
  pair_lohi<O>(mu, O, lane, mlo, mhi);
  pair_lohi<O>(z, O, lane, zlo, zhi);
  const float mx = fmaxf(mlo, mhi);
  const float clo = exp2_fast(mlo - mx);
  const float chi = exp2_fast(mhi - mx);
  z = zlo * clo + zhi * chi;
  mu = mx;
#pragma unroll
  for (int r = 0; r < S; ++r)
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const uint32_t a = __float_as_uint(in[r][k]), b = __float_as_uint(in[r][k + W]);
      float lo, hi;
      if constexpr (O == 32) {
        const auto sw = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        lo = __uint_as_float(sw[0]);
        hi = __uint_as_float(sw[1]);
      } else {
        static_assert(O == 16, "cross-row swaps");
        const auto sw = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        lo = __uint_as_float(sw[0]);
        hi = __uint_as_float(sw[1]);
      }
      out[r][k] = lo * clo + hi * chi;
    }
}

template <int S, int V>
__device__ inline void merge_step(float& mu, float& z, float (&acc)[S][V], int o, int lane) {
  if (o == 32) merge_state<32>(mu, z, acc, o, lane);
  else if (o == 16) merge_state<16>(mu, z, acc, o, lane);
  else merge_state<0>(mu, z, acc, o, lane);
}

template <int HL>
__device__ inline float head_sum_t(float x, int hl) {
  if constexpr (HL == 0) {
    return head_sum(x, hl);
  } else {
    if constexpr (HL >= 2) x += dpp<0xB1>(x);
    if constexpr (HL >= 4) x += dpp<0x4E>(x);
    if constexpr (HL >= 8) x += dpp<0x141>(x);
    if constexpr (HL >= 16) x += dpp<0x140>(x);
    static_assert(HL <= 16, "wider heads take the runtime path");
    return x;
  }
}

__device__ inline float head_sum(float x, int hl) {
  if (hl >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  if (hl >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  if (hl >= 8) x += dpp<0x141>(x);   // row_half_mirror: quad 0 <-> quad 1
  if (hl >= 16) x += dpp<0x140>(x);  // row_mirror: half-row 0 <-> 1
  if (hl >= 32) x += __shfl_xor(x, 16);
  if (hl >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ K1

template <int LMAX, int V, typename T, bool WS>
__global__ __launch_bounds__(256) void k_eaas(EaasArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lg = a.lane_log;
  const int sub = lane >> lg;
  const int gl = lane & ((1 << lg) - 1);
  const int64_t atom = ((int64_t)blockIdx.x * kWavesPerBlock + w) * (64 >> lg) + sub;
  if (atom >= a.n) return;
  const int C = a.C;
  const Frame f = make_frame(a.r[3 * atom], a.r[3 * atom + 1], a.r[3 * atom + 2]);
  const Dy2 d = make_dy2(f);
  const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
  const T* src = static_cast<const T*>(a.h_in) + atom * (int64_t)S * C;
  T* dst = static_cast<T*>(a.h_out) + atom * (int64_t)(WS ? S + 1 : S) * C;
  for (int c0 = gl * V; c0 < C; c0 += V << lg) {
    float x[S][V];
#pragma unroll
    for (int s = 0; s < S; ++s) VecIO<T, V>::load(src + s * C + c0, x[s]);
    if constexpr (WS) {
      VecIO<T, V>::store(dst + c0, x[0]);
      VecIO<T, V>::store(static_cast<T*>(a.q_out) + atom * C + c0, x[0]);
    }
    float y[S][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float xv[S], yv[S];
#pragma unroll
      for (int s = 0; s < S; ++s) xv[s] = x[s][v];
      eaas_channel<LMAX>(xv, yv, f, d, R);
#pragma unroll
      for (int s = 0; s < S; ++s) y[s][v] = yv[s];
    }
#pragma unroll
    for (int s = 0; s < S; ++s) VecIO<T, V>::store(dst + (WS ? s + 1 : s) * C + c0, y[s]);
  }
}

// ------------------------------------------------------------------ K2

constexpr float kSlack = 8.0f;   // lazy-rescale slack of the running max (base 2)

// Four waves a workgroup (one measured the same at Scale-out: short, even work).
constexpr int kAggWaves = 4;   // waves per workgroup

// SPLIT: V == 2 P (two channels of each lane per subgroup in the epilogue),
// chosen by the launcher from the lane layout.
template <int LMAX, int V, typename T, int U, int HL, bool BUF, bool ENV, bool SPLIT = false>
__global__ __launch_bounds__(64 * kAggWaves) void k_aggregate(AggArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  __shared__ int s_nb[kAggWaves][kTile];
  __shared__ float s_le[kAggWaves][ENV ? kTile : 1];  // log2 envelope of each sorted slot
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Workgroups are dealt to the XCDs round-robin; give XCD x the x-th
  // contiguous stretch of the schedule so that the waves sharing an L2 work
  // on neighbouring targets (the grid is a multiple of kXcds).
  const int64_t per_xcd = (int64_t)gridDim.x / kXcds;
  const int64_t blk = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int64_t slot = blk * kAggWaves + w;
  if (slot >= a.N) return;  // whole wave: no workgroup barrier below
  const int64_t i = a.sched ? (int64_t)a.sched[slot] : slot;
  if (i < 0 || i >= a.N) return;
  const int lg = a.lane_log;
  const int P = 64 >> lg;
  const int sub = lane >> lg;
  const int c0 = (lane & ((1 << lg) - 1)) * V;
  const bool act = c0 < a.C;
  const int c0_load = act ? c0 : 0;  // idle lanes read a valid column and never store
  const int C = a.C;
  const int K = a.K;
  const int64_t N = a.N;
  const int64_t row = (int64_t)(S + 1) * C;  // elements per atom in the workspace
  const T* ws = static_cast<const T*>(a.ws);
  // buffer path: the host only selects it when N * row bytes fits 32 bits
  const uint32_t row_bytes = (uint32_t)(row * (int64_t)sizeof(T));
  const uint32_t cbytes = (uint32_t)C * (uint32_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t rsrc =
      make_rsrc(a.ws, BUF ? (uint32_t)(N * row * (int64_t)sizeof(T)) : 0u);

  float q[V];
  if (act) {
    VecIO<T, V>::load(static_cast<const T*>(a.q) + i * C + c0, q);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) q[v] = 0.0f;
  }
  float mu = -1e30f;  // running max (base-2 units); finite so that empty merges stay finite
  float z = 0.0f;     // running normaliser
  float acc[S][V];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[s][v] = 0.0f;

  const int32_t* irow = a.idx + i * K;
  const uint8_t* mrow = a.mask + i * K;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  int* nb = s_nb[w];
  for (int t0 = 0; t0 < K; t0 += kTile) {
    // compact this tile's valid slots (mask = 1 and index in range) into LDS
    // (every chunk's index and mask loads issued before the first ballot)
    constexpr int NC = kTile / 64;
    int jv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int slot = t0 + c * 64 + lane;
      int j = -1;
      if (slot < K) {
        const uint8_t m = mrow[slot];
        const int jj = irow[slot];
        j = (m != 0 && jj >= 0 && (int64_t)jj < N) ? jj : -1;
      }
      jv[c] = j;
    }
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (t0 + c * 64 >= K) break;   // uniform
      const bool ok = jv[c] >= 0;
      const uint64_t b = __ballot(ok);
      if (ok) nb[cnt + __popcll(b & below)] = jv[c];
      cnt += __popcll(b);
    }
    // Sort the tile's neighbours by atom index (bitonic, in registers).  All
    // waves then sweep shared neighbours in the same order, so rows fetched
    // by one target are still in L2 when nearby targets ask for them; and the
    // visiting order, hence the rounding, no longer depends on slot order.
    wave_sort<kTile>(reinterpret_cast<uint32_t*>(nb), cnt, lane, 0x7fffffffu);
    if constexpr (ENV) {
      // log2 of the distance envelope per sorted slot; it joins the base-2 logit,
      // so the slot's weight is e_ij exp(s_ij) in numerator and normaliser alike
      // (-inf at or beyond the cutoff: weight 0)
      const float xi = a.pos[3 * i], yi = a.pos[3 * i + 1], zi = a.pos[3 * i + 2];
      for (int e = lane; e < cnt; e += 64) {
        const int j = nb[e];
        s_le[w][e] = envelope_term(xi, yi, zi, a.pos[3 * j], a.pos[3 * j + 1], a.pos[3 * j + 2],
                                   a.env_rc).log2u;
      }
      wave_sync();
    }

    for (int n0 = 0; n0 < cnt; n0 += P * U) {
      // Past the end of the list a subgroup re-reads the tile's last valid
      // neighbour (finite, already part of this target's sum) with weight 0,
      // so every load is unconditional and nothing needs clearing.
      Raw<T, V> kv[U][S + 1];
      bool val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * P + sub;
        val[u] = n < cnt;
        const int jn = nb[val[u] ? n : cnt - 1];
        if constexpr (BUF) {
          const uint32_t voff = (uint32_t)jn * row_bytes + (uint32_t)c0_load * (uint32_t)sizeof(T);
#pragma unroll
          for (int r = 0; r <= S; ++r) buffer_load_raw<T, V>(rsrc, voff, (uint32_t)r * cbytes, kv[u][r]);
        } else {
          const T* src = ws + (int64_t)jn * row + c0_load;
#pragma unroll
          for (int r = 0; r <= S; ++r) VecIO<T, V>::load_raw(src + r * C, kv[u][r]);
        }
      }
      float s[U];
      float mx = mu;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dt = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) dt = fmaf(q[v], kv[u][0].get(v), dt);
        dt = head_sum_t<HL>(dt, a.head_lanes);
        float le = 0.0f;
        if constexpr (ENV) le = s_le[w][val[u] ? n0 + u * P + sub : 0];
        s[u] = val[u] ? dt * a.scale_log2e + le : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      // Lazy rescale: mu only has to bound the logits seen so far to within
      // kSlack (base 2), so weights stay below 2^kSlack until the final
      // normalisation; the state is rescaled only when a logit exceeds it by more
      if (__any(mx > mu + kSlack)) {
        const float corr = exp2_fast(mu - mx);
        z *= corr;
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
          for (int v = 0; v < V; ++v) acc[r][v] *= corr;
        mu = mx;
      }
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = exp2_fast(s[u] - mu);
        z += p[u];
      }
#pragma unroll
      for (int r = 0; r < S; ++r)
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float t = acc[r][v];
#pragma unroll
          for (int u = 0; u < U; ++u) t = fmaf(p[u], kv[u][r + 1].get(v), t);
          acc[r][v] = t;
        }
    }
    wave_sync();  // every read of s_nb is done before the next tile rewrites it
  }

  if constexpr (SPLIT) {
    // reduce-scatter of the subgroups' partial softmax states (same channels,
    // other neighbours), largest lane distance first, so that subgroup g ends
    // with channels 2g and 2g + 1 of each lane's V, merged; it finishes them.
    static_assert(V == 4 || V == 8, "two or four subgroups");
    float m2[S][2];
    if constexpr (V == 8) {
      float h[S][4];
      merge_halve<32>(mu, z, acc, h, lane);
      merge_halve<16>(mu, z, h, m2, lane);
    } else {
      merge_halve<32>(mu, z, acc, m2, lane);
    }
    if (!act) return;
    if (sub == 0 && a.lse != nullptr && (lane & (a.head_lanes - 1)) == 0) {
      const int d = a.C / a.heads;
      a.lse[i * a.heads + c0 / d] =
          z > 0.0f ? (mu + log2f(z)) * 0.6931471805599453f : -INFINITY;
    }
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int k = 0; k < 2; ++k) m2[r][k] *= inv;
    const int cs = c0 + 2 * sub;
    if (a.out_msg != nullptr) {
      if (a.msg_f32) {   // the message in fp32 whatever the storage type
        float* mp = static_cast<float*>(a.out_msg) + i * (int64_t)S * C + cs;
#pragma unroll
        for (int r = 0; r < S; ++r) VecIO<float, 2>::store(mp + r * C, m2[r]);
      } else {
        T* mp = static_cast<T*>(a.out_msg) + i * (int64_t)S * C + cs;
#pragma unroll
        for (int r = 0; r < S; ++r) VecIO<T, 2>::store(mp + r * C, m2[r]);
      }
    }
    const Frame f = make_frame(a.pos[3 * i], a.pos[3 * i + 1], a.pos[3 * i + 2]);
    const Dy2 d = make_dy2(f);
    const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
    T* op = static_cast<T*>(a.out) + i * (int64_t)S * C + cs;
    float y[S][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float xv[S], yv[S];
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) xv[s2] = m2[s2][k];
      eaas_channel<LMAX>(xv, yv, f, d, R);
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) y[s2][k] = yv[s2];
    }
#pragma unroll
    for (int r = 0; r < S; ++r) VecIO<T, 2>::store(op + r * C, y[r]);
    return;
  }
  // merge the subgroups' partial softmax states; every subgroup ends with the
  // same bits, and subgroup 0 finishes
  for (int o = 1 << lg; o < 64; o <<= 1) merge_step(mu, z, acc, o, lane);
  if (sub != 0 || !act) return;
  if (a.lse != nullptr && (lane & (a.head_lanes - 1)) == 0) {
    // natural log-sum-exp of this head's logits (base-2 running state times ln 2)
    const int d = a.C / a.heads;
    a.lse[i * a.heads + c0 / d] =
        z > 0.0f ? (mu + log2f(z)) * 0.6931471805599453f : -INFINITY;
  }
  const float inv = z > 0.0f ? 1.0f / z : 0.0f;  // no valid slot: m_i = 0, out_i = 0
#pragma unroll
  for (int r = 0; r < S; ++r)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[r][v] *= inv;
  if (a.out_msg != nullptr) {
    if (a.msg_f32) {   // the message in fp32 whatever the storage type
      float* mp = static_cast<float*>(a.out_msg) + i * (int64_t)S * C + c0;
#pragma unroll
      for (int r = 0; r < S; ++r) VecIO<float, V>::store(mp + r * C, acc[r]);
    } else {
      T* mp = static_cast<T*>(a.out_msg) + i * (int64_t)S * C + c0;
#pragma unroll
      for (int r = 0; r < S; ++r) VecIO<T, V>::store(mp + r * C, acc[r]);
    }
  }
  const Frame f = make_frame(a.pos[3 * i], a.pos[3 * i + 1], a.pos[3 * i + 2]);
  const Dy2 d = make_dy2(f);
  const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
  T* op = static_cast<T*>(a.out) + i * (int64_t)S * C + c0;
  float y[S][V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float xv[S], yv[S];
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) xv[s2] = acc[s2][v];
    eaas_channel<LMAX>(xv, yv, f, d, R);
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) y[s2][v] = yv[s2];
  }
#pragma unroll
  for (int r = 0; r < S; ++r) VecIO<T, V>::store(op + r * C, y[r]);
}

// ------------------------------------------------ K2, targets sharing rows
//
// The same three steps for T spatially adjacent targets per wavefront (fp32
// storage, 4 channels per lane).  Their valid slots are merged into one
// union of distinct sources; each union source's S + 1 rows are read once and
// applied to every target that lists it (a source in c of a target's slots
// weighs c exp(s), so repeated slots still count once each).  With the distance
// envelope, each (target, source) pair's log2 u is tabulated in LDS while the
// slots are counted and joins that pair's logit.  Adjacent targets share most
// of their neighbours, so the rows read per target drop by the union's sharing
// factor.
//
// Subgroup g streams the union sources j with j mod P == g in increasing j,
// and a target's state is touched only by sources it lists (a subgroup-uniform
// branch), so every target's arithmetic -- which subgroup adds which source,
// in which order -- depends on its own neighbour set alone: not on the other
// targets sharing the wave, the schedule, or slot order.
constexpr int kMtMaxK = kShareMaxK;   // longest neighbour row this kernel takes
// Four targets per wave, one union source per subgroup in flight: on the
// Hilbert-curve schedule the union of four adjacent targets' rows is a small
// enough share of their lengths that it beats three targets with two in flight
// (0.835 against 0.850 ms at Large) and two targets with one or two (0.93).
// The envelope variant keeps three targets with two in flight: its log2 u table
// grows with the targets, and at four it would hold a CU to four workgroups.
constexpr int kMtTargets = 4;       // targets per wave
constexpr int kMtInflight = 1;      // union sources per subgroup in flight
constexpr int kMtTargetsEnv = 3;    // the same with the distance envelope
constexpr int kMtInflightEnv = 2;

// One wave a workgroup: the waves share nothing, and a workgroup's LDS and slot
// are freed only when its last wave ends, so with four waves the early ones
// idled (one: 0.93 ms at Large against 0.98 with four).
constexpr int kMtWaves = 1;   // waves per workgroup

// The last sixteenth of each XCD's stretch in closing units of two targets (see
// unit_map): at 32,768 atoms the stretch is about four units per wave slot; an
// eighth, a quarter, a twenty-fourth and a thirty-second in units of two, a
// sixteenth in units of one and an eighth in units of three measured slower.
constexpr int kMtTailDen = 16;
constexpr int kMtTailT = 2;

template <int LMAX, int T, int U, int HL, bool ENV>
__global__ __launch_bounds__(64 * kMtWaves) void k_aggregate_mt(AggArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  constexpr int V = 4;
  constexpr int EN = ShareLds<T>::EN;
  constexpr int CW = ShareLds<T>::CW;
  __shared__ ShareLds<T> s_un[kMtWaves];
  // log2 of the distance envelope per (target, union source), with the envelope
  __shared__ float s_le[kMtWaves][ENV ? T : 1][ENV ? EN : 1];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Workgroups are dealt to the XCDs round-robin: XCD x runs units x, x + kXcds, ...
  // of the grid, in order, over its own stretch of the schedule, closing units last
  static_assert(kMtWaves == 1, "one wave a workgroup");
  (void)w;
  int64_t slot0, xend;
  int cnt;   // targets of this unit
  unit_of_block(unit_map(a.N, T, kMtTailDen, kMtTailT), blockIdx.x, T, kMtTailT, slot0, cnt,
                xend);
  if (slot0 >= a.N) return;  // whole wave: no workgroup barrier below
  const int64_t N = a.N;
  const int C = a.C;
  int64_t tg[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t sl = slot0 + t;
    int64_t i = -1;
    if (t < cnt && sl < N && sl < xend) i = a.sched ? (int64_t)a.sched[sl] : sl;
    tg[t] = (i >= 0 && i < N) ? i : -1;
  }
  const int lg = a.lane_log;
  const int lgp = 6 - lg;                    // log2 of the subgroups per wave
  const int sub = lane >> lg;
  const int c0 = (lane & ((1 << lg) - 1)) * V;
  const bool act = c0 < C;
  const int c0_load = act ? c0 : 0;
  const int64_t row = (int64_t)(S + 1) * C;
  const uint32_t row_bytes = (uint32_t)(row * 4);
  const uint32_t cbytes = (uint32_t)C * 4u;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.ws, (uint32_t)(N * row * 4));
  ShareLds<T>& un = s_un[w];
  const int32_t* uj = un.uj;

  // 1-3. the union of the targets' sources, bucket by bucket, with slot counts
  (void)share_union_rows<T>(un, a.idx, a.mask, N, a.K, tg, lgp, lane,
                       [&](int t, int u, int32_t j) {
                         if constexpr (ENV) {
                           // the pair's envelope (a repeated slot writes the same value again)
                           int64_t ti = tg[0];
#pragma unroll
                           for (int tt = 1; tt < T; ++tt)
                             if (t == tt) ti = tg[tt];
                           s_le[w][t][u] =
                               envelope_term(a.pos[3 * ti], a.pos[3 * ti + 1], a.pos[3 * ti + 2],
                                             a.pos[3 * j], a.pos[3 * j + 1], a.pos[3 * j + 2],
                                             a.env_rc).log2u;
                         }
                       });
  const int my_cnt = un.bcnt[sub];
  const int my_start = un.bstart[sub];
  int maxlen = my_cnt;
  for (int o = 1; o < 64; o <<= 1) maxlen = max(maxlen, __shfl_xor(maxlen, o));

  // 4. stream the union once for all targets
  float q[T][V];
  float mu[T], z[T];
  float acc[T][S][V];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (act && tg[t] >= 0) {
      VecIO<float, V>::load(static_cast<const float*>(a.q) + tg[t] * C + c0, q[t]);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) q[t][v] = 0.0f;
    }
    mu[t] = -1e30f;
    z[t] = 0.0f;
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[t][r][v] = 0.0f;
  }
  // union entry of the subgroup's k-th source; past the end of its bucket a
  // subgroup re-reads some valid source and adds nothing
  auto entry = [&](int k) {
    return k < my_cnt ? my_start + k : (my_cnt > 0 ? my_start + my_cnt - 1 : 0);
  };
  int jcur[U];   // the sources of the coming iteration, read one iteration ahead
#pragma unroll
  for (int u = 0; u < U; ++u) jcur[u] = uj[entry(u)];
#pragma unroll 1
  for (int it = 0; it < maxlen; it += U) {
    Raw<float, V> kv[U][S + 1];
    uint32_t cw[U][CW];
    float le[U][ENV ? T : 1];   // log2 of the envelope per (source, target), read with the rows
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool val = it + u < my_cnt;
      const int nn = entry(it + u);
      const uint32_t voff = (uint32_t)jcur[u] * row_bytes + (uint32_t)c0_load * 4u;
#pragma unroll
      for (int r = 0; r <= S; ++r)
        buffer_load_raw<float, V>(rsrc, voff, (uint32_t)r * cbytes, kv[u][r]);
#pragma unroll
      for (int c = 0; c < CW; ++c) cw[u][c] = val ? un.cnt[c][nn] : 0u;
      if constexpr (ENV) {
#pragma unroll
        for (int t = 0; t < T; ++t) le[u][t] = s_le[w][t][nn];
      }
    }
    // the next iteration's sources, while these rows are in flight
#pragma unroll
    for (int u = 0; u < U; ++u) jcur[u] = uj[entry(it + U + u)];
    // keep every source's loads in flight before the first use
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t m = share_count<CW>(cw[u], t);
        if (m != 0u) {   // uniform within the subgroup: targets that do not list j are untouched
          float dt = 0.0f;
#pragma unroll
          for (int v = 0; v < V; ++v) dt = fmaf(q[t][v], kv[u][0].get(v), dt);
          dt = head_sum_t<HL>(dt, a.head_lanes);
          float sc = dt * a.scale_log2e;
          // log2 of the envelope joins the base-2 logit (-inf beyond the cutoff: weight 0)
          if constexpr (ENV) sc += le[u][t];
          // lazy rescale, as in the single-target kernel, but decided per lane
          // (per head and subgroup): whether the other subgroup happens to be
          // updating this target must not move this subgroup's reference point
          const bool need = sc > mu[t] + kSlack;
          if (__any(need)) {
            const float mx = need ? sc : mu[t];
            const float corr = exp2_fast(mu[t] - mx);   // exactly 1 where not needed
            z[t] *= corr;
#pragma unroll
            for (int r = 0; r < S; ++r)
#pragma unroll
              for (int v = 0; v < V; ++v) acc[t][r][v] *= corr;
            mu[t] = mx;
          }
          // c slots of the same source weigh c times
          const float p = exp2_fast(sc - mu[t]) * (float)m;
          z[t] += p;
#pragma unroll
          for (int r = 0; r < S; ++r)
#pragma unroll
            for (int v = 0; v < V; ++v)
              acc[t][r][v] = fmaf(p, kv[u][r + 1].get(v), acc[t][r][v]);
        }
      }
    }
  }

  // 6. per target: normalise, target-side EAAS, store (the lanes of one subgroup)
  auto finish = [&](int64_t i, float (&m)[S][V], float zt, float mut) {
    if (a.lse != nullptr && (lane & (a.head_lanes - 1)) == 0) {
      const int d = C / a.heads;
      a.lse[i * a.heads + c0 / d] =
          zt > 0.0f ? (mut + log2f(zt)) * 0.6931471805599453f : -INFINITY;
    }
    const float inv = zt > 0.0f ? 1.0f / zt : 0.0f;
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) m[r][v] *= inv;
    if (a.out_msg != nullptr) {
      float* mp = static_cast<float*>(a.out_msg) + i * (int64_t)S * C + c0;
#pragma unroll
      for (int r = 0; r < S; ++r) VecIO<float, V>::store(mp + r * C, m[r]);
    }
    const Frame f = make_frame(a.pos[3 * i], a.pos[3 * i + 1], a.pos[3 * i + 2]);
    const Dy2 d = make_dy2(f);
    const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
    float* op = static_cast<float*>(a.out) + i * (int64_t)S * C + c0;
    float y[S][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float xv[S], yv[S];
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) xv[s2] = m[s2][v];
      eaas_channel<LMAX>(xv, yv, f, d, R);
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) y[s2][v] = yv[s2];
    }
#pragma unroll
    for (int r = 0; r < S; ++r) VecIO<float, V>::store(op + r * C, y[r]);
  };

  // 5. merge the subgroups' partial states per target
  if (T == 2 && lg == 5) {
    // two subgroups, two targets: a reduce-scatter.  One swap of target 0's and
    // target 1's value hands the lower half both copies of target 0's, and the
    // upper half both copies of target 1's, the lower lane's first; subgroup t
    // finishes target t.
    float clo[T], chi[T], zm[T], mm[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float mlo, mhi, zlo, zhi;
      pair_lohi<32>(mu[t], 32, lane, mlo, mhi);
      pair_lohi<32>(z[t], 32, lane, zlo, zhi);
      mm[t] = fmaxf(mlo, mhi);
      clo[t] = exp2_fast(mlo - mm[t]);
      chi[t] = exp2_fast(mhi - mm[t]);
      zm[t] = zlo * clo[t] + zhi * chi[t];
    }
    const bool up = sub != 0;
    const float cl = up ? clo[T - 1] : clo[0], ch = up ? chi[T - 1] : chi[0];
    float m[S][V];
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0][r][v]),
                                                         __float_as_uint(acc[T - 1][r][v]),
                                                         false, false);
        m[r][v] = __uint_as_float(sw[0]) * cl + __uint_as_float(sw[1]) * ch;
      }
    const int64_t i = up ? tg[T - 1] : tg[0];
    if (!act || i < 0) return;
    finish(i, m, up ? zm[T - 1] : zm[0], up ? mm[T - 1] : mm[0]);
    return;
  }
  // otherwise an all-reduce: every subgroup ends with the same bits; subgroup t
  // finishes target t (with fewer subgroups than targets, subgroup 0 finishes
  // them one by one)
  for (int o = 1 << lg; o < 64; o <<= 1) {
#pragma unroll
    for (int t = 0; t < T; ++t) merge_step(mu[t], z[t], acc[t], o, lane);
  }
  if (!act) return;
  const bool split = (64 >> lg) >= T;
  if (split && sub >= T) return;
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    if (split && tt > 0) break;
    // this lane's target: tt, or its subgroup's one
    int64_t i = tg[tt];
    float zt = z[tt], mut = mu[tt];
    float m[S][V];
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) m[r][v] = acc[tt][r][v];
    if (split) {
#pragma unroll
      for (int t = 1; t < T; ++t) {
        if (sub == t) {
          i = tg[t];
          zt = z[t];
          mut = mu[t];
#pragma unroll
          for (int r = 0; r < S; ++r)
#pragma unroll
            for (int v = 0; v < V; ++v) m[r][v] = acc[t][r][v];
        }
      }
    } else if (sub != 0) {
      return;
    }
    if (i < 0) continue;   // uniform within the subgroup
    finish(i, m, zt, mut);
  }
}

// ------------------------------------------------------------ helpers

__global__ __launch_bounds__(256) void k_frames(int lmax, int64_t n, const float* r, float* Q,
                                                float* D) {
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a >= n) return;
  const Frame f = make_frame(r[3 * a], r[3 * a + 1], r[3 * a + 2]);
  const Dy2 d = make_dy2(f);
  float* q = Q + 9 * a;
  // Q = R_y(-t) R_z(-p)
  q[0] = f.ct * f.c1; q[1] = f.ct * f.s1; q[2] = -f.st;
  q[3] = -f.s1;       q[4] = f.c1;        q[5] = 0.0f;
  q[6] = f.st * f.c1; q[7] = f.st * f.s1; q[8] = f.ct;
  float* dd = D + 35 * a;
  dd[0] = 1.0f;
  // column k of D(Q) = rotate_in applied to the k-th unit vector
  for (int col = 1; col < 9; ++col) {
    const int l = col < 4 ? 1 : 2;
    if (l > lmax) break;
    float e[9];
    for (int s = 0; s < 9; ++s) e[s] = s == col ? 1.0f : 0.0f;
    rotate_in<2>(e, f, d);
    const int base = l == 1 ? 1 : 10;
    const int off = l * l;  // first flat index of the block
    const int dim = 2 * l + 1;
    for (int row = 0; row < dim; ++row) dd[base + row * dim + (col - off)] = e[off + row];
  }
}

__global__ __launch_bounds__(256) void k_clear_flag(int32_t* flag) { *flag = 0; }

__global__ __launch_bounds__(256) void k_validate(int64_t total, int64_t N, const int32_t* idx,
                                                  const uint8_t* mask, int32_t* flag) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  if (mask[t] != 0) {
    const int32_t j = idx[t];
    if (j < 0 || (int64_t)j >= N) *flag = 1;  // every writer stores the same value
  }
}

// ------------------------------------------------- target schedule
//
// Targets are visited in Hilbert-curve order of a grid of 2^bits cells per
// axis over the bounding box of the positions, built with a counting
// sort: bounding box, per-cell counts, one scan, scatter.  The order inside
// a cell is whatever the atomics produce; it only changes which wave takes
// which target, never a target's arithmetic, so outputs do not depend on it.

// spread the low 10 bits of v to every third bit (three-way bit interleave)
__device__ inline uint32_t spread3(uint32_t v) {
  v &= 0x3ffu;
  v = (v | (v << 16)) & 0x030000ffu;
  v = (v | (v << 8)) & 0x0300f00fu;
  v = (v | (v << 4)) & 0x030c30c3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}

// Position along the Hilbert curve of the cell (x, y, z), each coordinate of
// `bits` bits: J. Skilling's transform (Programming the Hilbert curve, AIP
// Conf. Proc. 707, 2004) to the curve's transposed form, whose bits, taken
// from the top level down and x, y, z within a level, spell the index.  Cells
// adjacent in the index are adjacent in space (the Z-curve jumps at every
// block boundary), so the targets in flight at once cover a more compact region.
__device__ inline uint32_t hilbert3(uint32_t x, uint32_t y, uint32_t z, int bits) {
  uint32_t X[3] = {x, y, z};
  const uint32_t top = 1u << (bits - 1);
  for (uint32_t q = top; q > 1u; q >>= 1) {   // undo the excess rotations, level by level
    const uint32_t p = q - 1u;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (X[i] & q) {
        X[0] ^= p;
      } else {
        const uint32_t t = (X[0] ^ X[i]) & p;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  X[1] ^= X[0];   // Gray code
  X[2] ^= X[1];
  uint32_t t = 0;
  for (uint32_t q = top; q > 1u; q >>= 1)
    if (X[2] & q) t ^= q - 1u;
  return (spread3(X[0] ^ t) << 2) | (spread3(X[1] ^ t) << 1) | spread3(X[2] ^ t);
}

__global__ __launch_bounds__(256) void k_sched_bbox(int64_t N, const float* pos, float* partial,
                                                    int32_t* counts, int64_t ncell) {
  __shared__ float red[6][256];
  const int t = threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t c = (int64_t)blockIdx.x * 256 + t; c < ncell; c += stride) counts[c] = 0;
  float v[6] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int64_t at = (int64_t)blockIdx.x * 256 + t; at < N; at += stride) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float x = pos[3 * at + d];
      v[d] = fminf(v[d], x);
      v[3 + d] = fmaxf(v[3 + d], x);
    }
  }
#pragma unroll
  for (int d = 0; d < 6; ++d) red[d][t] = v[d];
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

__global__ __launch_bounds__(256) void k_sched_count(int64_t N, const float* pos,
                                                     const float* partial, int bits,
                                                     int32_t* cell, int32_t* counts) {
  static_assert(kBboxBlocks == 256, "one partial box per thread");
  __shared__ float red[6][256];
  const int t = threadIdx.x;
#pragma unroll
  for (int d = 0; d < 6; ++d) red[d][t] = partial[t * 6 + d];
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
  float bb[6];
#pragma unroll
  for (int d = 0; d < 6; ++d) bb[d] = red[d][0];
  const int64_t at = (int64_t)blockIdx.x * 256 + t;
  if (at >= N) return;
  const int n = 1 << bits;
  uint32_t q[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    const float lo = bb[d], ext = bb[3 + d] - bb[d];
    const float u = ext > 0.0f ? (pos[3 * at + d] - lo) * ((float)n / ext) : 0.0f;
    // comparisons keep NaN and infinities out of the integer conversion
    q[d] = u >= 1.0f ? (u < (float)(n - 1) ? (uint32_t)u : (uint32_t)(n - 1)) : 0u;
  }
  const int32_t c = (int32_t)hilbert3(q[0], q[1], q[2], bits);
  cell[at] = c;
  atomicAdd(&counts[c], 1);
}

// exclusive scan of counts[0..kSchedCells) in place: one 1024-thread
// workgroup, eight tiles of 4096 counts with a running carry, each tile moved
// as one coalesced 16-byte access a thread
__global__ __launch_bounds__(1024) void k_sched_scan(int32_t* counts) {
  static_assert(kSchedCells == 8 * 4096, "eight tiles of 4096 counts");
  __shared__ int32_t part[16];
  const int t = threadIdx.x;
  int4* p = reinterpret_cast<int4*>(counts);
  int4 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = p[k * 1024 + t];
  int32_t carry = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int32_t sum = v[k].x + v[k].y + v[k].z + v[k].w;
    int32_t total;
    int32_t run = carry + block_exclusive_scan_1024(sum, part, &total);
    int4 o;
    o.x = run; run += v[k].x;
    o.y = run; run += v[k].y;
    o.z = run; run += v[k].z;
    o.w = run;
    p[k * 1024 + t] = o;
    carry += total;
    __syncthreads();   // part is rewritten by the next tile's scan
  }
}

__global__ __launch_bounds__(256) void k_sched_scatter(int64_t N, const int32_t* cell,
                                                       int32_t* offsets, int32_t* sched) {
  const int64_t at = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (at >= N) return;
  sched[atomicAdd(&offsets[cell[at]], 1)] = (int32_t)at;
}

// ---------------------------------------------------------- launchers

namespace {

int last_error() { return static_cast<int>(hipGetLastError()); }

template <int L, typename T, bool WS>
int eaas_go(int V, const EaasArgs& a, const EaasCoef& cf, hipStream_t s) {
  const int64_t per_block = (int64_t)kWavesPerBlock * (64 >> a.lane_log);
  const dim3 grid((unsigned)((a.n + per_block - 1) / per_block));
  (void)hipGetLastError();
  switch (V) {
    case 1: hipLaunchKernelGGL((k_eaas<L, 1, T, WS>), grid, dim3(256), 0, s, a, cf); break;
    case 2: hipLaunchKernelGGL((k_eaas<L, 2, T, WS>), grid, dim3(256), 0, s, a, cf); break;
    case 4: hipLaunchKernelGGL((k_eaas<L, 4, T, WS>), grid, dim3(256), 0, s, a, cf); break;
    case 8:
      if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((k_eaas<L, 8, T, WS>), grid, dim3(256), 0, s, a, cf);
        break;
      }
      return static_cast<int>(hipErrorInvalidValue);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return last_error();
}

// The single-target kernel, with the split epilogue when each lane's V channels
// are twice the subgroups (P = 64 >> lane_log)
template <int L, int V, typename T, int U, int HL, bool BUF, bool E>
void launch_single(const AggArgs& a, const EaasCoef& cf, dim3 grid, dim3 blk, hipStream_t s) {
  if (V == 2 * (64 >> a.lane_log))
    hipLaunchKernelGGL((k_aggregate<L, V, T, U, HL, BUF, E, true>), grid, blk, 0, s, a, cf);
  else
    hipLaunchKernelGGL((k_aggregate<L, V, T, U, HL, BUF, E, false>), grid, blk, 0, s, a, cf);
}

template <int L, typename T, bool E>
int agg_go(int V, const AggArgs& a, const EaasCoef& cf, hipStream_t s) {
  constexpr int U = 4;  // neighbours per subgroup in flight per iteration
  const int64_t blocks = (a.N + kAggWaves - 1) / kAggWaves;
  const dim3 grid((unsigned)((blocks + kXcds - 1) / kXcds * kXcds));
  const dim3 blk(64 * kAggWaves);
  // 4 channels per lane with 1, 2 or 4 lanes per head and a workspace under
  // 4 GiB take the specialised buffer-load kernels; anything else the general one
  const bool buf = (int64_t)a.N * (ncomp(L) + 1) * a.C * (int64_t)sizeof(T) < ((int64_t)1 << 32);
  (void)hipGetLastError();
  if constexpr (sizeof(T) == 2) {
    // bf16, 8 channels per lane: one neighbour per subgroup per iteration
    if (V == 8 && buf && a.head_lanes == 1) {
      launch_single<L, 8, T, 1, 1, true, E>(a, cf, grid, blk, s);
      return last_error();
    }
    if (V == 8 && buf && a.head_lanes == 2) {
      launch_single<L, 8, T, 1, 2, true, E>(a, cf, grid, blk, s);
      return last_error();
    }
    if (V == 8) {
      hipLaunchKernelGGL((k_aggregate<L, 8, T, 1, 0, false, E>), grid, blk, 0, s, a, cf);
      return last_error();
    }
  }
  if constexpr (sizeof(T) == 4) {
    // fp32, 4 channels per lane, rows of at most kMtMaxK slots, more than
    // kMtMinAtoms targets: several targets per wave share every row they read
    if (V == 4 && buf && a.K <= kMtMaxK && (a.N > kMtMinAtoms || a.shared) &&
        a.N < ((int64_t)1 << 30) &&
        (a.head_lanes == 1 || a.head_lanes == 2 || a.head_lanes == 4)) {
      constexpr int TM = E ? kMtTargetsEnv : kMtTargets;
      constexpr int UM = E ? kMtInflightEnv : kMtInflight;
      const dim3 mgrid((unsigned)(unit_map(a.N, TM, kMtTailDen, kMtTailT).per_xcd * kXcds));
      const dim3 mblk(64 * kMtWaves);
      switch (a.head_lanes) {
        case 1: hipLaunchKernelGGL((k_aggregate_mt<L, TM, UM, 1, E>), mgrid, mblk, 0, s, a, cf); break;
        case 2: hipLaunchKernelGGL((k_aggregate_mt<L, TM, UM, 2, E>), mgrid, mblk, 0, s, a, cf); break;
        default: hipLaunchKernelGGL((k_aggregate_mt<L, TM, UM, 4, E>), mgrid, mblk, 0, s, a, cf); break;
      }
      return last_error();
    }
  }
  if (V == 4 && buf && a.head_lanes == 2) {
    launch_single<L, 4, T, U, 2, true, E>(a, cf, grid, blk, s);
  } else if (V == 4 && buf && a.head_lanes == 1) {
    launch_single<L, 4, T, U, 1, true, E>(a, cf, grid, blk, s);
  } else if (V == 4 && buf && a.head_lanes == 4) {
    launch_single<L, 4, T, U, 4, true, E>(a, cf, grid, blk, s);
  } else {
    switch (V) {
      case 1: hipLaunchKernelGGL((k_aggregate<L, 1, T, U, 0, false, E>), grid, blk, 0, s, a, cf); break;
      case 2: hipLaunchKernelGGL((k_aggregate<L, 2, T, U, 0, false, E>), grid, blk, 0, s, a, cf); break;
      case 4: hipLaunchKernelGGL((k_aggregate<L, 4, T, U, 0, false, E>), grid, blk, 0, s, a, cf); break;
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  }
  return last_error();
}

template <typename T>
int eaas_l(int lmax, int V, bool ws, const EaasArgs& a, const EaasCoef& cf, hipStream_t s) {
  switch (lmax) {
    case 0: return ws ? eaas_go<0, T, true>(V, a, cf, s) : eaas_go<0, T, false>(V, a, cf, s);
    case 1: return ws ? eaas_go<1, T, true>(V, a, cf, s) : eaas_go<1, T, false>(V, a, cf, s);
    case 2: return ws ? eaas_go<2, T, true>(V, a, cf, s) : eaas_go<2, T, false>(V, a, cf, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

template <typename T, bool E>
int agg_l(int lmax, int V, const AggArgs& a, const EaasCoef& cf, hipStream_t s) {
  switch (lmax) {
    case 0: return agg_go<0, T, E>(V, a, cf, s);
    case 1: return agg_go<1, T, E>(V, a, cf, s);
    case 2: return agg_go<2, T, E>(V, a, cf, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace

int launch_eaas(int lmax, int dtype, int V, bool to_workspace, const EaasArgs& a,
                const EaasCoef& cf, hipStream_t s) {
  return dtype == 0 ? eaas_l<float>(lmax, V, to_workspace, a, cf, s)
                    : eaas_l<uint16_t>(lmax, V, to_workspace, a, cf, s);
}

int launch_aggregate(int lmax, int dtype, int V, const AggArgs& a, const EaasCoef& cf,
                     hipStream_t s) {
  if (a.env_inv_rc > 0.0f)
    return dtype == 0 ? agg_l<float, true>(lmax, V, a, cf, s)
                      : agg_l<uint16_t, true>(lmax, V, a, cf, s);
  return dtype == 0 ? agg_l<float, false>(lmax, V, a, cf, s)
                    : agg_l<uint16_t, false>(lmax, V, a, cf, s);
}

int launch_frames(int lmax, int64_t n, const float* r, float* Q, float* D, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_frames, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, lmax, n, r, Q,
                     D);
  return last_error();
}

int launch_validate(int64_t N, int K, const int32_t* idx, const uint8_t* mask, int32_t* flag,
                    hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_clear_flag, dim3(1), dim3(1), 0, s, flag);
  const int64_t total = N * (int64_t)K;
  hipLaunchKernelGGL(k_validate, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, total, N,
                     idx, mask, flag);
  return last_error();
}

int launch_schedule(int64_t N, const float* pos, const SchedScratch& sc, hipStream_t s) {
  (void)hipGetLastError();
  const dim3 grid_n((unsigned)((N + 255) / 256));
  hipLaunchKernelGGL(k_sched_bbox, dim3(kBboxBlocks), dim3(256), 0, s, N, pos, sc.partial,
                     sc.counts, (int64_t)kSchedCells);
  hipLaunchKernelGGL(k_sched_count, grid_n, dim3(256), 0, s, N, pos, sc.partial, sc.bits, sc.cell,
                     sc.counts);
  hipLaunchKernelGGL(k_sched_scan, dim3(1), dim3(1024), 0, s, sc.counts);
  hipLaunchKernelGGL(k_sched_scatter, grid_n, dim3(256), 0, s, N, sc.cell, sc.counts, sc.sched);
  return last_error();
}

}  // namespace e2f
