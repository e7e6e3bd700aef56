// e2f_backward.hip -- vector-Jacobian product of the on-the-fly attention (fp32
// arithmetic; bf16 storage is widened exactly into fp32 copies first, and dL/dh
// is rounded back at the end).
//
// For L = <G, out> with out_i = T(r_i) m_i, m_i = sum_j a_ij h'_j and
// h'_j = T(r_j) h_j (T(r) = the EAAS coupling with R(r)), the gradients are
//   dm_i   = T(r_i)^T G_i                                   (adjoint EAAS)
//   D_ih   = <dm_i, m_i>_h                                  (per head)
//   ds_ijh = a_ijh (<dm_i, h'_j>_h - D_ih)                  (softmax backward)
//   dq_i   = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i
//   dh'_j  = sum_i a_ij dm_i
//   dh_j   = T(r_j)^T dh'_j + e_(l=0) (dq_j + dk_j)
//   dpos_i = grad_r <G_i, T(r) m_i> at r_i + grad_r <dh'_i, T(r) h_i> at r_i
// with a_ij recomputed from the forward's saved log-sum-exp, as in the
// recompute scheme of FlashAttention-2, so no per-edge tensor is stored.
// q_i is read from the forward workspace's query rows.  Through learned
// projections (BwdArgs::dk set) h is the value rows v = h W_V, and the source
// pass stores dk_j and dv_j = T(r_j)^T dh'_j apart; the projections' own
// backward follows in e2f_project_bwd.hip.
//
// k_bwd_prep    per atom: dm, D, the step-3 part of dpos
// k_bwd_q       per target, streaming its sorted neighbours: dq
// k_bwd_q_mt    the same for three targets a wave (two with the envelope),
//               reading the union of their rows once
// k_bwd_src     per source, streaming the targets that list it (reverse list,
//               sorted): dh', dk, then dh and the step-1 part of dpos
// k_bwd_src_mt  the same for two sources a wave over the union of their
//               reverse lists (sources listed at most kSrcShareMaxL times)
// The reverse list is a CSR built with a count, a scan and a fill (atomics
// aggregated in LDS per group of spatially adjacent targets); the per-source
// sort makes the summation order independent of the fill order (lists longer
// than kRevTile, read in tiles, are sorted whole first, up to kRevSortMax).  Rows are read through buffer resources
// (32-bit offsets) when the row arrays fit 4 GiB.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {
namespace {

__device__ inline float exp2_b(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ inline float dpp_b(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int HL>
__device__ inline float head_sum_b(float x, int hl) {
  if constexpr (HL > 0) {
    if constexpr (HL >= 2) x += dpp_b<0xB1>(x);
    if constexpr (HL >= 4) x += dpp_b<0x4E>(x);
    if constexpr (HL >= 8) x += dpp_b<0x141>(x);
    if constexpr (HL >= 16) x += dpp_b<0x140>(x);
    return x;
  } else {
    if (hl >= 2) x += dpp_b<0xB1>(x);
    if (hl >= 4) x += dpp_b<0x4E>(x);
    if (hl >= 8) x += dpp_b<0x141>(x);
    if (hl >= 16) x += dpp_b<0x140>(x);
    if (hl >= 32) x += __shfl_xor(x, 16);
    if (hl >= 64) x += __shfl_xor(x, 32);
    return x;
  }
}

__device__ inline void wave_sync_b() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int V>
__device__ inline void ld(const float* p, float* o) {
  VecIO<float, V>::load(p, o);
}
template <int V>
__device__ inline void st(float* p, const float* o) {
  VecIO<float, V>::store(p, o);
}

// ascending sort of nb[0..cnt) by one wave (cnt <= MAXN)
template <int MAXN>
__device__ inline void sort_list(int* nb, int cnt, int lane) {
  wave_sort<MAXN>(reinterpret_cast<uint32_t*>(nb), cnt, lane, 0x7fffffffu);
}

// the target or source handled by this wave (Hilbert-curve schedule, XCD-aware order)
__device__ inline int64_t scheduled_atom(const int32_t* sched, int64_t N, int w) {
  const int64_t per_xcd = (int64_t)gridDim.x / kXcds;
  const int64_t blk = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int64_t slot = blk * kWavesPerBlock + w;
  if (slot >= N) return -1;
  const int64_t i = sched ? (int64_t)sched[slot] : slot;
  return (i >= 0 && i < N) ? i : -1;
}

// ---------------------------------------------------------------- prep

template <int LMAX, int V, int HL>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lg = a.lane_log;
  const int G2 = 1 << lg;
  const int sub = lane >> lg;
  const int gl = lane & (G2 - 1);
  const int64_t atom = ((int64_t)blockIdx.x * kWavesPerBlock + w) * (64 >> lg) + sub;
  if (atom >= a.N) return;  // whole subgroup: the reductions below stay inside it
  const int C = a.C;
  const int c0 = gl * V;
  const bool act = c0 < C;
  const int cl = act ? c0 : 0;
  const Frame f = make_frame(a.pos[3 * atom], a.pos[3 * atom + 1], a.pos[3 * atom + 2]);
  const Dy2 d = make_dy2(f);
  const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
  Reindex<LMAX> Rrad, Rhat;
  make_grad_reindex<LMAX>(cf, f, Rrad, Rhat);

  const int64_t base = atom * (int64_t)S * C;
  float g[S][V], m[S][V], dm[S][V], q[V];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    ld<V>(a.gout + base + s * C + cl, g[s]);
    ld<V>(a.msg + base + s * C + cl, m[s]);
  }
  ld<V>(a.q + atom * C + cl, q);
  float Dp = 0.0f;
  float acc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float gv[S], mv[S], out[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      gv[s] = g[s][v];
      mv[s] = m[s][v];
    }
    eaas_channel_t<LMAX>(gv, out, f, d, R);  // gv is rotated in place
#pragma unroll
    for (int s = 0; s < S; ++s) {
      dm[s][v] = out[s];
      Dp = fmaf(out[s], mv[s], Dp);
    }
    // position gradient of <G, T(r) m>: both in the aligned frame (gv already is)
    rotate_in<LMAX>(mv, f, d);
    pos_grad_channel<LMAX>(mv, gv, Rrad, Rhat, acc);
  }
  if (!act) {
    Dp = 0.0f;
    acc[0] = acc[1] = acc[2] = 0.0f;
  }
  Dp = head_sum_b<HL>(Dp, a.head_lanes);
  if (act && (gl & (a.head_lanes - 1)) == 0) a.dh[atom * a.heads + c0 / (C / a.heads)] = Dp;
  for (int o = 1; o < G2; o <<= 1) {
#pragma unroll
    for (int k = 0; k < 3; ++k) acc[k] += __shfl_xor(acc[k], o);
  }
  if (gl == 0) {
    float gp[3];
    frame_to_global(f, acc, gp);
#pragma unroll
    for (int k = 0; k < 3; ++k) a.grad_pos[3 * atom + k] = gp[k];
  }
  if (act) {
    float* row = a.brows + atom * (int64_t)(S + 1) * C;
    st<V>(row + c0, q);
#pragma unroll
    for (int s = 0; s < S; ++s) st<V>(row + (s + 1) * C + c0, dm[s]);
  }
}

// -------------------------------------------------- target-centric dq

template <int LMAX, int V, int U, int HL, bool BUF, bool ENV>
__global__ __launch_bounds__(256) void k_bwd_q(BwdArgs a) {
  constexpr int S = ncomp(LMAX);
  __shared__ int s_nb[kWavesPerBlock][kTile];
  // envelope per sorted slot: log2 u, then d ln u / d r_i as a vector
  __shared__ float4 s_env[kWavesPerBlock][ENV ? kTile : 1];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t i = scheduled_atom(a.sched, a.N, w);
  if (i < 0) return;
  const int lg = a.lane_log;
  const int P = 64 >> lg;
  const int sub = lane >> lg;
  const int c0 = (lane & ((1 << lg) - 1)) * V;
  const bool act = c0 < a.C;
  const int cl = act ? c0 : 0;
  const int C = a.C, K = a.K;
  const int64_t N = a.N;
  const int64_t row = (int64_t)(S + 1) * C;
  const int head = cl / (C / a.heads);
  const uint32_t row_bytes = (uint32_t)(row * 4);
  const uint32_t cbytes = (uint32_t)C * 4u;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.ws, BUF ? (uint32_t)(N * row * 4) : 0u);

  float q[V], dm[S][V];
  ld<V>(a.brows + i * row + cl, q);
#pragma unroll
  for (int s = 0; s < S; ++s) ld<V>(a.brows + i * row + (s + 1) * C + cl, dm[s]);
  const float L2 = a.lse[i * a.heads + head] * 1.4426950408889634f;
  const float Dv = a.dh[i * a.heads + head];
  float dq[V];
#pragma unroll
  for (int v = 0; v < V; ++v) dq[v] = 0.0f;
  float gpos[3] = {0.0f, 0.0f, 0.0f};   // envelope part of dL/dr_i, this lane's head share

  const int32_t* irow = a.idx + i * K;
  const uint8_t* mrow = a.mask + i * K;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* nb = s_nb[w];
  for (int t0 = 0; t0 < K; t0 += kTile) {
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
    sort_list<kTile>(nb, cnt, lane);
    if constexpr (ENV) {
      const float xi = a.pos[3 * i], yi = a.pos[3 * i + 1], zi = a.pos[3 * i + 2];
      for (int e = lane; e < cnt; e += 64) {
        const int j = nb[e];
        const float xj = a.pos[3 * j], yj = a.pos[3 * j + 1], zj = a.pos[3 * j + 2];
        const float dx = xi - xj, dy = yi - yj, dz = zi - zj;
        const EnvTerm et = envelope_term(xi, yi, zi, xj, yj, zj, a.env_rc);
        s_env[w][e] = make_float4(et.log2u, et.dlog * dx, et.dlog * dy, et.dlog * dz);
      }
      wave_sync_b();
    }
    for (int n0 = 0; n0 < cnt; n0 += P * U) {
      Raw<float, V> kv[U][S + 1];
      bool val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * P + sub;
        val[u] = n < cnt;
        const int jn = nb[val[u] ? n : cnt - 1];
        if constexpr (BUF) {
          const uint32_t voff = (uint32_t)jn * row_bytes + (uint32_t)cl * 4u;
#pragma unroll
          for (int r = 0; r <= S; ++r) buffer_load_raw<float, V>(rsrc, voff, (uint32_t)r * cbytes, kv[u][r]);
        } else {
          const float* src = a.ws + (int64_t)jn * row + cl;
#pragma unroll
          for (int r = 0; r <= S; ++r) ld<V>(src + r * C, kv[u][r].f);
        }
      }
      // keep every neighbour's loads in flight before the first use
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float qk = 0.0f, dp = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) qk = fmaf(q[v], kv[u][0].f[v], qk);
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
          for (int v = 0; v < V; ++v) dp = fmaf(dm[r][v], kv[u][r + 1].f[v], dp);
        qk = head_sum_b<HL>(qk, a.head_lanes);
        dp = head_sum_b<HL>(dp, a.head_lanes);
        float4 env = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if constexpr (ENV) env = s_env[w][val[u] ? n0 + u * P + sub : 0];
        // a slot beyond the envelope weighs 0 (its target's lse may itself be -inf)
        const float alpha =
            (val[u] && env.x != -INFINITY) ? exp2_b(qk * a.scale_log2e + env.x - L2) : 0.0f;
        const float dsn = alpha * (dp - Dv);   // gradient of this head's (natural) logit
        const float ds = dsn * a.scale;
#pragma unroll
        for (int v = 0; v < V; ++v) dq[v] = fmaf(ds, kv[u][0].f[v], dq[v]);
        if constexpr (ENV) {
          // ln u_ij enters every head's logit: d/dr_i sums dsn over the heads
          gpos[0] = fmaf(dsn, env.y, gpos[0]);
          gpos[1] = fmaf(dsn, env.z, gpos[1]);
          gpos[2] = fmaf(dsn, env.w, gpos[2]);
        }
      }
    }
    wave_sync_b();
  }
  for (int o = 1 << lg; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < V; ++v) dq[v] += __shfl_xor(dq[v], o);
  }
  if constexpr (ENV) {
    // every head's value sits on head_lanes active lanes of each subgroup
    const float wgt = act ? 1.0f / (float)a.head_lanes : 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      float t = gpos[k] * wgt;
      for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
      gpos[k] = t;
    }
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 3; ++k) a.grad_pos[3 * i + k] += gpos[k];  // prep wrote its part
    }
  }
  if (sub == 0 && act) st<V>(a.dq + i * C + c0, dq);
}

// ------------------------------- target-centric dq, targets sharing rows
//
// k_bwd_q for T spatially adjacent targets per wavefront (fp32, 4 channels
// per lane, rows of at most kShareMaxK slots), built like the forward's shared
// aggregate: the targets' sources form one union (share_union), subgroup g
// streams the sources with j mod P == g in increasing j, each source's rows
// are read once and applied to every target that lists it (c slots weigh c
// times), and a target's state is touched only by its own sources, so its
// arithmetic depends on its own neighbour set alone.
// Three targets a wave (the smaller union beat two by 4% of the backward);
// with the envelope two, whose per-pair table would otherwise leave LDS for
// one block a CU.
// One wave a workgroup for the shared passes: the waves share nothing, and a
// workgroup's LDS is freed only when its last wave ends (backward 2.62 -> 2.51
// ms at Large against four waves).
constexpr int kBwWaves = 1;   // waves per workgroup of the shared passes
// closing units of both shared passes (unit_map): the last 1/kBwTailDen of each XCD's
// stretch in units of kBwTailT targets (target pass) or of one source (source pass)
constexpr int kBwTailDen = 16;
constexpr int kBwTailT = 2;
constexpr int kBqTargets = 3;      // targets per wave
constexpr int kBqTargetsEnv = 2;   // targets per wave, envelope variant
constexpr int kBqInflight = 2;     // union sources per subgroup in flight

template <int LMAX, int T, int U, int HL, bool ENV>
__global__ __launch_bounds__(64 * kBwWaves) void k_bwd_q_mt(BwdArgs a) {
  constexpr int S = ncomp(LMAX);
  constexpr int V = 4;
  constexpr int EN = ShareLds<T>::EN;
  constexpr int CW = ShareLds<T>::CW;
  __shared__ ShareLds<T> s_un[kBwWaves];
  // envelope per (target, union source): log2 u and the radial d ln u (the
  // direction comes from the source's position, gathered with its row), 8 bytes
  // a pair so that two blocks fit a CU
  __shared__ float2 s_env[kBwWaves][ENV ? T : 1][ENV ? EN : 1];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  static_assert(kBwWaves == 1, "one wave a workgroup");
  (void)w;
  int64_t slot0, xend;
  int cnt;   // targets of this unit
  unit_of_block(unit_map(a.N, T, ENV ? 0 : kBwTailDen, kBwTailT), blockIdx.x, T, kBwTailT, slot0,
                cnt, xend);
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
  const int lgp = 6 - lg;
  const int sub = lane >> lg;
  const int c0 = (lane & ((1 << lg) - 1)) * V;
  const bool act = c0 < C;
  const int cl = act ? c0 : 0;
  const int64_t row = (int64_t)(S + 1) * C;
  const int head = cl / (C / a.heads);
  const uint32_t row_bytes = (uint32_t)(row * 4);
  const uint32_t cbytes = (uint32_t)C * 4u;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.ws, (uint32_t)(N * row * 4));
  ShareLds<T>& un = s_un[w];

  (void)share_union_rows<T>(un, a.idx, a.mask, N, a.K, tg, lgp, lane,
                       [&](int t, int u, int32_t j) {
                         if constexpr (ENV) {
                           int64_t ti = tg[0];
#pragma unroll
                           for (int tt = 1; tt < T; ++tt)
                             if (t == tt) ti = tg[tt];
                           const EnvTerm et =
                               envelope_term(a.pos[3 * ti], a.pos[3 * ti + 1], a.pos[3 * ti + 2],
                                             a.pos[3 * j], a.pos[3 * j + 1], a.pos[3 * j + 2],
                                             a.env_rc);
                           s_env[w][t][u] = make_float2(et.log2u, et.dlog);
                         }
                       });
  const int my_cnt = un.bcnt[sub];
  const int my_start = un.bstart[sub];
  int maxlen = my_cnt;
  for (int o = 1; o < 64; o <<= 1) maxlen = max(maxlen, __shfl_xor(maxlen, o));

  // per-target state: q, dm (from the prep pass), lse (base 2), D, dq, envelope dpos
  float q[T][V], dm[T][S][V], L2[T], Dv[T], dq[T][V], gpos[T][3], pt[ENV ? T : 1][3];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t i = tg[t] >= 0 ? tg[t] : 0;
    if constexpr (ENV) {
      pt[t][0] = a.pos[3 * i];
      pt[t][1] = a.pos[3 * i + 1];
      pt[t][2] = a.pos[3 * i + 2];
    }
    ld<V>(a.brows + i * row + cl, q[t]);
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) ld<V>(a.brows + i * row + (s2 + 1) * C + cl, dm[t][s2]);
    L2[t] = a.lse[i * a.heads + head] * 1.4426950408889634f;
    Dv[t] = a.dh[i * a.heads + head];
#pragma unroll
    for (int v = 0; v < V; ++v) dq[t][v] = 0.0f;
    gpos[t][0] = gpos[t][1] = gpos[t][2] = 0.0f;
  }
#pragma unroll 1
  for (int it = 0; it < maxlen; it += U) {
    Raw<float, V> kv[U][S + 1];
    uint32_t cw[U][CW];
    int nidx[U];
    float pj[ENV ? U : 1][3];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool val = it + u < my_cnt;
      // a subgroup past the end of its bucket re-reads some valid source and adds nothing
      const int nn = val ? my_start + it + u : (my_cnt > 0 ? my_start + my_cnt - 1 : 0);
      nidx[u] = nn;
      const int64_t jn = un.uj[nn];
      const uint32_t voff = (uint32_t)jn * row_bytes + (uint32_t)cl * 4u;
      if constexpr (ENV) {
        pj[u][0] = a.pos[3 * jn];
        pj[u][1] = a.pos[3 * jn + 1];
        pj[u][2] = a.pos[3 * jn + 2];
      }
#pragma unroll
      for (int r = 0; r <= S; ++r)
        buffer_load_raw<float, V>(rsrc, voff, (uint32_t)r * cbytes, kv[u][r]);
#pragma unroll
      for (int c = 0; c < CW; ++c) cw[u][c] = val ? un.cnt[c][nn] : 0u;
    }
    // keep every source's loads in flight before the first use
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t m = share_count<CW>(cw[u], t);
        if (m != 0u) {   // uniform within the subgroup
          float qk = 0.0f, dp = 0.0f;
#pragma unroll
          for (int v = 0; v < V; ++v) qk = fmaf(q[t][v], kv[u][0].f[v], qk);
#pragma unroll
          for (int r = 0; r < S; ++r)
#pragma unroll
            for (int v = 0; v < V; ++v) dp = fmaf(dm[t][r][v], kv[u][r + 1].f[v], dp);
          qk = head_sum_b<HL>(qk, a.head_lanes);
          dp = head_sum_b<HL>(dp, a.head_lanes);
          float2 env = make_float2(0.0f, 0.0f);
          if constexpr (ENV) env = s_env[w][t][nidx[u]];
          // c slots of the source count c times; a pair beyond the envelope weighs 0
          const float alpha = env.x != -INFINITY
                                  ? exp2_b(qk * a.scale_log2e + env.x - L2[t]) * (float)m
                                  : 0.0f;
          const float dsn = alpha * (dp - Dv[t]);
          const float ds = dsn * a.scale;
#pragma unroll
          for (int v = 0; v < V; ++v) dq[t][v] = fmaf(ds, kv[u][0].f[v], dq[t][v]);
          if constexpr (ENV) {
            // d ln u / d r_target along r_target - r_source
            gpos[t][0] = fmaf(dsn, env.y * (pt[t][0] - pj[u][0]), gpos[t][0]);
            gpos[t][1] = fmaf(dsn, env.y * (pt[t][1] - pj[u][1]), gpos[t][1]);
            gpos[t][2] = fmaf(dsn, env.y * (pt[t][2] - pj[u][2]), gpos[t][2]);
          }
        }
      }
    }
  }
  // sum the subgroups (additions of two terms commute exactly)
  for (int o = 1 << lg; o < 64; o <<= 1) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < V; ++v) dq[t][v] += __shfl_xor(dq[t][v], o);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t i = tg[t];
    if constexpr (ENV) {
      // every head's value sits on head_lanes active lanes of each subgroup
      const float wgt = act ? 1.0f / (float)a.head_lanes : 0.0f;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        float v = gpos[t][k] * wgt;
        for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
        gpos[t][k] = v;
      }
      if (i >= 0 && lane == 0) {
#pragma unroll
        for (int k = 0; k < 3; ++k) a.grad_pos[3 * i + k] += gpos[t][k];  // prep wrote its part
      }
    }
    if (i >= 0 && sub == 0 && act) st<V>(a.dq + i * C + c0, dq[t]);
  }
}

// ------------------------------------------ source-centric dh', dk, dh, dpos

// dh_j and the step-1 part of dpos_j from the summed dh'_j, dk_j and envelope
// dpos of source j; run by the lanes of one subgroup (2^lg lanes, V channels each).
template <int LMAX, int V>
__device__ __forceinline__ void src_finish(const BwdArgs& a, const EaasCoef& cf, int64_t j,
                                           const float (&gdk)[V],
                                           const float (&gdhp)[ncomp(LMAX)][V],
                                           const float (&genv)[3], int lg, int gl, bool act,
                                           int cl, int c0) {
  constexpr int S = ncomp(LMAX);
  const int C = a.C;
  const Frame f = make_frame(a.pos[3 * j], a.pos[3 * j + 1], a.pos[3 * j + 2]);
  const Dy2 d = make_dy2(f);
  const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
  Reindex<LMAX> Rrad, Rhat;
  make_grad_reindex<LMAX>(cf, f, Rrad, Rhat);
  const int64_t base = j * (int64_t)S * C;
  const bool split = a.dk != nullptr;   // dk apart, and dh' only (the projections follow)
  float hj[S][V], dqj[V], gh[S][V];
#pragma unroll
  for (int s2 = 0; s2 < S; ++s2) ld<V>(a.h + base + s2 * C + cl, hj[s2]);
  if (!split) ld<V>(a.dq + j * C + cl, dqj);
  float acc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float gv[S], xv[S], out[S];
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
      gv[s2] = gdhp[s2][v];
      xv[s2] = hj[s2][v];
    }
    eaas_channel_t<LMAX>(gv, out, f, d, R);  // gv is rotated in place
    if (!split) out[0] += dqj[v] + gdk[v];
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) gh[s2][v] = out[s2];
    rotate_in<LMAX>(xv, f, d);
    pos_grad_channel<LMAX>(xv, gv, Rrad, Rhat, acc);
  }
  if (!act) acc[0] = acc[1] = acc[2] = 0.0f;
  // within the subgroup, whose lanes are all active here
  for (int o = 1; o < (1 << lg); o <<= 1) {
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) acc[kk] += __shfl_xor(acc[kk], o);
  }
  if (act) {
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) st<V>(a.grad_h + base + s2 * C + c0, gh[s2]);
    if (split) st<V>(a.dk + j * C + c0, gdk);
  }
  if (gl == 0) {
    float gp[3];
    frame_to_global(f, acc, gp);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) a.grad_pos[3 * j + kk] += gp[kk] + genv[kk];  // prep wrote the step-3 part
  }
}

// skip_le >= 0: sources listed by at most skip_le targets are left out (another
// kernel has done them).
template <int LMAX, int V, int U, int HL, bool BUF, bool ENV>
__global__ __launch_bounds__(256) void k_bwd_src(BwdArgs a, EaasCoef cf, int skip_le) {
  constexpr int S = ncomp(LMAX);
  __shared__ int s_nb[kWavesPerBlock][kRevTile];
  // envelope per sorted target: log2 u, then d ln u / d r_target as a vector
  __shared__ float4 s_env[kWavesPerBlock][ENV ? kRevTile : 1];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t j = scheduled_atom(a.sched, a.N, w);
  if (j < 0) return;
  if (skip_le >= 0 && a.rev_off[j + 1] - a.rev_off[j] <= skip_le) return;
  const int lg = a.lane_log;
  const int P = 64 >> lg;
  const int sub = lane >> lg;
  const int gl = lane & ((1 << lg) - 1);
  const int c0 = gl * V;
  const bool act = c0 < a.C;
  const int cl = act ? c0 : 0;
  const int C = a.C;
  const int64_t row = (int64_t)(S + 1) * C;
  const int head = cl / (C / a.heads);
  const uint32_t row_bytes = (uint32_t)(row * 4);
  const uint32_t cbytes = (uint32_t)C * 4u;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.brows, BUF ? (uint32_t)(a.N * row * 4) : 0u);

  float k[V], hp[S][V];
  ld<V>(a.ws + j * row + cl, k);
#pragma unroll
  for (int s = 0; s < S; ++s) ld<V>(a.ws + j * row + (s + 1) * C + cl, hp[s]);
  float dhp[S][V], dk[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    dk[v] = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) dhp[s][v] = 0.0f;
  }

  float gpos[3] = {0.0f, 0.0f, 0.0f};   // envelope part of dL/dr_j, this lane's head share
  const int beg = a.rev_off[j], end = a.rev_off[j + 1];
  int* nb = s_nb[w];
  for (int t0 = beg; t0 < end; t0 += kRevTile) {
    const int cnt = end - t0 < kRevTile ? end - t0 : kRevTile;
    for (int e = lane; e < cnt; e += 64) nb[e] = a.rev_idx[t0 + e];
    sort_list<kRevTile>(nb, cnt, lane);
    if constexpr (ENV) {
      const float xj = a.pos[3 * j], yj = a.pos[3 * j + 1], zj = a.pos[3 * j + 2];
      for (int e = lane; e < cnt; e += 64) {
        const int ti = nb[e];
        const float xi = a.pos[3 * ti], yi = a.pos[3 * ti + 1], zi = a.pos[3 * ti + 2];
        const float dx = xi - xj, dy = yi - yj, dz = zi - zj;
        const EnvTerm et = envelope_term(xi, yi, zi, xj, yj, zj, a.env_rc);
        s_env[w][e] = make_float4(et.log2u, et.dlog * dx, et.dlog * dy, et.dlog * dz);
      }
      wave_sync_b();
    }
    for (int n0 = 0; n0 < cnt; n0 += P * U) {
      Raw<float, V> qd[U][S + 1];
      float L2[U], Dv[U];
      bool val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * P + sub;
        val[u] = n < cnt;
        const int64_t ti = nb[val[u] ? n : cnt - 1];
        if constexpr (BUF) {
          const uint32_t voff = (uint32_t)ti * row_bytes + (uint32_t)cl * 4u;
#pragma unroll
          for (int r = 0; r <= S; ++r) buffer_load_raw<float, V>(rsrc, voff, (uint32_t)r * cbytes, qd[u][r]);
        } else {
          const float* src = a.brows + ti * row + cl;
#pragma unroll
          for (int r = 0; r <= S; ++r) ld<V>(src + r * C, qd[u][r].f);
        }
        L2[u] = a.lse[ti * a.heads + head] * 1.4426950408889634f;
        Dv[u] = a.dh[ti * a.heads + head];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float qk = 0.0f, dp = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) qk = fmaf(qd[u][0].f[v], k[v], qk);
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
          for (int v = 0; v < V; ++v) dp = fmaf(qd[u][r + 1].f[v], hp[r][v], dp);
        qk = head_sum_b<HL>(qk, a.head_lanes);
        dp = head_sum_b<HL>(dp, a.head_lanes);
        float4 env = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if constexpr (ENV) env = s_env[w][val[u] ? n0 + u * P + sub : 0];
        const float alpha =
            (val[u] && env.x != -INFINITY) ? exp2_b(qk * a.scale_log2e + env.x - L2[u]) : 0.0f;
        const float dsn = alpha * (dp - Dv[u]);
        const float ds = dsn * a.scale;
#pragma unroll
        for (int v = 0; v < V; ++v) dk[v] = fmaf(ds, qd[u][0].f[v], dk[v]);
        if constexpr (ENV) {
          // d ln u_ij / d r_j = -(d ln u_ij / d r_i)
          gpos[0] = fmaf(-dsn, env.y, gpos[0]);
          gpos[1] = fmaf(-dsn, env.z, gpos[1]);
          gpos[2] = fmaf(-dsn, env.w, gpos[2]);
        }
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
          for (int v = 0; v < V; ++v) dhp[r][v] = fmaf(alpha, qd[u][r + 1].f[v], dhp[r][v]);
      }
    }
    wave_sync_b();
  }
  for (int o = 1 << lg; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      dk[v] += __shfl_xor(dk[v], o);
#pragma unroll
      for (int s = 0; s < S; ++s) dhp[s][v] += __shfl_xor(dhp[s][v], o);
    }
  }
  if constexpr (ENV) {
    const float wgt = act ? 1.0f / (float)a.head_lanes : 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      float t = gpos[k] * wgt;
      for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
      gpos[k] = t;
    }
  }
  if (sub != 0) return;
  src_finish<LMAX, V>(a, cf, j, dk, dhp, gpos, lg, gl, act, cl, c0);
}

// ------------------------------ source pass, two sources per wave sharing rows
//
// The same sums as k_bwd_src for T sources of adjacent schedule slots (the
// schedule orders atoms along a space-filling curve, so neighbouring sources
// are listed by mostly the same targets).  Their reverse-list segments are
// merged into one union of targets, each with its slot count per source; the
// subgroups of the wave split the union into buckets, so each union target's
// row (q, dm) is read once for all T sources.  A target listing a source c
// times counts c times.  A source listed by more than kSrcShareMaxL targets is
// left to k_bwd_src, so which kernel handles a source, and its summation order
// (its own sorted segment, bucket by bucket), depend on its own segment alone.
// The sources' h' sits in LDS (read once per union target and source), which
// leaves registers for two union targets in flight at two waves a SIMD.  (The
// envelope variant stays with k_bwd_src: its per-pair table would leave LDS for
// one block a CU.)
constexpr int kBsSources = 2;                 // sources per wave
constexpr int kBsInflight = 2;                // union targets per subgroup in flight
constexpr int kSrcShareMaxL = 384;            // longest reverse-list segment shared

// Four channels a lane; needs at least T subgroups (lane_log <= 5).
template <int LMAX, int T, int U, int HL>
__global__ __launch_bounds__(64 * kBwWaves) void k_bwd_src_mt(BwdArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  constexpr int V = 4;
  using Lds = ShareLds<T, kSrcShareMaxL>;
  constexpr int CW = Lds::CW;
  __shared__ Lds s_un[kBwWaves];
  // h' of the wave's sources, one float4 per (source, component, lane of a subgroup)
  __shared__ float4 s_hp[kBwWaves][T][S][32];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  static_assert(kBwWaves == 1, "one wave a workgroup");
  (void)w;
  int64_t slot0, xend;
  int cnt;   // sources of this unit
  unit_of_block(unit_map(a.N, T, kBwTailDen, 1), blockIdx.x, T, 1, slot0, cnt, xend);
  if (slot0 >= a.N) return;  // whole wave: no workgroup barrier below
  const int64_t N = a.N;
  const int C = a.C;
  int64_t jo[T];
  int beg[T], len[T];
  bool any = false;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t sl = slot0 + t;
    int64_t j = -1;
    if (t < cnt && sl < N && sl < xend) j = a.sched ? (int64_t)a.sched[sl] : sl;
    beg[t] = 0;
    len[t] = 0;
    if (j >= 0 && j < N) {
      beg[t] = a.rev_off[j];
      len[t] = a.rev_off[j + 1] - beg[t];
      if (len[t] > kSrcShareMaxL) {  // k_bwd_src's
        j = -1;
        len[t] = 0;
      }
    } else {
      j = -1;
    }
    jo[t] = j;
    any |= j >= 0;
  }
  if (!any) return;
  const int lg = a.lane_log;
  const int lgp = 6 - lg;
  const int sub = lane >> lg;
  const int gl = lane & ((1 << lg) - 1);
  const int c0 = gl * V;
  const bool act = c0 < C;
  const int cl = act ? c0 : 0;
  const int64_t row = (int64_t)(S + 1) * C;
  const int head = cl / (C / a.heads);
  const uint32_t row_bytes = (uint32_t)(row * 4);
  const uint32_t cbytes = (uint32_t)C * 4u;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.brows, (uint32_t)(N * row * 4));
  Lds& un = s_un[w];

  (void)share_union<T, kSrcShareMaxL>(
      un, len,
      [&](int t, int sl) -> int {
        int b = beg[0];
#pragma unroll
        for (int tt = 1; tt < T; ++tt)
          if (t == tt) b = beg[tt];
        return a.rev_idx[b + sl];
      },
      lgp, lane, [](int, int, int32_t) {});
  const int my_cnt = un.bcnt[sub];
  const int my_start = un.bstart[sub];
  int maxlen = my_cnt;
  for (int o = 1; o < 64; o <<= 1) maxlen = max(maxlen, __shfl_xor(maxlen, o));

  // per-source state: k (registers), h' (LDS), dk, dh'
  float k[T][V], dk[T][V], dhp[T][S][V];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t j = jo[t] >= 0 ? jo[t] : 0;
    ld<V>(a.ws + j * row + cl, k[t]);
    if (sub == 0) {  // 2^lg <= 32 lanes
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2)
        s_hp[w][t][s2][gl] = *reinterpret_cast<const float4*>(a.ws + j * row + (s2 + 1) * C + cl);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      dk[t][v] = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) dhp[t][s2][v] = 0.0f;
    }
  }
  wave_sync_b();
#pragma unroll 1
  for (int it = 0; it < maxlen; it += U) {
    Raw<float, V> qd[U][S + 1];
    uint32_t cw[U][CW];
    int nidx[U];
    float L2[U], Dv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool val = it + u < my_cnt;
      // a subgroup past the end of its bucket re-reads some valid target and adds nothing
      const int nn = val ? my_start + it + u : (my_cnt > 0 ? my_start + my_cnt - 1 : 0);
      nidx[u] = nn;
      const int64_t ti = un.uj[nn];
      const uint32_t voff = (uint32_t)ti * row_bytes + (uint32_t)cl * 4u;
#pragma unroll
      for (int r = 0; r <= S; ++r)
        buffer_load_raw<float, V>(rsrc, voff, (uint32_t)r * cbytes, qd[u][r]);
      L2[u] = a.lse[ti * a.heads + head] * 1.4426950408889634f;
      Dv[u] = a.dh[ti * a.heads + head];
#pragma unroll
      for (int c = 0; c < CW; ++c) cw[u][c] = val ? un.cnt[c][nn] : 0u;
    }
    // keep every target's loads in flight before the first use
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t m = share_count<CW>(cw[u], t);
        if (m != 0u) {   // uniform within the subgroup
          float qk = 0.0f, dp = 0.0f;
#pragma unroll
          for (int v = 0; v < V; ++v) qk = fmaf(qd[u][0].f[v], k[t][v], qk);
#pragma unroll
          for (int r = 0; r < S; ++r) {
            const float4 x = s_hp[w][t][r][gl];
            dp = fmaf(qd[u][r + 1].f[0], x.x, dp);
            dp = fmaf(qd[u][r + 1].f[1], x.y, dp);
            dp = fmaf(qd[u][r + 1].f[2], x.z, dp);
            dp = fmaf(qd[u][r + 1].f[3], x.w, dp);
          }
          qk = head_sum_b<HL>(qk, HL);
          dp = head_sum_b<HL>(dp, HL);
          // c slots count c times
          const float alpha = exp2_b(qk * a.scale_log2e - L2[u]) * (float)m;
          const float ds = alpha * (dp - Dv[u]) * a.scale;
#pragma unroll
          for (int v = 0; v < V; ++v) dk[t][v] = fmaf(ds, qd[u][0].f[v], dk[t][v]);
#pragma unroll
          for (int r = 0; r < S; ++r)
#pragma unroll
            for (int v = 0; v < V; ++v) dhp[t][r][v] = fmaf(alpha, qd[u][r + 1].f[v], dhp[t][r][v]);
        }
      }
    }
  }
  // sum the subgroups (additions of two terms commute exactly)
  for (int o = 1 << lg; o < 64; o <<= 1) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        dk[t][v] += __shfl_xor(dk[t][v], o);
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) dhp[t][s2][v] += __shfl_xor(dhp[t][s2][v], o);
      }
  }
  // subgroup t finishes source t
  if (sub >= T) return;
  int64_t j = jo[0];
  float gdk[V], gdhp[S][V];
  const float genv[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int v = 0; v < V; ++v) {
    gdk[v] = dk[0][v];
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) gdhp[s2][v] = dhp[0][s2][v];
  }
#pragma unroll
  for (int t = 1; t < T; ++t) {
    if (sub == t) {
      j = jo[t];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        gdk[v] = dk[t][v];
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) gdhp[s2][v] = dhp[t][s2][v];
      }
    }
  }
  if (j >= 0) src_finish<LMAX, V>(a, cf, j, gdk, gdhp, genv, lg, gl, act, cl, c0);
}

// -------------------------------------------------------- reverse list

__global__ __launch_bounds__(256) void k_fill_i32(int64_t n, int32_t* p, int32_t v) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = v;
}

// Reverse-list count and fill, aggregated in LDS.  A 256-thread workgroup
// takes `per` consecutive targets of the schedule (at most kRevSlots slots);
// spatially adjacent targets share most sources, so an LDS hash table of
// (source, count) turns most global atomics into LDS atomics: one global atomic
// per distinct source per workgroup.  The fill also returns each slot's rank
// within its source and workgroup, so one atomic per source reserves the
// workgroup's block of entries.
// 8 slots a thread (8 targets of K = 256 a workgroup); 16 measured slower: the
// larger hash tables cost more than the global atomics they save.
constexpr int kRevPerThread = 8;                // slots per thread
constexpr int kRevSlots = 256 * kRevPerThread;  // slots per workgroup
constexpr int kRevHash = 2 * kRevSlots;         // hash table entries (load factor <= 1/2)
constexpr int kRevHashBits = kRevHash == 4096 ? 12 : (kRevHash == 8192 ? 13 : 14);
static_assert((1 << kRevHashBits) == kRevHash, "hash size");

__device__ inline int rev_hash_insert(int* keys, int* vals, int j, int* rank) {
  unsigned hh = ((unsigned)j * 2654435761u) >> (32 - kRevHashBits);
  while (true) {
    const int k = atomicCAS(&keys[hh], -1, j);
    if (k == -1 || k == j) {
      *rank = atomicAdd(&vals[hh], 1);
      return (int)hh;
    }
    hh = (hh + 1) & (kRevHash - 1);
  }
}

template <bool FILL>
__global__ __launch_bounds__(256) void k_rev_pass(int64_t N, int K, int per, const int32_t* idx,
                                                  const uint8_t* mask, const int32_t* sched,
                                                  int32_t* cnt_or_cur, int32_t* entries) {
  __shared__ int keys[kRevHash];
  __shared__ int vals[kRevHash];
  __shared__ int base[FILL ? kRevHash : 1];
  const int t = threadIdx.x;
  for (int e = t; e < kRevHash; e += 256) {
    keys[e] = -1;
    vals[e] = 0;
  }
  __syncthreads();
  const int64_t g0 = (int64_t)blockIdx.x * per;
  // every slot's target, then every slot's index and mask, are loaded before
  // the first insert, so the loads overlap instead of queueing behind the atomics
  constexpr int PT = kRevPerThread;
  int tg[PT], jv[PT], hs[PT], rk[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = t + 256 * u;
    const int64_t slot_t = g0 + e / K;
    tg[u] = -1;
    if (e < per * K && slot_t < N) tg[u] = sched ? sched[slot_t] : (int)slot_t;
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    jv[u] = -1;
    if (tg[u] >= 0) {
      const int64_t sl = (int64_t)tg[u] * K + (t + 256 * u) % K;
      const uint8_t m = mask[sl];
      const int32_t j = idx[sl];
      jv[u] = (m != 0 && j >= 0 && (int64_t)j < N) ? j : -1;
    }
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    hs[u] = -1;
    if (jv[u] >= 0) hs[u] = rev_hash_insert(keys, vals, jv[u], &rk[u]);
  }
  __syncthreads();
  for (int e = t; e < kRevHash; e += 256) {
    if (keys[e] >= 0) {
      const int b = atomicAdd(&cnt_or_cur[keys[e]], vals[e]);
      if constexpr (FILL) base[e] = b;
    }
  }
  if constexpr (FILL) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PT; ++u)
      if (hs[u] >= 0) entries[base[hs[u]] + rk[u]] = tg[u];
  }
}

// Sources listed by more than kRevTile targets: their lists are read in tiles of
// kRevTile in list order, so the fill's (atomic, run-dependent) order would leak
// into the summation order.  Each workgroup checks 256 sources; every long list
// among them (up to kRevSortMax entries) is sorted ascending by the whole
// workgroup in LDS (bitonic), so that the tiles are consecutive runs of the
// sorted list and the sums depend on the graph alone.
constexpr int kRevSortMax = 16384;

__global__ __launch_bounds__(256) void k_rev_sort_long(int64_t N, const int32_t* off,
                                                       int32_t* entries) {
  __shared__ int32_t s_key[kRevSortMax];
  __shared__ int32_t s_long[256];
  __shared__ int s_nlong;
  const int t = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * 256 + t;
  if (t == 0) s_nlong = 0;
  __syncthreads();
  if (j < N) {
    const int len = off[j + 1] - off[j];
    if (len > kRevTile && len <= kRevSortMax) s_long[atomicAdd(&s_nlong, 1)] = (int32_t)j;
  }
  __syncthreads();
  const int nl = s_nlong;
  for (int q = 0; q < nl; ++q) {   // uniform: every thread reads the same count
    const int32_t src = s_long[q];
    const int beg = off[src], len = off[src + 1] - beg;
    int n2 = 1;
    while (n2 < len) n2 <<= 1;
    for (int e = t; e < n2; e += 256) s_key[e] = e < len ? entries[beg + e] : 0x7fffffff;
    __syncthreads();
    for (int kk = 2; kk <= n2; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int e = t; e < n2; e += 256) {
          const int p = e ^ jj;
          if (p > e) {
            const int32_t a = s_key[e], b = s_key[p];
            const bool up = (e & kk) == 0;
            if ((a > b) == up) {
              s_key[e] = b;
              s_key[p] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int e = t; e < len; e += 256) entries[beg + e] = s_key[e];
    __syncthreads();   // s_key is rewritten for the next long list
  }
}

// exclusive scan, pass 1: each 1024-thread block scans kScanTile elements in place
__global__ __launch_bounds__(1024) void k_scan_tiles(int64_t n, int32_t* a, int32_t* tile_sums) {
  __shared__ int32_t part[16];
  const int t = threadIdx.x;
  const int64_t e0 = (int64_t)blockIdx.x * kScanTile + 4 * t;
  int32_t v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = e0 + k < n ? a[e0 + k] : 0;
  const int32_t sum = v[0] + v[1] + v[2] + v[3];
  int32_t total;
  int32_t run = block_exclusive_scan_1024(sum, part, &total);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (e0 + k < n) a[e0 + k] = run;
    run += v[k];
  }
  if (t == 1023) tile_sums[blockIdx.x] = total;
}

// pass 2: one block scans the tile totals (at most kScanTile of them); a[n] = total
__global__ __launch_bounds__(1024) void k_scan_top(int64_t n, int ntiles, int32_t* tile_sums,
                                                   int32_t* a) {
  __shared__ int32_t part[16];
  const int t = threadIdx.x;
  int32_t v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = 4 * t + k < ntiles ? tile_sums[4 * t + k] : 0;
  const int32_t sum = v[0] + v[1] + v[2] + v[3];
  int32_t total;
  int32_t run = block_exclusive_scan_1024(sum, part, &total);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (4 * t + k < ntiles) tile_sums[4 * t + k] = run;
    run += v[k];
  }
  if (t == 1023) a[n] = total;
}

// pass 3: add the tile offsets; keep a copy as the fill cursors
__global__ __launch_bounds__(256) void k_scan_fix(int64_t n, int32_t* a, const int32_t* tile_sums,
                                                  int32_t* cur) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int32_t v = a[e] + tile_sums[e / kScanTile];
  a[e] = v;
  cur[e] = v;
}

int last_err() { return static_cast<int>(hipGetLastError()); }

template <int L, int V, int HL, bool E>
int bwd_go(const BwdArgs& a, const EaasCoef& cf, hipStream_t s) {
  constexpr int UQ = 4;  // neighbours per subgroup in flight, target pass
  constexpr int US = 2;  // targets per subgroup in flight, source pass (more live registers)
  const int64_t per_block = (int64_t)kWavesPerBlock * (64 >> a.lane_log);
  const dim3 grid_prep((unsigned)((a.N + per_block - 1) / per_block));
  const int64_t blocks = (a.N + kWavesPerBlock - 1) / kWavesPerBlock;
  const dim3 grid((unsigned)((blocks + kXcds - 1) / kXcds * kXcds));
  // 32-bit buffer offsets when the row arrays fit 4 GiB
  const bool buf = a.N * (ncomp(L) + 1) * (int64_t)a.C * 4 < ((int64_t)1 << 32);
  hipLaunchKernelGGL((k_bwd_prep<L, V, HL>), grid_prep, dim3(256), 0, s, a, cf);
  if constexpr (V == 4 && HL > 0) {
    // several atoms per wave sharing every row they read (enough atoms to fill the
    // chip): the target pass for rows of at most kShareMaxK slots, the source pass
    // when each source gets a subgroup
    if (buf && (a.N > kMtMinAtoms || a.shared) && a.N < ((int64_t)1 << 30)) {
      if (a.K <= kShareMaxK) {
        constexpr int TQ = E ? kBqTargetsEnv : kBqTargets;
        const dim3 qgrid((unsigned)(unit_map(a.N, TQ, E ? 0 : kBwTailDen, kBwTailT).per_xcd * kXcds));
        hipLaunchKernelGGL((k_bwd_q_mt<L, TQ, kBqInflight, HL, E>), qgrid, dim3(64 * kBwWaves),
                           0, s, a);
      } else {
        hipLaunchKernelGGL((k_bwd_q<L, V, UQ, HL, true, E>), grid, dim3(256), 0, s, a);
      }
      if (!E && (64 >> a.lane_log) >= kBsSources) {
        const dim3 sgrid((unsigned)(unit_map(a.N, kBsSources, kBwTailDen, 1).per_xcd * kXcds));
        hipLaunchKernelGGL((k_bwd_src_mt<L, kBsSources, kBsInflight, HL>), sgrid,
                           dim3(64 * kBwWaves), 0, s, a, cf);
        // sources listed by more targets than the shared union holds
        hipLaunchKernelGGL((k_bwd_src<L, V, US, HL, true, E>), grid, dim3(256), 0, s, a, cf,
                           kSrcShareMaxL);
      } else {
        hipLaunchKernelGGL((k_bwd_src<L, V, US, HL, true, E>), grid, dim3(256), 0, s, a, cf, -1);
      }
      return last_err();
    }
  }
  if (buf) {
    hipLaunchKernelGGL((k_bwd_q<L, V, UQ, HL, true, E>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_bwd_src<L, V, US, HL, true, E>), grid, dim3(256), 0, s, a, cf, -1);
  } else {
    hipLaunchKernelGGL((k_bwd_q<L, V, UQ, HL, false, E>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_bwd_src<L, V, US, HL, false, E>), grid, dim3(256), 0, s, a, cf, -1);
  }
  return last_err();
}

template <int L, bool E>
int bwd_v(int V, const BwdArgs& a, const EaasCoef& cf, hipStream_t s) {
  if (V == 4 && a.head_lanes == 2) return bwd_go<L, 4, 2, E>(a, cf, s);
  if (V == 4 && a.head_lanes == 1) return bwd_go<L, 4, 1, E>(a, cf, s);
  switch (V) {
    case 1: return bwd_go<L, 1, 0, E>(a, cf, s);
    case 2: return bwd_go<L, 2, 0, E>(a, cf, s);
    case 4: return bwd_go<L, 4, 0, E>(a, cf, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

template <int L>
int bwd_l(int V, const BwdArgs& a, const EaasCoef& cf, hipStream_t s) {
  return a.env_inv_rc > 0.0f ? bwd_v<L, true>(V, a, cf, s) : bwd_v<L, false>(V, a, cf, s);
}

}  // namespace

int launch_scan_exclusive(int64_t n, int32_t* a, int32_t* tile_sums, int32_t* cur,
                          hipStream_t s) {
  const int ntiles = (int)((n + kScanTile - 1) / kScanTile);
  hipLaunchKernelGGL(k_scan_tiles, dim3((unsigned)ntiles), dim3(1024), 0, s, n, a, tile_sums);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(1024), 0, s, n, ntiles, tile_sums, a);
  hipLaunchKernelGGL(k_scan_fix, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, a,
                     tile_sums, cur);
  return last_err();
}

int launch_reverse_list(int64_t N, int K, const int32_t* idx, const uint8_t* mask,
                        const int32_t* sched, int32_t* off, int32_t* cur, int32_t* tile_sums,
                        int32_t* entries, hipStream_t s) {
  (void)hipGetLastError();
  const unsigned gn = (unsigned)((N + 255) / 256);
  // targets per workgroup: as many whole rows as fit kRevSlots (rows longer than
  // that are split over several workgroups by the slot range below)
  const int per = K <= kRevSlots ? kRevSlots / K : 1;
  if (K > kRevSlots) return static_cast<int>(hipErrorInvalidValue);
  const unsigned gr = (unsigned)((N + per - 1) / per);
  hipLaunchKernelGGL(k_fill_i32, dim3(gn), dim3(256), 0, s, N, off, 0);
  hipLaunchKernelGGL(k_rev_pass<false>, dim3(gr), dim3(256), 0, s, N, K, per, idx, mask, sched,
                     off, (int32_t*)nullptr);
  const int st = launch_scan_exclusive(N, off, tile_sums, cur, s);
  if (st != 0) return st;
  hipLaunchKernelGGL(k_rev_pass<true>, dim3(gr), dim3(256), 0, s, N, K, per, idx, mask, sched,
                     cur, entries);
  hipLaunchKernelGGL(k_rev_sort_long, dim3(gn), dim3(256), 0, s, N, off, entries);
  return last_err();
}

namespace {

// eight elements a thread, 16-byte loads of bf16; tails element by element
__global__ __launch_bounds__(256) void k_widen_bf16(int64_t n, const uint16_t* src, float* dst) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 + 8 <= n) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + e0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float4* o = reinterpret_cast<float4*>(dst + e0);
    o[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                       __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
    o[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                       __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
  } else {
    for (int64_t e = e0; e < n; ++e) dst[e] = bf16_to_f32(src[e]);
  }
}

__global__ __launch_bounds__(256) void k_narrow_bf16(int64_t n, const float* src, uint16_t* dst) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 + 8 <= n) {
    const float4 a = reinterpret_cast<const float4*>(src + e0)[0];
    const float4 b = reinterpret_cast<const float4*>(src + e0)[1];
    auto pk = [](float lo, float hi) { return f32x2_to_bf16x2(lo, hi); };
    *reinterpret_cast<uint4*>(dst + e0) = make_uint4(pk(a.x, a.y), pk(a.z, a.w), pk(b.x, b.y),
                                                     pk(b.z, b.w));
  } else {
    for (int64_t e = e0; e < n; ++e) dst[e] = f32_to_bf16(src[e]);
  }
}

}  // namespace

int launch_widen_bf16(int64_t n, const uint16_t* src, float* dst, hipStream_t s) {
  if (n <= 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_widen_bf16, dim3((unsigned)((n + 2047) / 2048)), dim3(256), 0, s, n, src,
                     dst);
  return last_err();
}

int launch_narrow_bf16(int64_t n, const float* src, uint16_t* dst, hipStream_t s) {
  if (n <= 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_narrow_bf16, dim3((unsigned)((n + 2047) / 2048)), dim3(256), 0, s, n, src,
                     dst);
  return last_err();
}

int launch_backward(int lmax, int V, const BwdArgs& a, const EaasCoef& cf, hipStream_t s) {
  (void)hipGetLastError();
  switch (lmax) {
    case 0: return bwd_l<0>(V, a, cf, s);
    case 1: return bwd_l<1>(V, a, cf, s);
    case 2: return bwd_l<2>(V, a, cf, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace e2f
