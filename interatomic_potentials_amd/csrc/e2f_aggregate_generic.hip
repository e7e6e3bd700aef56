// e2f_aggregate_generic.hip -- steps 2 and 3 (write-up section 3.2; gist.science
// summary 2.2) for any channel / head layout with C % H == 0: head widths that
// are not a power of two (d = 3, 5, 6, 12, ...) and rows too wide for one
// lane-vector per channel group (C up to 512 at fp32 and bf16).
//
// One wavefront per target.  Lane l owns channels c = l + 64 k, k < NCH.  Per
// neighbour, every lane multiplies its query and key channels and leaves the
// products in LDS; the lanes then sum each head's d products in channel order
// (one lane a head), and read back the logit of their own channels.  The online
// softmax state (running reference and normaliser, base 2, lazy rescale) is kept
// per channel slot; the channels of one head see the same logits, so they take
// the same decisions.  Neighbours are visited in increasing atom index after a
// ballot compaction and a register sort, as in the other aggregate kernels, so a
// target's result does not depend on its slot order.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {
namespace {

constexpr int kGenWaves = 4;          // waves (targets) per workgroup
constexpr float kGenSlack = 8.0f;     // lazy-rescale slack of the running reference (base 2)

__device__ inline void gen_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ inline float load1(const T* p) {
  float v;
  VecIO<T, 1>::load(p, &v);
  return v;
}

template <typename T>
__device__ inline void store1(T* p, float v) {
  VecIO<T, 1>::store(p, &v);
}

// NCH channel slots a lane (C <= 64 NCH)
template <int LMAX, typename T, int NCH, bool ENV>
__global__ __launch_bounds__(64 * kGenWaves) void k_aggregate_generic(AggArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  __shared__ int s_nb[kGenWaves][kTile];
  __shared__ float s_le[kGenWaves][ENV ? kTile : 1];   // log2 envelope per sorted slot
  __shared__ float s_prod[kGenWaves][64 * NCH];        // q_c k_c of one neighbour
  __shared__ float s_logit[kGenWaves][64 * NCH];       // head logits, one per head
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t per_xcd = (int64_t)gridDim.x / kXcds;
  const int64_t blk = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int64_t slot = blk * kGenWaves + w;
  if (slot >= a.N) return;   // whole wave
  const int64_t i = a.sched ? (int64_t)a.sched[slot] : slot;
  if (i < 0 || i >= a.N) return;
  const int C = a.C, K = a.K, H = a.heads;
  const int d = C / H;
  const int64_t N = a.N;
  const int64_t row = (int64_t)(S + 1) * C;
  const T* ws = static_cast<const T*>(a.ws);

  float q[NCH], mu[NCH], z[NCH], acc[NCH][S];
  int head[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    q[k] = c < C ? load1<T>(static_cast<const T*>(a.q) + i * C + c) : 0.0f;
    head[k] = c < C ? c / d : 0;
    mu[k] = -1e30f;
    z[k] = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) acc[k][s] = 0.0f;
  }

  const int32_t* irow = a.idx + i * K;
  const uint8_t* mrow = a.mask + i * K;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* nb = s_nb[w];
  float* prod = s_prod[w];
  float* logit = s_logit[w];
  for (int t0 = 0; t0 < K; t0 += kTile) {
    // compact this tile's valid, in-range slots into LDS, then sort them by atom index
    int cnt = 0;
    for (int c0 = 0; c0 < kTile && t0 + c0 < K; c0 += 64) {
      const int sl = t0 + c0 + lane;
      int j = -1;
      if (sl < K) {
        const uint8_t m = mrow[sl];
        const int jj = irow[sl];
        j = (m != 0 && jj >= 0 && (int64_t)jj < N) ? jj : -1;
      }
      const bool ok = j >= 0;
      const uint64_t b = __ballot(ok);
      if (ok) nb[cnt + __popcll(b & below)] = j;
      cnt += __popcll(b);
    }
    wave_sort<kTile>(reinterpret_cast<uint32_t*>(nb), cnt, lane, 0x7fffffffu);
    if constexpr (ENV) {
      const float xi = a.pos[3 * i], yi = a.pos[3 * i + 1], zi = a.pos[3 * i + 2];
      for (int e = lane; e < cnt; e += 64) {
        const int j = nb[e];
        s_le[w][e] = envelope_term(xi, yi, zi, a.pos[3 * j], a.pos[3 * j + 1], a.pos[3 * j + 2],
                                   a.env_rc).log2u;
      }
      gen_wave_sync();
    }
    for (int n = 0; n < cnt; ++n) {
      const int j = nb[n];
      const T* src = ws + (int64_t)j * row;
      // per-head logits: products through LDS, each head summed in channel order by one lane
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c = lane + 64 * k;
        if (c < C) prod[c] = q[k] * load1<T>(src + c);
      }
      gen_wave_sync();
      for (int h = lane; h < H; h += 64) {
        float sum = 0.0f;
        for (int c = h * d; c < (h + 1) * d; ++c) sum += prod[c];
        logit[h] = sum;
      }
      gen_wave_sync();
      float le = 0.0f;
      if constexpr (ENV) le = s_le[w][n];
      float sc[NCH];
      bool need_any = false;
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        sc[k] = logit[head[k]] * a.scale_log2e + le;
        need_any |= sc[k] > mu[k] + kGenSlack;
      }
      if (__any(need_any)) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const bool need = sc[k] > mu[k] + kGenSlack;
          const float mx = need ? sc[k] : mu[k];
          const float corr = __builtin_amdgcn_exp2f(mu[k] - mx);   // exactly 1 where not needed
          z[k] *= corr;
#pragma unroll
          for (int s = 0; s < S; ++s) acc[k][s] *= corr;
          mu[k] = mx;
        }
      }
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c = lane + 64 * k;
        const float p = __builtin_amdgcn_exp2f(sc[k] - mu[k]);
        z[k] += p;
        if (c < C) {
#pragma unroll
          for (int s = 0; s < S; ++s) acc[k][s] = fmaf(p, load1<T>(src + (s + 1) * C + c), acc[k][s]);
        }
      }
      gen_wave_sync();   // the next neighbour's products overwrite this one's
    }
    gen_wave_sync();     // every read of s_nb is done before the next tile rewrites it
  }

  // normalise (0 for a target without valid slots), lse, message, target-side EAAS, store
  const Frame f = make_frame(a.pos[3 * i], a.pos[3 * i + 1], a.pos[3 * i + 2]);
  const Dy2 dy = make_dy2(f);
  const Reindex<LMAX> R = make_reindex<LMAX>(cf, f);
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (c >= C) continue;
    if (a.lse != nullptr && c % d == 0)
      a.lse[i * H + c / d] = z[k] > 0.0f ? (mu[k] + log2f(z[k])) * 0.6931471805599453f : -INFINITY;
    const float inv = z[k] > 0.0f ? 1.0f / z[k] : 0.0f;
    float m[S], y[S];
#pragma unroll
    for (int s = 0; s < S; ++s) m[s] = acc[k][s] * inv;
    if (a.out_msg != nullptr) {
      if (a.msg_f32) {   // the message in fp32 whatever the storage type
        float* mp = static_cast<float*>(a.out_msg) + i * (int64_t)S * C + c;
#pragma unroll
        for (int s = 0; s < S; ++s) mp[s * C] = m[s];
      } else {
        T* mp = static_cast<T*>(a.out_msg) + i * (int64_t)S * C + c;
#pragma unroll
        for (int s = 0; s < S; ++s) store1<T>(mp + s * C, m[s]);
      }
    }
    eaas_channel<LMAX>(m, y, f, dy, R);
    T* op = static_cast<T*>(a.out) + i * (int64_t)S * C + c;
#pragma unroll
    for (int s = 0; s < S; ++s) store1<T>(op + s * C, y[s]);
  }
}

template <int L, typename T, bool E>
int gen_go(const AggArgs& a, const EaasCoef& cf, hipStream_t s) {
  const int64_t blocks = (a.N + kGenWaves - 1) / kGenWaves;
  const dim3 grid((unsigned)((blocks + kXcds - 1) / kXcds * kXcds));
  const dim3 blk(64 * kGenWaves);
  (void)hipGetLastError();
  const int nch = (a.C + 63) / 64;
  if (nch <= 1)
    hipLaunchKernelGGL((k_aggregate_generic<L, T, 1, E>), grid, blk, 0, s, a, cf);
  else if (nch <= 2)
    hipLaunchKernelGGL((k_aggregate_generic<L, T, 2, E>), grid, blk, 0, s, a, cf);
  else if (nch <= 4)
    hipLaunchKernelGGL((k_aggregate_generic<L, T, 4, E>), grid, blk, 0, s, a, cf);
  else if (nch <= 8)
    hipLaunchKernelGGL((k_aggregate_generic<L, T, 8, E>), grid, blk, 0, s, a, cf);
  else
    return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

template <typename T, bool E>
int gen_l(int lmax, const AggArgs& a, const EaasCoef& cf, hipStream_t s) {
  switch (lmax) {
    case 0: return gen_go<0, T, E>(a, cf, s);
    case 1: return gen_go<1, T, E>(a, cf, s);
    case 2: return gen_go<2, T, E>(a, cf, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace

int launch_aggregate_generic(int lmax, int dtype, const AggArgs& a, const EaasCoef& cf,
                             hipStream_t s) {
  const bool env = a.env_inv_rc > 0.0f;
  if (dtype == 0) return env ? gen_l<float, true>(lmax, a, cf, s) : gen_l<float, false>(lmax, a, cf, s);
  return env ? gen_l<uint16_t, true>(lmax, a, cf, s) : gen_l<uint16_t, false>(lmax, a, cf, s);
}

}  // namespace e2f
