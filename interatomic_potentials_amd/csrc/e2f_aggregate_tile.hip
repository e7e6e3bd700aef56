// e2f_aggregate_tile.hip -- steps 2 and 3 (write-up section 3.2; gist.science
// summary 2.2, Eq. 6) for 16 spatially adjacent targets per workgroup, with the
// per-head logits and the weighted sums on the matrix cores.
//
// Sixteen consecutive targets of the spatial schedule list mostly the same
// sources: at 32,768 atoms with K = 256 their union is about 540 sources for
// 3,400 valid slots.  The workgroup reads every union row once and forms, per
// head h, the dense 16-target x 8-source blocks
//   logits  S_h = Q_h K_h^T      (v_mfma_f32_16x16x4f32, two steps over d = 8)
//   sums    O_h += P_h V_h        (the same MFMA, two steps of four sources)
// where P_h[t][j] is zero for a source target t does not list.  The MFMA
// accumulates its four products one after another, each exactly rounded like a
// fused multiply-add, in increasing k (measured on MI355X against that model on
// a million cases, zeros included).  A zero weight therefore leaves the sum
// exactly as it was, and each target's result is the chain of fused
// multiply-adds over its own sources in increasing source index: it does not
// depend on which other targets share the tile, the schedule or the slot order.
//
// So that no weight needs rescaling, the softmax reference is each (target,
// head)'s exact maximum logit, found in a first pass over the union's key rows
// (the same MFMA, so the same logits).  The weight sum rides along as one
// more column of V equal to 1.
//
// Per workgroup (8 waves, wave w owning heads 2w and 2w + 1):
//  1. keys (j << 4) | t for every valid slot of the 16 rows, sorted by the
//     workgroup (bitonic, 8 keys a thread in registers);
//  2. the union in increasing j with a 16-bit target mask per entry; a slot
//     repeating its predecessor's (j, t) opens a new entry, so a source listed
//     c times by a target is added c times;
//  3. pass 1: logits of every union entry, the maximum per (target, head);
//  4. pass 2, eight entries at a time: their rows (k and h', 5 KB a source at
//     C = 128) are staged in LDS with 16-byte loads (the next eight in flight in
//     registers meanwhile), then logits, weights and sums on the MFMA;
//  5. per target and head: normalise (0 for an empty row), the target-side
//     EAAS, one store.
// A tile in which some chunk holds a non-finite value (0 x inf would reach the
// targets that do not list its source) is redone on the vector ALUs: the same
// fused multiply-adds in the same order, skipping non-members, so finite results
// keep their bits and a non-finite source only reaches the targets that list it.
//
// Served layout: fp32 storage, C = 128, H = 16 (d = 8), rows of at most 256
// slots, N < 2^27; the host picks the other kernels for anything else.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "e2f_device.hpp"
#include "e2f_internal.hpp"

namespace e2f {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTtTargets = 16;                 // targets per workgroup (4 bits of a key)
constexpr int kTtWaves = 8;                    // waves per workgroup: two heads each
constexpr int kTtThreads = 64 * kTtWaves;
constexpr int kTtKpt = kTtTargets * kTileMaxK / kTtThreads;   // sort keys per thread
constexpr int kTtKeys = kTtTargets * kTileMaxK;
constexpr int kTtC = 128;
constexpr int kTtD = 8;                        // channels per head
constexpr int kTtPitch = kTtC + 8;             // floats per staged row (bank spread)
constexpr uint32_t kTtPad = 0xffffffffu;       // sorts after every key
constexpr int kTtChunk = 8;                    // union entries staged per step: two MFMA steps
static_assert(kTtKpt == 8, "sort layout");

template <int LMAX, int CH>
struct TileLds {
  static constexpr int S = ncomp(LMAX);
  uint32_t key[kTtKeys];                       // sort scratch, then the union's sources
  uint32_t mask[kTtKeys / 2];                  // 16-bit target masks, two entries a word
  alignas(16) float rows[CH * (S + 1) * kTtPitch];   // staged rows of one chunk
  int32_t part[kTtWaves];                      // scan partials
  int32_t bad[2];                              // chunk id + 1 when the chunk holds a non-finite value
};

__device__ inline void tt_sync() { __syncthreads(); }

// Bitonic sort of kTtThreads * KPT keys held blocked in registers (thread t:
// elements [t KPT, (t + 1) KPT)), ascending.  Strides below KPT compare within
// a thread, strides below 64 KPT across the lanes of a wave, larger ones across
// waves through LDS.
template <int KPT>
__device__ inline void tt_sort(uint32_t (&k)[KPT], uint32_t* lds, int tid) {
  constexpr int NK = kTtThreads * KPT;
  const int lane = tid & 63;
#pragma unroll
  for (int kk = 2; kk <= NK; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj >= 64 * KPT) {
#pragma unroll
        for (int r = 0; r < KPT; ++r) lds[tid * KPT + r] = k[r];
        tt_sync();
        const int pt = tid ^ (jj / KPT);
        const bool up = ((tid * KPT) & kk) == 0;
        const bool keep_min = ((tid & (jj / KPT)) == 0) == up;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
          const uint32_t p = lds[pt * KPT + r];
          k[r] = keep_min ? min(k[r], p) : max(k[r], p);
        }
        tt_sync();
      } else if (jj >= KPT) {
        const int dl = jj / KPT;
        const bool up = ((tid * KPT) & kk) == 0;
        const bool keep_min = ((lane & dl) == 0) == up;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
          const uint32_t p = (uint32_t)__shfl_xor((int)k[r], dl);
          k[r] = keep_min ? min(k[r], p) : max(k[r], p);
        }
      } else {
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
          if (r & jj) continue;
          const int r2 = r + jj;
          const bool up = ((tid * KPT + r) & kk) == 0;
          const uint32_t lo = min(k[r], k[r2]), hi = max(k[r], k[r2]);
          k[r] = up ? lo : hi;
          k[r2] = up ? hi : lo;
        }
      }
    }
  }
}

// Exclusive prefix of v over the workgroup's threads in thread order, and the total.
__device__ inline int32_t tt_scan(int32_t v, int32_t* part, int32_t* total, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  int32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t up = __shfl_up(inc, o);
    if (lane >= o) inc += up;
  }
  if (lane == 63) part[w] = inc;
  tt_sync();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int q = 0; q < kTtWaves; ++q) {
    before += q < w ? part[q] : 0;
    all += part[q];
  }
  *total = all;
  return before + inc - v;
}


__device__ inline float tt_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// a source's weight for one head: 2^(logit log2(e) scale - max), one fused
// multiply-add before the exponential on both the matrix-core and the vector path
__device__ inline float tt_weight(float logit, float sl2e, float mx) {
  return tt_exp2(fmaf(logit, sl2e, -mx));
}

// CH union entries a chunk (CH / 4 MFMA steps).  Four waves a SIMD (two workgroups a CU, so
// that one's union build, barriers and loads overlap the other's matrix work): the
// accumulators of two heads, the next chunk's rows in flight and the operands fit in 128
// registers at CH = 8.
template <int LMAX, int CH>
__global__ __launch_bounds__(kTtThreads, 4) void k_aggregate_tile(AggArgs a, EaasCoef cf) {
  constexpr int S = ncomp(LMAX);
  constexpr int ZC = S * kTtD;                     // column of the weight sum (V = 1)
  constexpr int NB = (ZC + 1 + 15) / 16;           // 16-column blocks of one head
  constexpr int RP = kTtPitch;
  constexpr int RS = (S + 1) * RP;                 // floats per staged source
  constexpr int PPS = (S + 1) * (kTtC / 4);        // 16-byte pieces per source
  constexpr int PIECES = CH * PPS;
  constexpr int KS = CH / 4;                       // MFMA steps of four entries a chunk
  static_assert(CH == 8 || CH == 16, "chunk of two or four MFMA steps");
  constexpr int PPT = (PIECES + kTtThreads - 1) / kTtThreads;
  constexpr int ZB = ZC / 16, ZG = (ZC % 16) / 4, ZR = ZC % 4;   // where the sum lands
  __shared__ TileLds<LMAX, CH> L;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane & 15;     // MFMA column: the target of the tile / a row of the A operand
  const int g = lane >> 4;       // MFMA lane group
  const int64_t N = a.N;
  const int K = a.K;
  // XCD-aware mapping of workgroups onto the schedule (the grid is a multiple of kXcds)
  const int64_t per_xcd = (int64_t)gridDim.x / kXcds;
  const int64_t blk = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int64_t slot0 = blk * kTtTargets;
  if (slot0 >= N) return;   // whole workgroup

  // 1. keys of the 16 rows' valid slots; empty slots and absent targets pad
  uint32_t k[kTtKpt];
  {
    const int f0 = tid * kTtKpt;                  // blocked: thread t holds keys [8t, 8t + 8)
    const bool vec = K % kTtKpt == 0 && (reinterpret_cast<uintptr_t>(a.idx) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.mask) & 7u) == 0;
    if (vec) {
      // the thread's eight slots lie in one row
      const int t = f0 / K, sl = f0 - t * K;
      const int64_t sidx = slot0 + t;
      int64_t i = -1;
      if (t < kTtTargets && sidx < N) i = a.sched ? (int64_t)a.sched[sidx] : sidx;
      if (i >= 0 && i < N) {
        const int4* ip = reinterpret_cast<const int4*>(a.idx + i * K + sl);
        const int4 j0 = ip[0], j1 = ip[1];
        const uint2 mm = *reinterpret_cast<const uint2*>(a.mask + i * K + sl);
        const int32_t js[8] = {j0.x, j0.y, j0.z, j0.w, j1.x, j1.y, j1.z, j1.w};
#pragma unroll
        for (int r = 0; r < kTtKpt; ++r) {
          const uint32_t mb = ((r < 4 ? mm.x : mm.y) >> (8 * (r & 3))) & 0xffu;
          const int32_t j = js[r];
          k[r] = (mb != 0u && j >= 0 && (int64_t)j < N) ? ((uint32_t)j << 4) | (uint32_t)t
                                                        : kTtPad;
        }
      } else {
#pragma unroll
        for (int r = 0; r < kTtKpt; ++r) k[r] = kTtPad;
      }
    } else {
#pragma unroll
      for (int r = 0; r < kTtKpt; ++r) {
        const int f = f0 + r;
        uint32_t key = kTtPad;
        const int t = f / K, sl = f - t * K;
        const int64_t sidx = slot0 + t;
        if (t < kTtTargets && sidx < N) {
          const int64_t i = a.sched ? (int64_t)a.sched[sidx] : sidx;
          if (i >= 0 && i < N) {
            const uint8_t m = a.mask[i * K + sl];
            const int32_t j = a.idx[i * K + sl];
            if (m != 0 && j >= 0 && (int64_t)j < N) key = ((uint32_t)j << 4) | (uint32_t)t;
          }
        }
        k[r] = key;
      }
    }
  }
  for (int e = tid; e < kTtKeys / 2; e += kTtThreads) L.mask[e] = 0u;
  if (tid < 2) L.bad[tid] = 0;
  tt_sort<kTtKpt>(k, L.key, tid);

  // 2. the union: an entry starts at a new source, or at a slot repeating its
  //    predecessor's (source, target); positions by a scan, targets or-ed into masks
  uint32_t prev;
  {
    L.key[tid * kTtKpt + kTtKpt - 1] = k[kTtKpt - 1];   // each thread's last key, for its successor
    tt_sync();
    prev = tid > 0 ? L.key[tid * kTtKpt - 1] : kTtPad;
  }
  auto starts = [](uint32_t pk, uint32_t kr) {
    return pk == kTtPad || (pk >> 4) != (kr >> 4) || pk == kr;
  };
  int nh = 0;
  {
    uint32_t pk = prev;
#pragma unroll
    for (int r = 0; r < kTtKpt; ++r) {
      if (k[r] != kTtPad && starts(pk, k[r])) ++nh;
      pk = k[r];
    }
  }
  int32_t n_u;
  const int32_t base = tt_scan(nh, L.part, &n_u, tid);
  tt_sync();   // every read of L.key above is done before the union overwrites it
  {
    int u = base - 1;
    uint32_t pk = prev;
#pragma unroll
    for (int r = 0; r < kTtKpt; ++r) {
      const uint32_t kr = k[r];
      if (kr != kTtPad) {
        if (starts(pk, kr)) {
          ++u;
          L.key[u] = kr >> 4;   // the union's sources, in increasing j
        }
        atomicOr(&L.mask[u >> 1], 1u << ((kr & 15u) + 16u * (uint32_t)(u & 1)));
      }
      pk = kr;
    }
  }
  tt_sync();
  const uint32_t* uj = L.key;
  auto member = [&](int u, int t) -> bool {
    return (L.mask[u >> 1] >> (16 * (u & 1) + t)) & 1u;
  };

  // this lane's target (MFMA column) and its query slices: channels 16w + 8hh + 2g + kappa
  int64_t ti = -1;
  {
    const int64_t sidx = slot0 + col;
    if (sidx < N) ti = a.sched ? (int64_t)a.sched[sidx] : sidx;
    if (ti >= N) ti = -1;
  }
  const int cq = 16 * w + 2 * g;   // channel of the lane's first query / key slice
  float qv[2][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (ti >= 0) {
      const float2 q2 = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q) +
                                                         ti * kTtC + cq + 8 * hh);
      qv[hh][0] = q2.x;
      qv[hh][1] = q2.y;
    } else {
      qv[hh][0] = qv[hh][1] = 0.0f;
    }
  }
  const float sl2e = a.scale_log2e;
  const uint32_t row_bytes = (uint32_t)((S + 1) * kTtC * 4);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.ws, (uint32_t)(N * (int64_t)row_bytes));

  // 3. pass 1: the maximum base-2 logit per (target, head) over the target's sources.
  //    Output row 4g + r of the logit block is entry u0 + 4g + r; row i of the A
  //    operand (lane col) is entry u0 + col.
  float mx[2] = {-INFINITY, -INFINITY};
  if (n_u > 0) {
    constexpr int P1 = 4;   // groups of 16 entries whose key slices are in flight together
    auto kload = [&](int u0, uint32_t (&kk)[P1][2][2]) {
#pragma unroll
      for (int p = 0; p < P1; ++p) {
        const int u = min(u0 + 16 * p + col, n_u - 1);
        const uint32_t off = uj[u] * row_bytes + (uint32_t)cq * 4u;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(off + 32u * hh), 0, 0);
          kk[p][hh][0] = v[0];
          kk[p][hh][1] = v[1];
        }
      }
    };
    uint32_t kc[P1][2][2], kn[P1][2][2];
    kload(0, kc);
    for (int u0 = 0; u0 < n_u; u0 += 16 * P1) {
      if (u0 + 16 * P1 < n_u) kload(u0 + 16 * P1, kn);
#pragma unroll
      for (int p = 0; p < P1; ++p) {
        const int ug = u0 + 16 * p;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          v4f lg = {0.0f, 0.0f, 0.0f, 0.0f};
          lg = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kc[p][hh][0]), qv[hh][0], lg, 0, 0, 0);
          lg = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kc[p][hh][1]), qv[hh][1], lg, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int u = ug + 4 * g + r;
            if (u < n_u && member(u, col)) mx[hh] = fmaxf(mx[hh], lg[r] * sl2e);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < P1; ++p)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          kc[p][hh][0] = kn[p][hh][0];
          kc[p][hh][1] = kn[p][hh][1];
        }
    }
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    mx[hh] = fmaxf(mx[hh], __shfl_xor(mx[hh], 16));
    mx[hh] = fmaxf(mx[hh], __shfl_xor(mx[hh], 32));
  }

  // 4. pass 2: weighted sums, eight union entries at a time.  acc[hh][b] holds
  //    columns 16b + 4g + r of head 2w + hh for target col: column s d + c is
  //    component s of channel c, column ZC the weight sum.
  v4f acc[2][NB];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[hh][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int n_chunks = (n_u + CH - 1) / CH;
  bool bad_tile = false;
  uint4 pf[PPT];
  // piece p = e kTtThreads + tid of a chunk: source slot p / PPS, 16-byte piece p % PPS of its
  // rows.  Entries past the union's end load its last source again (no member weighs them).
  auto fetch = [&](int c) {
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const int p = e * kTtThreads + tid;
      const int ss = p / PPS, rem = p - ss * PPS;
      const int u = min(c * CH + ss, n_u - 1);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (PIECES % kTtThreads == 0 || p < PIECES) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(uj[u] * row_bytes + rem * 16u), 0, 0);
        v = make_uint4(x[0], x[1], x[2], x[3]);
      }
      pf[e] = v;
    }
  };
  // stage the pieces in LDS; a chunk holding an infinity or NaN is flagged (x * 0 + t
  // turns t into NaN exactly then)
  auto stage = [&](int c) {
    float t = 0.0f;
    uint4* rows4 = reinterpret_cast<uint4*>(L.rows);
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const int p = e * kTtThreads + tid;
      if (PIECES % kTtThreads == 0 || p < PIECES) {
        const int ss = p / PPS, rem = p - ss * PPS;
        const int r = rem / (kTtC / 4), c4 = rem - r * (kTtC / 4);
        const uint4 v = pf[e];
        t = fmaf(__uint_as_float(v.x), 0.0f, t);
        t = fmaf(__uint_as_float(v.y), 0.0f, t);
        t = fmaf(__uint_as_float(v.z), 0.0f, t);
        t = fmaf(__uint_as_float(v.w), 0.0f, t);
        rows4[ss * (RS / 4) + r * (RP / 4) + c4] = v;
      }
    }
    if (t != t) L.bad[c & 1] = c + 1;
  };
  static_assert(RS % 4 == 0 && RP % 4 == 0, "16-byte aligned rows");
  if (n_chunks > 0) fetch(0);
  // lane-constant parts of the LDS addresses of the A operands; logit rows 4g' + r' with
  // r' >= KS read entry 0 and weigh 0
  const bool la_k_on = (col & 3) < KS;
  const int la_k = (la_k_on ? (4 * (col & 3) + (col >> 2)) * RS : 0) + cq;
  const int la_v = g * RS + (1 + (col >> 3)) * RP + 16 * w + (col & 7);   // V^T block 0, step 0
  for (int c = 0; c < n_chunks; ++c) {
    tt_sync();                 // every wave is done with the previous chunk's rows
    stage(c);
    if (c + 1 < n_chunks) fetch(c + 1);
    tt_sync();
    if (L.bad[c & 1] == c + 1) {   // the same for every wave: leave together
      bad_tile = true;
      break;
    }
    const int cu = c * CH;
    // logits of entries 4r + g (r < KS) for target col, output register r, both heads
    v4f lg[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float2 kk = *reinterpret_cast<const float2*>(&L.rows[la_k + 8 * hh]);
      const float k0 = la_k_on ? kk.x : 0.0f, k1 = la_k_on ? kk.y : 0.0f;
      lg[hh] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      lg[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(k0, qv[hh][0], lg[hh], 0, 0, 0);
      lg[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(k1, qv[hh][1], lg[hh], 0, 0, 0);
    }
    // which of the entries target col lists (the same for both heads)
    bool mem[KS];
#pragma unroll
    for (int r = 0; r < KS; ++r) {
      const int u = cu + 4 * r + g;
      const int uc = min(u, kTtKeys - 1);
      mem[r] = u < n_u && ((L.mask[uc >> 1] >> (16 * (uc & 1) + col)) & 1u);
    }
    float p[2][KS];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int r = 0; r < KS; ++r) {
        const float wgt = tt_weight(lg[hh][r], sl2e, mx[hh]);
        p[hh][r] = mem[r] ? wgt : 0.0f;
      }
    // step r outer, then head and block: consecutive MFMAs write different accumulators
#pragma unroll
    for (int r = 0; r < KS; ++r) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int cc = 16 * b + col;   // this lane's A row: column cc of V_h^T
          // the sum column reads 1, padding columns 0 (their address is kept in range)
          const int ai = min(la_v + 4 * r * RS + 2 * b * RP + 8 * hh, CH * RS - 1);
          const float lv = L.rows[ai];
          const float av = (16 * b + 15 < ZC || cc < ZC) ? lv : (cc == ZC ? 1.0f : 0.0f);
          acc[hh][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, p[hh][r], acc[hh][b], 0, 0, 0);
        }
      }
    }
  }

  // A chunk held a non-finite value: the whole tile again on the vector ALUs, the same
  // fused multiply-adds in the same order for members only, so finite results keep their
  // bits and a non-finite row reaches only the targets that list its source.  Rows are
  // staged one chunk at a time without prefetch (this path is for broken inputs).
  if (bad_tile) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[hh][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < n_chunks; ++c) {
      tt_sync();
      fetch(c);
      stage(c);
      tt_sync();
      const int cu = c * CH;
#pragma unroll 1
      for (int e = 0; e < CH; ++e) {
        const int u = cu + e;
        if (ti < 0 || u >= n_u || !member(u, col)) continue;
        const float* src = &L.rows[e * RS];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ch0 = 16 * w + 8 * hh;
          const float* qt = static_cast<const float*>(a.q) + ti * kTtC + ch0;
          float x = 0.0f;
#pragma unroll
          for (int kp = 0; kp < 2; ++kp)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) x = fmaf(src[ch0 + 2 * gg + kp], qt[2 * gg + kp], x);
          const float pe = tt_weight(x, sl2e, mx[hh]);
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int cc = 16 * b + 4 * g + r;
              if (cc < ZC)
                acc[hh][b][r] = fmaf(src[(1 + cc / kTtD) * RP + ch0 + cc % kTtD], pe, acc[hh][b][r]);
              else if (cc == ZC)
                acc[hh][b][r] = fmaf(1.0f, pe, acc[hh][b][r]);
            }
        }
      }
    }
  }

  // 5. per (target, head): normalise, target-side EAAS, store.  After the swap of
  //    the two lane halves a lane holds channels 4(g & 1) + 2(g >> 1) + {0, 1} of
  //    its head, all S components.
  Frame f{};
  Dy2 d{};
  Reindex<LMAX> R{};
  if (ti >= 0) {
    f = make_frame(a.pos[3 * ti], a.pos[3 * ti + 1], a.pos[3 * ti + 2]);
    d = make_dy2(f);
    R = make_reindex<LMAX>(cf, f);
  }
  const int chl = 4 * (g & 1) + 2 * (g >> 1);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const float z = __shfl(acc[hh][ZB][ZR], 16 * ZG + col);
    float x[2][2 * NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[hh][b][r]),
                                                         __float_as_uint(acc[hh][b][r + 2]),
                                                         false, false);
        x[r][2 * b] = __uint_as_float(sw[0]);
        x[r][2 * b + 1] = __uint_as_float(sw[1]);
      }
    if (ti < 0) continue;
    const int h = 2 * w + hh;
    if (a.lse != nullptr && g == 0)
      a.lse[ti * a.heads + h] = z > 0.0f ? (mx[hh] + log2f(z)) * 0.6931471805599453f : -INFINITY;
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    const int c0 = 16 * w + 8 * hh + chl;
    float m[2][S];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int s = 0; s < S; ++s) m[r][s] = x[r][s] * inv;
    if (a.out_msg != nullptr) {
      float* mp = static_cast<float*>(a.out_msg) + ti * (int64_t)S * kTtC + c0;
#pragma unroll
      for (int s = 0; s < S; ++s) *reinterpret_cast<float2*>(mp + s * kTtC) = make_float2(m[0][s], m[1][s]);
    }
    float y[2][S];
#pragma unroll
    for (int r = 0; r < 2; ++r) eaas_channel<LMAX>(m[r], y[r], f, d, R);
    float* op = static_cast<float*>(a.out) + ti * (int64_t)S * kTtC + c0;
#pragma unroll
    for (int s = 0; s < S; ++s) *reinterpret_cast<float2*>(op + s * kTtC) = make_float2(y[0][s], y[1][s]);
  }
}

template <int L>
void tile_go(const AggArgs& a, const EaasCoef& cf, hipStream_t s) {
  const int64_t blocks = (a.N + kTtTargets - 1) / kTtTargets;
  const dim3 grid((unsigned)((blocks + kXcds - 1) / kXcds * kXcds));
  hipLaunchKernelGGL((k_aggregate_tile<L, kTtChunk>), grid, dim3(kTtThreads), 0, s, a, cf);
}

}  // namespace

bool tile_supported(int lmax, int dtype, const AggArgs& a) {
  const int64_t block_bytes = (int64_t)(ncomp(lmax) + 1) * a.C * 4;   // k + h' rows of a source
  return lmax >= 0 && lmax <= kMaxLmax && dtype == 0 && a.C == kTtC && a.heads * kTtD == kTtC &&
         a.K >= 1 && a.K <= kTileMaxK && a.N >= 1 && a.N < ((int64_t)1 << 27) &&
         a.env_inv_rc <= 0.0f && a.N * block_bytes < ((int64_t)1 << 32);
}

int launch_aggregate_tile(int lmax, const AggArgs& a, const EaasCoef& cf, hipStream_t s) {
  (void)hipGetLastError();
  switch (lmax) {
    case 0: tile_go<0>(a, cf, s); break;
    case 1: tile_go<1>(a, cf, s); break;
    case 2: tile_go<2>(a, cf, s); break;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace e2f
