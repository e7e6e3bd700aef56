// e2f_internal.hpp -- argument blocks shared by the host side of libe2f and
// its kernels.  Not part of the public ABI (include/e2f.h is).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace e2f {

constexpr int kMaxLmax = 2;
constexpr int kMaxPaths = 15;       // triangle-allowed (li, lf, lo) with all <= 2
constexpr int kWavesPerBlock = 4;   // 256-thread workgroups, one wave per target
constexpr int kTile = 256;          // neighbour slots compacted per pass
constexpr int kXcds = 8;            // gfx950 (MI350 series): 8 XCDs, workgroups dealt round-robin
constexpr int kBboxBlocks = 256;    // partial bounding boxes reduced by the schedule builder
constexpr int kSchedMaxBits = 5;    // Morton bits per axis of the schedule grid, at most
constexpr int kSchedCells = 1 << (3 * kSchedMaxBits);  // count entries always scanned

// Target schedule scratch, carved from the caller's workspace after the
// pre-coupled rows and the validation flag.
struct SchedScratch {
  int32_t* sched;      // [N] target order: atoms sorted by Morton cell
  int32_t* cell;       // [N] cell of each atom
  int32_t* counts;     // [kSchedCells] per-cell counts, then running offsets
  float* partial;      // [kBboxBlocks][6] partial (min, max) of the positions
  int bits;            // Morton bits per axis (<= kSchedMaxBits); cells used = 2^(3 bits)
};

// Sparse reindex weights, one row per path (lexicographic (li, lf, lo)):
// c[p][m] = w_p <li m lf 0 | lo m> for m = 0..2 (Condon-Shortley).
struct EaasCoef {
  float c[kMaxPaths][kMaxLmax + 1];
};

struct EaasArgs {
  const float* r;      // [n, 3]
  const void* h_in;    // [n, S, C]
  void* h_out;         // [n, S, C] or workspace [n, S + 1, C]
  int64_t n;
  int C;
  int lane_log;        // log2 of the lanes serving one atom (power of two <= 64)
};

struct AggArgs {
  const float* pos;        // [N, 3]
  const int32_t* idx;      // [N, K]
  const uint8_t* mask;     // [N, K]
  const void* ws;          // [N, S + 1, C]: row 0 = k, rows 1..S = h'
  void* out;               // [N, S, C]
  void* out_msg;           // [N, S, C] or nullptr
  int64_t N;
  int K;
  int C;
  int lane_log;            // log2 of the lanes serving one neighbour row
  int head_lanes;          // lanes per head = d / V (power of two)
  float scale_log2e;       // logit scale times log2(e)
  const int32_t* sched;    // [N] processing order of the targets
};

// launchers (kernels file); return 0 or a hipError_t value
int launch_eaas(int lmax, int dtype, int V, bool to_workspace, const EaasArgs& a,
                const EaasCoef& cf, hipStream_t s);
int launch_aggregate(int lmax, int dtype, int V, const AggArgs& a, const EaasCoef& cf,
                     hipStream_t s);
int launch_frames(int lmax, int64_t n, const float* r, float* Q, float* D, hipStream_t s);
int launch_validate(int64_t N, int K, const int32_t* idx, const uint8_t* mask, int32_t* flag,
                    hipStream_t s);
int launch_schedule(int64_t N, const float* pos, const SchedScratch& sc, hipStream_t s);

}  // namespace e2f
