// e2f_internal.hpp -- argument blocks shared by the host side of libe2f and
// its kernels.  Not part of the public ABI (include/e2f.h is).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace e2f {

constexpr int kMaxLmax = 2;
constexpr int kMaxPaths = 15;       // triangle-allowed (li, lf, lo) with all <= 2
constexpr int kWavesPerBlock = 4;   // 256-thread workgroups of the one-target-a-wave kernels
constexpr int kTile = 256;          // neighbour slots compacted per pass
// Up to this many atoms the kernels that share rows between several atoms of a
// wave launch too few waves to fill the chip (N/3 of them): one atom a wave is
// faster there (measured crossover on MI355X, 256 CUs: about 4,096 atoms at
// K = 256; at 1,024 atoms one a wave takes 0.044 ms against 0.147).
constexpr int64_t kMtMinAtoms = 4096;
constexpr int kXcds = 8;            // gfx950 (MI350 series): 8 XCDs, workgroups dealt round-robin
constexpr int kBboxBlocks = 256;    // partial bounding boxes reduced by the schedule builder
constexpr int kSchedMaxBits = 5;    // bits per axis of the schedule grid, at most
constexpr int kSchedCells = 1 << (3 * kSchedMaxBits);  // count entries always scanned

// Target schedule scratch, carved from the caller's workspace after the
// pre-coupled rows and the validation flag.
struct SchedScratch {
  int32_t* sched;      // [N] target order: atoms sorted by their cell's Hilbert index
  int32_t* cell;       // [N] cell of each atom
  int32_t* counts;     // [kSchedCells] per-cell counts, then running offsets
  float* partial;      // [kBboxBlocks][6] partial (min, max) of the positions
  int bits;            // grid bits per axis (<= kSchedMaxBits); cells used = 2^(3 bits)
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
  void* q_out;         // workspace mode: query rows [n, C] (a copy of the l = 0 row)
  int64_t n;
  int C;
  int lane_log;        // log2 of the lanes serving one atom (power of two <= 64)
};

struct AggArgs {
  const float* pos;        // [N, 3]
  const int32_t* idx;      // [N, K]
  const uint8_t* mask;     // [N, K]
  const void* ws;          // [N, S + 1, C]: row 0 = k, rows 1..S = h'
  const void* q;           // [N, C] query rows
  void* out;               // [N, S, C]
  void* out_msg;           // [N, S, C] or nullptr
  int64_t N;
  int K;
  int C;
  int lane_log;            // log2 of the lanes serving one neighbour row
  int head_lanes;          // lanes per head = d / V (power of two)
  float scale_log2e;       // logit scale times log2(e)
  const int32_t* sched;    // [N] processing order of the targets
  float* lse;              // [N, H] natural log-sum-exp of each target's logits, or nullptr
  int heads;               // H
  float env_inv_rc;        // 1 / r_env of the distance envelope (kernels with the envelope only)
  float env_rc;            // r_env itself
  int msg_f32;             // out_msg is fp32 whatever T is
  int shared;              // row-sharing kernels whatever N (else above kMtMinAtoms only)
  int tile;                // the 16-target matrix-core kernel whatever N, where it serves the layout
};

// Backward pass (vector-Jacobian product) arguments, fp32 storage.
struct BwdArgs {
  const float* pos;        // [N, 3]
  const float* h;          // [N, S, C] forward input
  const int32_t* idx;      // [N, K]
  const uint8_t* mask;     // [N, K]
  const float* ws;         // forward workspace rows [N, S + 1, C] (k, h')
  const float* msg;        // [N, S, C] forward message m
  const float* lse;        // [N, H] forward log-sum-exp
  const float* gout;       // [N, S, C] upstream gradient of out
  float* grad_h;           // [N, S, C]
  float* grad_pos;         // [N, 3]
  const float* q;          // [N, C] query rows (the forward workspace's)
  float* dk;               // [N, C] or NULL: dk_j stored apart, grad_h then holds dv_j only
  float* brows;            // [N, S + 1, C] scratch: row 0 = q_i, rows 1..S = dm_i
  float* dq;               // [N, C] scratch
  float* dh;               // [N, H] scratch: per-head <dm_i, m_i>
  const int32_t* rev_off;  // [N + 1] reverse list offsets (targets of each source)
  const int32_t* rev_idx;  // [E] reverse list entries
  const int32_t* sched;    // [N] visiting order
  int64_t N;
  int K;
  int C;
  int heads;
  int lane_log;
  int head_lanes;
  float scale;
  float scale_log2e;
  float env_inv_rc;        // 1 / r_env of the distance envelope, 0 = none
  float env_rc;            // r_env itself
  int shared;              // row-sharing kernels whatever N (else above kMtMinAtoms only)
};

// Row products of the projections' backward (fp32): values x W_V, or
// gradients x W^T (+ dq W_Q^T + dk W_K^T on the l = 0 row).
struct RowsArgs {
  const float* x;          // [n, S, C] h (values) or dv (gradients)
  const float* dq;         // [n, C] (gradients)
  const float* dk;         // [n, C] (gradients)
  const float* w_q;        // [C, C] fp32
  const float* w_k;        // [C, C] fp32
  const float* w_v;        // [lmax + 1, C, C] fp32
  void* out;               // [n, S, C]: fp32 values, or dL/dh in the storage type
  int64_t n;
};

// One weight gradient sum_r X_r^T dY_r over rows r = (atom r / mult, component
// r % mult): row r of X starts at x + (r / mult) xs + (r % mult) C.
struct DwJob {
  const float* x;
  const float* dy;
  int64_t xs, ys;          // atom strides (floats)
  int64_t rows;
  int64_t chunk_rows;      // rows per partial sum (a multiple of 4)
  int64_t part_off;        // first partial matrix of the job
  float* out;              // [C, C]
  int mult;
  int C;
  int chunks;
};
constexpr int kDwMaxJobs = kMaxLmax + 3;   // W_Q, W_K, W_V[0..lmax]
struct DwArgs {
  DwJob job[kDwMaxJobs];
  float* partial;          // [sum of chunks, C, C]
  int njobs;
  int C;
};
bool rows_mfma(int C);
int launch_value_rows(int lmax, int C, const RowsArgs& a, hipStream_t s);
int launch_grad_rows(int lmax, int C, int dtype, const RowsArgs& a, hipStream_t s);
int launch_weight_grads(const DwArgs& a, hipStream_t s);

// Learned projections fused with the pre-coupling (storage type T for h and
// the weights, row-major [C_in, C_out] matrices applied from the right).
struct ProjArgs {
  const float* r;          // [n, 3]
  const void* h;           // [n, S, C]
  const void* w_q;         // [C, C]
  const void* w_k;         // [C, C]
  const void* w_v;         // [lmax + 1, C, C]
  void* ws;                // workspace rows [n, S + 1, C]: k, then h' = (h W_V) (x) R(r)
  void* q_out;             // [n, C] query rows h[l=0] W_Q
  int64_t n;
};
constexpr int kProjTileAtoms = 16;  // atoms per MFMA row tile

// Dense real Clebsch-Gordan tensors of every path (lexicographic (li, lf, lo)),
// each [2li+1][2lf+1][2lo+1] row-major, path weights folded in: 615 entries
// at lmax = 2 (the O(L^6) contraction EAAS replaces).
constexpr int kDenseCoefs = 615;
struct DenseCoef {
  float c[kDenseCoefs];
};

// launchers (kernels file); return 0 or a hipError_t value
int launch_eaas(int lmax, int dtype, int V, bool to_workspace, const EaasArgs& a,
                const EaasCoef& cf, hipStream_t s);
int launch_aggregate(int lmax, int dtype, int V, const AggArgs& a, const EaasCoef& cf,
                     hipStream_t s);
// the 16-target matrix-core aggregate (its own file): fp32, C = 128, H = 16, rows of at most
// kTileMaxK slots, no envelope
constexpr int kTileMaxK = 256;
bool tile_supported(int lmax, int dtype, const AggArgs& a);
int launch_aggregate_tile(int lmax, const AggArgs& a, const EaasCoef& cf, hipStream_t s);
// the aggregate for any layout with C % H == 0 and C <= kGenericMaxC (its own file): one
// target a wave, lane l owning channels l + 64 k, per-head sums through LDS
constexpr int kGenericMaxC = 512;
int launch_aggregate_generic(int lmax, int dtype, const AggArgs& a, const EaasCoef& cf,
                             hipStream_t s);
// fused projection + pre-coupling: on the matrix cores for C in {16, 32, 64, 128} (fp32) or
// {32, 64, 128} (bf16), on the vector ALUs for any other C up to kProjMaxC
constexpr int kProjMaxC = 1024;
bool proj_supported(int C, int dtype);
int launch_proj(int lmax, int dtype, int C, const ProjArgs& a, const EaasCoef& cf, hipStream_t s);
int launch_frames(int lmax, int64_t n, const float* r, float* Q, float* D, hipStream_t s);
// the dense-CG product (dense file): EaasArgs without the workspace fields
int launch_dense(int lmax, int dtype, int V, const EaasArgs& a, const DenseCoef& cf,
                 hipStream_t s);
int launch_validate(int64_t N, int K, const int32_t* idx, const uint8_t* mask, int32_t* flag,
                    hipStream_t s);
int launch_schedule(int64_t N, const float* pos, const SchedScratch& sc, hipStream_t s);
// reverse neighbour list (CSR by source) and the three backward passes
int launch_reverse_list(int64_t N, int K, const int32_t* idx, const uint8_t* mask,
                        const int32_t* sched, int32_t* off, int32_t* cur, int32_t* tile_sums,
                        int32_t* entries, hipStream_t s);
constexpr int kRevMaxK = 2048;      // longest neighbour row the reverse-list build takes
int launch_backward(int lmax, int V, const BwdArgs& a, const EaasCoef& cf, hipStream_t s);
// exact bf16 -> fp32 widening and round-to-nearest-even fp32 -> bf16 narrowing of n elements
int launch_widen_bf16(int64_t n, const uint16_t* src, float* dst, hipStream_t s);
int launch_narrow_bf16(int64_t n, const float* src, uint16_t* dst, hipStream_t s);
constexpr int kScanTile = 4096;     // elements per block of the generic scan
// exclusive scan of a[0, n) in place (n <= kScanTile^2), a[n] = total, cur = copy of the
// scanned values; tile_sums holds kScanTile ints.  Returns the first launch error since the
// caller last cleared them.
int launch_scan_exclusive(int64_t n, int32_t* a, int32_t* tile_sums, int32_t* cur,
                          hipStream_t s);

// host file: E2F_OK, or E2F_ERR_RUNTIME while two HIP runtimes are mapped; and the status
// of a HIP error (recorded for e2f_last_hip_error)
int runtime_status();
int hip_error_status(int err);

// padded neighbour lists (cell list) and the Morton order of the atoms
constexpr int kNlMaxBits = 7;        // Morton bits per axis of the cell grid, at most
constexpr int kNlMaxK = 1984;        // longest row the builder keeps
struct NlArgs {
  const float* pos;        // [N, 3]
  int64_t N;
  int K;
  double rc;               // cutoff (strict)
  int bmax;                // Morton bits per axis allowed by the workspace
  int32_t* idx;            // [N, K] out
  uint8_t* mask;           // [N, K] out
  int32_t* n_within;       // [N] out or nullptr
  int32_t* order;          // [N] out or nullptr: atoms grouped by cell, Morton order
  // workspace parts
  float* partial;          // [kBboxBlocks, 6]
  void* grid;              // 256 bytes
  int32_t* cell;           // [N]
  int32_t* starts;         // [2^(3 bmax) + 1] counts, then exclusive starts
  int32_t* cursor;         // [2^(3 bmax)]
  int32_t* tile_sums;      // [kScanTile]
  int32_t* sorted_idx;     // [N]
  float* sorted_pos;       // [N, 4]
};
int launch_neighbours(const NlArgs& a, hipStream_t s);
constexpr int kRevTile = 1024;      // reverse-list entries sorted per pass

}  // namespace e2f
