// e2f_host.cpp -- host side of libe2f: argument checks, constant tables,
// lane-mapping choice and kernel dispatch for the entry points of e2f.h.
//
// The sparse reindex weights <li m lf 0 | lo m> come from Racah's closed
// formula for Clebsch-Gordan coefficients (Condon-Shortley phase), evaluated
// here in double precision; the write-up (stapisi.com, section 2.2) states
// the reindex rule, and section 5.2 warns that the CG normalisation matters.
#include <link.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <complex>
#include <mutex>

#include <hip/hip_runtime_api.h>

#include "../../include/e2f.h"
#include "e2f_internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;  // per calling thread; read by e2f_last_hip_error

// a launcher's return value (0 or a hipError_t) as a status code
int hip_status(int err) {
  if (err == 0) return E2F_OK;
  g_last_hip_error = err;
  return E2F_ERR_HIP;
}

// ---------------------------------------------------------------- runtime
// A process that maps two HIP runtimes (e.g. this library's libamdhip64.so.7
// loaded before a Python framework that ships its own copy) hands this library
// streams and device pointers that belong to the other runtime; launches then
// fail or crash.  Every entry point that would touch HIP first counts the
// runtimes mapped; the loader's add/remove counters make the recount rare.
struct RuntimeScan {
  unsigned long long adds, subs;  // loader counters at the last full scan
  bool valid;                     // a scan has been made
  int runtimes;                   // HIP runtime objects found then
  bool early;                     // set by the callback when the counters are unchanged
};
std::mutex g_rt_mutex;
RuntimeScan g_rt = {0, 0, false, 0, false};

int runtime_scan_cb(struct dl_phdr_info* info, size_t, void* data) {
  RuntimeScan* sc = static_cast<RuntimeScan*>(data);
  if (sc->valid && info->dlpi_adds == sc->adds && info->dlpi_subs == sc->subs) {
    sc->early = true;   // nothing loaded or unloaded since the last scan
    return 1;
  }
  if (sc->valid) sc->valid = false;   // first object of a full scan
  sc->adds = info->dlpi_adds;
  sc->subs = info->dlpi_subs;
  const char* name = info->dlpi_name ? info->dlpi_name : "";
  const char* base = strrchr(name, '/');
  base = base ? base + 1 : name;
  if (strncmp(base, "libamdhip64", 11) == 0) ++sc->runtimes;
  return 0;
}

// E2F_OK when at most one HIP runtime is mapped, E2F_ERR_RUNTIME otherwise
int check_runtime() {
  RuntimeScan sc;
  {
    std::lock_guard<std::mutex> lk(g_rt_mutex);
    sc = g_rt;
  }
  sc.early = false;
  const bool had = sc.valid;
  const int before = sc.runtimes;
  sc.runtimes = 0;
  dl_iterate_phdr(runtime_scan_cb, &sc);
  if (sc.early) {
    sc.runtimes = before;
    sc.valid = had;
  } else {
    sc.valid = true;
    std::lock_guard<std::mutex> lk(g_rt_mutex);
    g_rt = sc;
  }
  return sc.runtimes > 1 ? E2F_ERR_RUNTIME : E2F_OK;
}

using e2f::EaasCoef;
using e2f::kMaxPaths;

double factorial(int n) {
  double r = 1.0;
  for (int k = 2; k <= n; ++k) r *= k;
  return r;
}

// <j1 m1 j2 m2 | J M>, integer angular momenta, Racah's formula
double clebsch_gordan(int j1, int m1, int j2, int m2, int J, int M) {
  if (M != m1 + m2) return 0.0;
  if (J < abs(j1 - j2) || J > j1 + j2) return 0.0;
  if (abs(m1) > j1 || abs(m2) > j2 || abs(M) > J) return 0.0;
  const double tri = factorial(J + j1 - j2) * factorial(J - j1 + j2) * factorial(j1 + j2 - J) /
                     factorial(j1 + j2 + J + 1);
  const double pre = sqrt((2 * J + 1) * tri * factorial(J + M) * factorial(J - M) *
                          factorial(j1 - m1) * factorial(j1 + m1) * factorial(j2 - m2) *
                          factorial(j2 + m2));
  double sum = 0.0;
  for (int k = 0; k <= j1 + j2 + J; ++k) {
    const int a[6] = {k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k,
                      J - j1 - m2 + k};
    bool ok = true;
    double den = 1.0;
    for (int t = 0; t < 6; ++t) {
      if (a[t] < 0) { ok = false; break; }
      den *= factorial(a[t]);
    }
    if (ok) sum += ((k & 1) ? -1.0 : 1.0) / den;
  }
  return pre * sum;
}

int path_count(int lmax) {
  int p = 0;
  for (int li = 0; li <= lmax; ++li)
    for (int lf = 0; lf <= lmax; ++lf)
      for (int lo = 0; lo <= lmax; ++lo)
        if (lo >= abs(li - lf) && lo <= li + lf) ++p;
  return p;
}

EaasCoef make_coef(int lmax, const float* path_w) {
  EaasCoef cf;
  memset(&cf, 0, sizeof(cf));
  int p = 0;
  for (int li = 0; li <= lmax; ++li)
    for (int lf = 0; lf <= lmax; ++lf)
      for (int lo = 0; lo <= lmax; ++lo) {
        if (lo < abs(li - lf) || lo > li + lf) continue;
        const double w = path_w ? (double)path_w[p] : 1.0;
        const int mmax = li < lo ? li : lo;
        for (int m = 0; m <= mmax; ++m)
          cf.c[p][m] = (float)(w * clebsch_gordan(li, m, lf, 0, lo, m));
        ++p;
      }
  return cf;
}

// Real-basis coupling tensors for the dense product, from the Condon-Shortley
// coefficients above and the change of basis between real components x and
// spherical components T of degree l:
//   T_0 = x_0;  T_{+m} = (-1)^m (x_m + i x_{-m}) / sqrt2;  T_{-m} = (x_m - i x_{-m}) / sqrt2.
// The coupled spherical components sum_{m1 + m2 = M} <li m1 lf m2 | lo M> A_m1 B_m2,
// taken back to real components, give a tensor that is real when li + lf + lo is
// even and imaginary when it is odd; odd tensors are multiplied by -i.  Factor
// order: feature (li) first, harmonic (lf) second.
std::complex<double> real_to_sph(int l, int m_sph, int m_real) {
  const double s = 1.0 / sqrt(2.0);
  if (m_sph == 0) return m_real == 0 ? 1.0 : 0.0;
  const int m = abs(m_sph);
  const double sg = (m % 2) ? -1.0 : 1.0;
  (void)l;
  if (m_sph > 0) {
    if (m_real == m) return {sg * s, 0.0};
    if (m_real == -m) return {0.0, sg * s};
  } else {
    if (m_real == m) return {s, 0.0};
    if (m_real == -m) return {0.0, -s};
  }
  return 0.0;
}

double real_cg(int li, int lf, int lo, int a, int b, int c) {  // a, b, c real m values
  std::complex<double> acc = 0.0;
  for (int m1 = -li; m1 <= li; ++m1)
    for (int m2 = -lf; m2 <= lf; ++m2) {
      const int M = m1 + m2;
      if (abs(M) > lo) continue;
      const double cg = clebsch_gordan(li, m1, lf, m2, lo, M);
      if (cg == 0.0) continue;
      acc += std::conj(real_to_sph(lo, M, c)) * cg * real_to_sph(li, m1, a) *
             real_to_sph(lf, m2, b);
    }
  if ((li + lf + lo) % 2) acc *= std::complex<double>(0.0, -1.0);
  return acc.real();
}

e2f::DenseCoef make_dense_coef(int lmax, const float* path_w) {
  e2f::DenseCoef cf;
  memset(&cf, 0, sizeof(cf));
  int p = 0, off = 0;
  for (int li = 0; li <= lmax; ++li)
    for (int lf = 0; lf <= lmax; ++lf)
      for (int lo = 0; lo <= lmax; ++lo) {
        if (lo < abs(li - lf) || lo > li + lf) continue;
        const double w = path_w ? (double)path_w[p] : 1.0;
        for (int a = -li; a <= li; ++a)
          for (int b = -lf; b <= lf; ++b)
            for (int c = -lo; c <= lo; ++c) cf.c[off++] = (float)(w * real_cg(li, lf, lo, a, b, c));
        ++p;
      }
  return cf;
}

bool bad_dtype(int dt) { return dt != E2F_F32 && dt != E2F_BF16; }
size_t esize(int dt) { return dt == E2F_F32 ? 4 : 2; }
int ncomp(int lmax) { return (lmax + 1) * (lmax + 1); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ceil_log2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}
size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

struct Range {
  const void* p;
  size_t n;
};
bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// per-lane vector width for the element-wise EAAS kernel
int eaas_width(int C, int dt) {
  const int vmax = dt == E2F_F32 ? 4 : 8;
  for (int v = vmax; v > 1; v >>= 1)
    if (C % v == 0) return v;
  return 1;
}

// per-lane vector width for the attention stream: V | d, d / V a power of
// two (heads aligned to lanes), C / V <= 64 (one row per wave at most).
// 16-byte loads where possible: 4 fp32 channels or 8 bf16 channels per lane.
// bf16 with 8 channels keeps loaded rows packed (one 32-bit register per two
// channels), so one neighbour per subgroup in flight fits the registers.
int attn_width(int C, int H, int dt) {
  const int d = C / H;
  const int vmax = dt == E2F_BF16 ? 8 : 4;
  for (int v = vmax; v >= 1; v >>= 1)
    if (d % v == 0 && is_pow2(d / v) && C / v <= 64) return v;
  return 0;
}

// workspace: [rows [N, S + 1, C]: k, h'][query rows [N, C]][256 B validation flag]
//            [schedule scratch], every part 256-byte aligned
size_t ws_rows_bytes(int64_t N, int lmax, int C, int dt) {
  return round256((size_t)N * (size_t)(ncomp(lmax) + 1) * (size_t)C * esize(dt));
}

size_t ws_body_bytes(int64_t N, int lmax, int C, int dt) {
  return ws_rows_bytes(N, lmax, C, dt) + round256((size_t)N * (size_t)C * esize(dt));
}

void* ws_query_rows(void* ws, int64_t N, int lmax, int C, int dt) {
  return static_cast<char*>(ws) + ws_rows_bytes(N, lmax, C, dt);
}

// Up to this many atoms every gathered row stays in cache whatever the visiting
// order, and the four schedule launches would cost more than they save.
constexpr int64_t kSchedMinAtoms = 2048;

// bits per axis of the target schedule's grid: about one cell per atom, at most 2^15 cells
int sched_bits(int64_t N) {
  int bits = 1;
  while (bits < e2f::kSchedMaxBits && ((int64_t)1 << (3 * bits)) < N) ++bits;
  return bits;
}

size_t sched_bytes(int64_t N) {
  return 2 * round256((size_t)N * 4) + round256((size_t)e2f::kSchedCells * 4) +
         round256((size_t)e2f::kBboxBlocks * 6 * 4);
}

// backward workspace: [q / dm rows][dq][per-head D][reverse list offsets, cursors,
// scan tile sums, entries][schedule scratch]; every part 256-byte aligned
// With bf16 storage the backward widens h and G exactly into fp32 copies, recomputes the
// forward in fp32 from them (workspace, message, log-sum-exp) and differentiates that with
// the fp32 passes: [h][fp32 attention workspace][m][lse][G][dL/dh, narrowed at the end].
// Through the learned projections it also holds the recomputed value rows v, dv, dk, the
// weight-gradient partial sums and (bf16) fp32 copies of the weights.
struct BwdLayout {
  size_t brows, dq, dh, off, cur, tiles, entries, sched, cell, counts, partial;
  size_t h32, ws32, msg32, lse32, g32, gh32;   // bf16 storage only
  size_t v32, dv32, dk32, w32, wpart;          // projections only
  size_t total;
};

// Rows of the weight gradients' partial sums: chunks sized for about kDwWaves waves
// (chunk x output tile) over all jobs, at least kDwChunk rows, and at most 2^25 floats of
// partial matrices in all (wide channel counts take longer chunks).
constexpr int64_t kDwChunk = 512;
constexpr int64_t kDwWaves = 4096;
struct DwPlan {
  int njobs;
  int mult[e2f::kDwMaxJobs];
  int chunks[e2f::kDwMaxJobs];
  int64_t rows[e2f::kDwMaxJobs], chunk_rows[e2f::kDwMaxJobs], part_off[e2f::kDwMaxJobs];
  int64_t total;   // partial matrices
};

// jobs: 0 = W_Q, 1 = W_K, 2 + l = W_V[l]
DwPlan dw_plan(int64_t N, int lmax, int C) {
  DwPlan P;
  P.njobs = lmax + 3;
  P.total = 0;
  int64_t cap = ((int64_t)1 << 25) / ((int64_t)C * C) / P.njobs;
  if (cap < 1) cap = 1;
  const int64_t tpd = e2f::rows_mfma(C) ? (C < 64 ? 1 : C / 64) : (C + 15) / 16;
  const int64_t total_rows = N * (2 + (int64_t)(lmax + 1) * (lmax + 1));
  int64_t target = (total_rows * tpd * tpd + kDwWaves - 1) / kDwWaves;
  if (target < kDwChunk) target = kDwChunk;
  for (int j = 0; j < P.njobs; ++j) {
    P.mult[j] = j < 2 ? 1 : 2 * (j - 2) + 1;
    P.rows[j] = N * P.mult[j];
    int64_t chunks = (P.rows[j] + target - 1) / target;
    if (chunks > cap) chunks = cap;
    if (chunks < 1) chunks = 1;
    int64_t cr = (P.rows[j] + chunks - 1) / chunks;
    cr = (cr + 3) / 4 * 4;
    if (cr < 4) cr = 4;
    chunks = (P.rows[j] + cr - 1) / cr;
    if (chunks < 1) chunks = 1;
    P.chunk_rows[j] = cr;
    P.chunks[j] = (int)chunks;
    P.part_off[j] = P.total;
    P.total += chunks;
  }
  return P;
}

BwdLayout bwd_layout(int64_t N, int K, int lmax, int C, int H, int dt, bool proj) {
  BwdLayout L;
  size_t p = 0;
  auto take = [&p](size_t bytes) {
    const size_t at = p;
    p += round256(bytes);
    return at;
  };
  const size_t feat = (size_t)N * ncomp(lmax) * C * 4;
  const bool wide = dt == E2F_BF16;
  L.h32 = take(wide ? feat : 0);
  L.ws32 = take(wide ? e2f_attn_workspace_bytes(N, lmax, C, E2F_F32) : 0);
  L.msg32 = take(wide ? feat : 0);
  L.lse32 = take(wide ? (size_t)N * H * 4 : 0);
  L.g32 = take(wide ? feat : 0);
  L.gh32 = take(wide && !proj ? feat : 0);
  L.v32 = take(proj ? feat : 0);
  L.dv32 = take(proj ? feat : 0);
  L.dk32 = take(proj ? (size_t)N * C * 4 : 0);
  L.w32 = take(proj && wide ? (size_t)(lmax + 3) * C * C * 4 : 0);
  L.wpart = take(proj ? (size_t)dw_plan(N, lmax, C).total * C * C * 4 : 0);
  L.brows = take((size_t)N * (ncomp(lmax) + 1) * C * 4);
  L.dq = take((size_t)N * C * 4);
  L.dh = take((size_t)N * H * 4);
  L.off = take((size_t)(N + 1) * 4);
  L.cur = take((size_t)N * 4);
  L.tiles = take((size_t)e2f::kScanTile * 4);
  L.entries = take((size_t)N * K * 4);
  L.sched = take((size_t)N * 4);
  L.cell = take((size_t)N * 4);
  L.counts = take((size_t)e2f::kSchedCells * 4);
  L.partial = take((size_t)e2f::kBboxBlocks * 6 * 4);
  L.total = p;
  return L;
}

// neighbour-list builder workspace: [bbox partials][grid][cell per atom][cell starts]
// [fill cursors][scan tile sums][atoms grouped by cell][their positions, float4];
// every part 256-byte aligned.  The cell grid has at most 2^bits cells per axis,
// with 2^(3 bits) about the atom count (at least 2 per axis, at most 2^kNlMaxBits).
constexpr int64_t kNlMaxAtoms = (int64_t)1 << 30;
struct NlLayout {
  int bits;
  size_t partial, grid, cell, starts, cursor, tiles, sorted_idx, sorted_pos, total;
};

NlLayout nl_layout(int64_t N) {
  NlLayout L;
  L.bits = 1;
  while (L.bits < e2f::kNlMaxBits && ((int64_t)1 << (3 * L.bits)) < N) ++L.bits;
  const size_t cells = (size_t)1 << (3 * L.bits);
  size_t p = 0;
  auto take = [&p](size_t bytes) {
    const size_t at = p;
    p += round256(bytes);
    return at;
  };
  L.partial = take((size_t)e2f::kBboxBlocks * 6 * 4);
  L.grid = take(256);
  L.cell = take((size_t)N * 4);
  L.starts = take((cells + 1) * 4);
  L.cursor = take(cells * 4);
  L.tiles = take((size_t)e2f::kScanTile * 4);
  L.sorted_idx = take((size_t)N * 4);
  L.sorted_pos = take((size_t)N * 16);
  L.total = p;
  return L;
}

e2f::SchedScratch sched_scratch(void* ws, int64_t N, int lmax, int C, int dt) {
  char* p = static_cast<char*>(ws) + ws_body_bytes(N, lmax, C, dt) + 256;
  e2f::SchedScratch sc;
  sc.bits = sched_bits(N);
  sc.sched = reinterpret_cast<int32_t*>(p);
  p += round256((size_t)N * 4);
  sc.cell = reinterpret_cast<int32_t*>(p);
  p += round256((size_t)N * 4);
  sc.counts = reinterpret_cast<int32_t*>(p);
  p += round256((size_t)e2f::kSchedCells * 4);
  sc.partial = reinterpret_cast<float*>(p);
  return sc;
}

int check_shape_common(int64_t n, int lmax, int C, int dt) {
  if (bad_dtype(dt)) return E2F_ERR_DTYPE;
  if (n < 0 || lmax < 0 || lmax > e2f::kMaxLmax || C < 1) return E2F_ERR_SHAPE;
  return E2F_OK;
}

// envelope cutoff: 0 = no envelope, else a positive finite radius
bool bad_env(float env_cutoff) {
  return !(env_cutoff == 0.0f || (env_cutoff > 0.0f && isfinite(env_cutoff)));
}
float env_inv(float env_cutoff) {
  return env_cutoff > 0.0f ? (float)(1.0 / (double)env_cutoff) : 0.0f;
}

// attention forward: any C % H == 0 layout up to kGenericMaxC channels (layouts without a
// lane-vector width go to the generic kernel)
int check_attn_shape(int64_t N, int K, int lmax, int C, int H, int dt, uint32_t flags) {
  const int st = check_shape_common(N, lmax, C, dt);
  if (st != E2F_OK) return st;
  if (K < 1 || H < 1 || C % H != 0) return E2F_ERR_SHAPE;
  if (flags & ~(E2F_VALIDATE_INDICES | E2F_TARGETS_IN_ORDER | E2F_MSG_F32 | E2F_SHARED_ROWS |
                E2F_MATRIX_TILES))
    return E2F_ERR_SHAPE;
  if (attn_width(C, H, dt) == 0 && C > e2f::kGenericMaxC) return E2F_ERR_UNSUPPORTED;
  return E2F_OK;
}

// the backward's lane mapping: its passes run in fp32 (bf16 storage is widened first), so
// they need an fp32 per-lane vector width (see attn_width)
int check_bwd_shape(int64_t N, int K, int lmax, int C, int H, int dt, uint32_t flags) {
  const int st = check_attn_shape(N, K, lmax, C, H, dt, flags);
  if (st != E2F_OK) return st;
  return attn_width(C, H, E2F_F32) == 0 ? E2F_ERR_UNSUPPORTED : E2F_OK;
}

int precouple_impl(hipStream_t stream, int64_t N, int lmax, int C, int dt, const float* pos,
                   const void* h, const float* path_w, void* ws, size_t ws_bytes) {
  const int V = eaas_width(C, dt);
  e2f::EaasArgs a;
  a.r = pos;
  a.h_in = h;
  a.h_out = ws;
  a.q_out = ws_query_rows(ws, N, lmax, C, dt);
  a.n = N;
  a.C = C;
  const int lanes = (C + V - 1) / V;
  a.lane_log = ceil_log2(lanes > 64 ? 64 : lanes);
  const EaasCoef cf = make_coef(lmax, path_w);
  (void)ws_bytes;
  return hip_status(e2f::launch_eaas(lmax, dt, V, true, a, cf, stream));
}

int aggregate_impl(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dt,
                   const float* pos, const int32_t* idx, const uint8_t* mask, float scale,
                   float env_cutoff, const float* path_w, void* ws, void* out, void* out_msg,
                   float* lse, uint32_t flags) {
  if (flags & E2F_VALIDATE_INDICES) {
    int32_t* flag = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                               ws_body_bytes(N, lmax, C, dt));
    int st = hip_status(e2f::launch_validate(N, K, idx, mask, flag, stream));
    if (st != E2F_OK) return st;
    int32_t host_flag = 0;
    st = hip_status(
        hipMemcpyAsync(&host_flag, flag, sizeof(host_flag), hipMemcpyDeviceToHost, stream));
    if (st != E2F_OK) return st;
    st = hip_status(hipStreamSynchronize(stream));
    if (st != E2F_OK) return st;
    if (host_flag != 0) return E2F_ERR_INDEX;
  }
  const int V = attn_width(C, H, dt);   // 0: no lane-vector layout, the generic kernel
  const int d = C / H;
  const int32_t* sched = nullptr;
  if (!(flags & E2F_TARGETS_IN_ORDER) && N > kSchedMinAtoms) {
    const e2f::SchedScratch sc = sched_scratch(ws, N, lmax, C, dt);
    const int st = hip_status(e2f::launch_schedule(N, pos, sc, stream));
    if (st != E2F_OK) return st;
    sched = sc.sched;
  }
  e2f::AggArgs a;
  a.pos = pos;
  a.idx = idx;
  a.mask = mask;
  a.ws = ws;
  a.q = ws_query_rows(ws, N, lmax, C, dt);
  a.out = out;
  a.out_msg = out_msg;
  a.N = N;
  a.K = K;
  a.C = C;
  a.lane_log = V ? ceil_log2(C / V) : 6;
  a.head_lanes = V ? d / V : 0;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)d);
  a.scale_log2e = (float)(sc * 1.4426950408889634);  // log2(e)
  a.sched = sched;
  a.lse = lse;
  a.heads = H;
  a.env_inv_rc = env_inv(env_cutoff);
  a.env_rc = env_cutoff > 0.0f ? env_cutoff : 0.0f;
  a.msg_f32 = (flags & E2F_MSG_F32) ? 1 : 0;
  a.shared = (flags & E2F_SHARED_ROWS) ? 1 : 0;
  a.tile = (flags & E2F_MATRIX_TILES) ? 1 : 0;
  const EaasCoef cf = make_coef(lmax, path_w);
  if (V == 0) return hip_status(e2f::launch_aggregate_generic(lmax, dt, a, cf, stream));
  if (!a.shared && a.tile && e2f::tile_supported(lmax, dt, a))
    return hip_status(e2f::launch_aggregate_tile(lmax, a, cf, stream));
  return hip_status(e2f::launch_aggregate(lmax, dt, V, a, cf, stream));
}

}  // namespace

extern "C" {

const char* e2f_status_string(int status) {
  switch (status) {
    case E2F_OK: return "E2F_OK";
    case E2F_ERR_NULL: return "E2F_ERR_NULL";
    case E2F_ERR_SHAPE: return "E2F_ERR_SHAPE";
    case E2F_ERR_DTYPE: return "E2F_ERR_DTYPE";
    case E2F_ERR_ALIGN: return "E2F_ERR_ALIGN";
    case E2F_ERR_WORKSPACE: return "E2F_ERR_WORKSPACE";
    case E2F_ERR_ALIAS: return "E2F_ERR_ALIAS";
    case E2F_ERR_HIP: return "E2F_ERR_HIP";
    case E2F_ERR_INDEX: return "E2F_ERR_INDEX";
    case E2F_ERR_UNSUPPORTED: return "E2F_ERR_UNSUPPORTED";
    case E2F_ERR_RUNTIME: return "E2F_ERR_RUNTIME";
    default: return "E2F_ERR_UNKNOWN";
  }
}

int e2f_last_hip_error(void) { return g_last_hip_error; }

const char* e2f_last_hip_error_name(void) {
  return hipGetErrorName(static_cast<hipError_t>(g_last_hip_error));
}

int e2f_path_count(int lmax) {
  if (lmax < 0 || lmax > e2f::kMaxLmax) return E2F_ERR_SHAPE;
  return path_count(lmax);
}

int e2f_eaas_couple(hipStream_t stream, int64_t n, int lmax, int C, int dtype, const float* r,
                    const void* h_in, const float* path_w, void* h_out) {
  if (const int rt = check_runtime()) return rt;
  int st = check_shape_common(n, lmax, C, dtype);
  if (st != E2F_OK) return st;
  if (n == 0) return E2F_OK;
  if (!r || !h_in || !h_out) return E2F_ERR_NULL;
  if (!aligned(r, 4) || !aligned(h_in, 16) || !aligned(h_out, 16) ||
      (path_w && !aligned(path_w, 4)))
    return E2F_ERR_ALIGN;
  const size_t hb = (size_t)n * ncomp(lmax) * C * esize(dtype);
  if (h_out != h_in && overlap({h_out, hb}, {h_in, hb})) return E2F_ERR_ALIAS;
  if (overlap({h_out, hb}, {r, (size_t)n * 12})) return E2F_ERR_ALIAS;
  const int V = eaas_width(C, dtype);
  e2f::EaasArgs a;
  a.r = r;
  a.h_in = h_in;
  a.h_out = h_out;
  a.q_out = nullptr;
  a.n = n;
  a.C = C;
  const int lanes = (C + V - 1) / V;
  a.lane_log = ceil_log2(lanes > 64 ? 64 : lanes);
  const EaasCoef cf = make_coef(lmax, path_w);
  return hip_status(e2f::launch_eaas(lmax, dtype, V, false, a, cf, stream));
}

int e2f_dense_couple(hipStream_t stream, int64_t n, int lmax, int C, int dtype, const float* r,
                     const void* h_in, const float* path_w, void* h_out) {
  if (const int rt = check_runtime()) return rt;
  int st = check_shape_common(n, lmax, C, dtype);
  if (st != E2F_OK) return st;
  if (n == 0) return E2F_OK;
  if (!r || !h_in || !h_out) return E2F_ERR_NULL;
  if (!aligned(r, 4) || !aligned(h_in, 16) || !aligned(h_out, 16) ||
      (path_w && !aligned(path_w, 4)))
    return E2F_ERR_ALIGN;
  const size_t hb = (size_t)n * ncomp(lmax) * C * esize(dtype);
  if (h_out != h_in && overlap({h_out, hb}, {h_in, hb})) return E2F_ERR_ALIAS;
  if (overlap({h_out, hb}, {r, (size_t)n * 12})) return E2F_ERR_ALIAS;
  const int V = C % 4 == 0 ? 4 : 1;   // the widths the dense kernel is built for
  e2f::EaasArgs a;
  a.r = r;
  a.h_in = h_in;
  a.h_out = h_out;
  a.q_out = nullptr;
  a.n = n;
  a.C = C;
  const int lanes = (C + V - 1) / V;
  a.lane_log = ceil_log2(lanes > 64 ? 64 : lanes);
  const e2f::DenseCoef cf = make_dense_coef(lmax, path_w);
  return hip_status(e2f::launch_dense(lmax, dtype, V, a, cf, stream));
}

size_t e2f_attn_workspace_bytes(int64_t N, int lmax, int C, int dtype) {
  if (check_shape_common(N, lmax, C, dtype) != E2F_OK) return 0;
  return ws_body_bytes(N, lmax, C, dtype) + 256 + sched_bytes(N);
}

int e2f_attn_precouple(hipStream_t stream, int64_t N, int lmax, int C, int dtype,
                       const float* pos, const void* h, const float* path_w, void* workspace,
                       size_t ws_bytes) {
  if (const int rt = check_runtime()) return rt;
  int st = check_shape_common(N, lmax, C, dtype);
  if (st != E2F_OK) return st;
  if (N == 0) return E2F_OK;
  if (!pos || !h || !workspace) return E2F_ERR_NULL;
  if (!aligned(pos, 4) || !aligned(h, 16) || !aligned(workspace, 16) ||
      (path_w && !aligned(path_w, 4)))
    return E2F_ERR_ALIGN;
  const size_t need = e2f_attn_workspace_bytes(N, lmax, C, dtype);
  if (ws_bytes < need) return E2F_ERR_WORKSPACE;
  const size_t hb = (size_t)N * ncomp(lmax) * C * esize(dtype);
  if (overlap({workspace, need}, {h, hb}) || overlap({workspace, need}, {pos, (size_t)N * 12}))
    return E2F_ERR_ALIAS;
  return precouple_impl(stream, N, lmax, C, dtype, pos, h, path_w, workspace, ws_bytes);
}

int e2f_attn_aggregate(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                       const float* pos, const int32_t* nbr_idx, const uint8_t* nbr_mask,
                       float scale, float env_cutoff, const float* path_w, void* workspace,
                       size_t ws_bytes, void* out, void* out_msg, float* lse, uint32_t flags) {
  if (const int rt = check_runtime()) return rt;
  int st = check_attn_shape(N, K, lmax, C, H, dtype, flags);
  if (st != E2F_OK) return st;
  if (bad_env(env_cutoff)) return E2F_ERR_SHAPE;
  if (N == 0) return E2F_OK;
  if (!pos || !nbr_idx || !nbr_mask || !workspace || !out) return E2F_ERR_NULL;
  if (!aligned(pos, 4) || !aligned(nbr_idx, 4) || !aligned(workspace, 16) || !aligned(out, 16) ||
      (out_msg && !aligned(out_msg, 16)) || (path_w && !aligned(path_w, 4)) ||
      (lse && !aligned(lse, 4)))
    return E2F_ERR_ALIGN;
  const size_t need = e2f_attn_workspace_bytes(N, lmax, C, dtype);
  if (ws_bytes < need) return E2F_ERR_WORKSPACE;
  const size_t ob = (size_t)N * ncomp(lmax) * C * esize(dtype);
  const size_t mb = (flags & E2F_MSG_F32) ? (size_t)N * ncomp(lmax) * C * 4 : ob;
  const size_t lb = (size_t)N * H * 4;
  const Range ins[4] = {{pos, (size_t)N * 12},
                        {nbr_idx, (size_t)N * K * 4},
                        {nbr_mask, (size_t)N * K},
                        {workspace, need}};
  for (const Range& r : ins) {
    if (overlap({out, ob}, r)) return E2F_ERR_ALIAS;
    if (out_msg && overlap({out_msg, mb}, r)) return E2F_ERR_ALIAS;
    if (lse && overlap({lse, lb}, r)) return E2F_ERR_ALIAS;
  }
  if (out_msg && overlap({out, ob}, {out_msg, mb})) return E2F_ERR_ALIAS;
  if (lse && (overlap({lse, lb}, {out, ob}) || (out_msg && overlap({lse, lb}, {out_msg, mb}))))
    return E2F_ERR_ALIAS;
  return aggregate_impl(stream, N, K, lmax, C, H, dtype, pos, nbr_idx, nbr_mask, scale,
                        env_cutoff, path_w, workspace, out, out_msg, lse, flags);
}

}  // extern "C"

namespace {

// weights of the projected variants: present, aligned, a supported C, and
// clear of the workspace
int check_proj(int lmax, int C, int dtype, const void* w_q, const void* w_k, const void* w_v,
               const void* workspace, size_t need) {
  if (!w_q || !w_k || !w_v) return E2F_ERR_NULL;
  if (!aligned(w_q, 16) || !aligned(w_k, 16) || !aligned(w_v, 16)) return E2F_ERR_ALIGN;
  if (!e2f::proj_supported(C, dtype)) return E2F_ERR_UNSUPPORTED;
  const size_t wb = (size_t)C * C * esize(dtype);
  if (overlap({workspace, need}, {w_q, wb}) || overlap({workspace, need}, {w_k, wb}) ||
      overlap({workspace, need}, {w_v, (size_t)(lmax + 1) * wb}))
    return E2F_ERR_ALIAS;
  return E2F_OK;
}

int precouple_proj_impl(hipStream_t stream, int64_t N, int lmax, int C, int dt, const float* pos,
                        const void* h, const void* w_q, const void* w_k, const void* w_v,
                        const float* path_w, void* ws) {
  e2f::ProjArgs a;
  a.r = pos;
  a.h = h;
  a.w_q = w_q;
  a.w_k = w_k;
  a.w_v = w_v;
  a.ws = ws;
  a.q_out = ws_query_rows(ws, N, lmax, C, dt);
  a.n = N;
  const EaasCoef cf = make_coef(lmax, path_w);
  return hip_status(e2f::launch_proj(lmax, dt, C, a, cf, stream));
}

// e2f_attn_forward and e2f_attn_forward_proj (w_q == nullptr: no projections)
int forward_impl(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                 const float* pos, const void* h, const void* w_q, const void* w_k,
                 const void* w_v, const int32_t* nbr_idx, const uint8_t* nbr_mask, float scale,
                 float env_cutoff, const float* path_w, void* workspace, size_t ws_bytes,
                 void* out, void* out_msg, float* lse, uint32_t flags, bool proj) {
  if (const int rt = check_runtime()) return rt;
  int st = check_attn_shape(N, K, lmax, C, H, dtype, flags);
  if (st != E2F_OK) return st;
  if (bad_env(env_cutoff)) return E2F_ERR_SHAPE;
  if (N == 0) return E2F_OK;
  if (!h) return E2F_ERR_NULL;
  if (!aligned(h, 16)) return E2F_ERR_ALIGN;
  const size_t hb = (size_t)N * ncomp(lmax) * C * esize(dtype);
  const size_t mb = (flags & E2F_MSG_F32) ? (size_t)N * ncomp(lmax) * C * 4 : hb;
  if (overlap({out, hb}, {h, hb}) || (out_msg && overlap({out_msg, mb}, {h, hb})))
    return E2F_ERR_ALIAS;
  // all remaining checks (and the workspace / h overlap) happen in the two stages,
  // the aggregate's before anything is enqueued
  if (!pos || !nbr_idx || !nbr_mask || !workspace || !out) return E2F_ERR_NULL;
  const size_t need = e2f_attn_workspace_bytes(N, lmax, C, dtype);
  if (ws_bytes < need) return E2F_ERR_WORKSPACE;
  if (overlap({workspace, need}, {h, hb})) return E2F_ERR_ALIAS;
  if (!aligned(pos, 4) || !aligned(nbr_idx, 4) || !aligned(workspace, 16) || !aligned(out, 16) ||
      (out_msg && !aligned(out_msg, 16)) || (path_w && !aligned(path_w, 4)) ||
      (lse && !aligned(lse, 4)))
    return E2F_ERR_ALIGN;
  const size_t lb = (size_t)N * H * 4;
  const Range ins[5] = {{pos, (size_t)N * 12},
                        {nbr_idx, (size_t)N * K * 4},
                        {nbr_mask, (size_t)N * K},
                        {workspace, need},
                        {h, hb}};
  for (const Range& r : ins) {
    if (overlap({out, hb}, r)) return E2F_ERR_ALIAS;
    if (out_msg && overlap({out_msg, mb}, r)) return E2F_ERR_ALIAS;
    if (lse && overlap({lse, lb}, r)) return E2F_ERR_ALIAS;
  }
  if (out_msg && overlap({out, hb}, {out_msg, mb})) return E2F_ERR_ALIAS;
  if (lse && (overlap({lse, lb}, {out, hb}) || (out_msg && overlap({lse, lb}, {out_msg, mb}))))
    return E2F_ERR_ALIAS;
  if (overlap({workspace, need}, {pos, (size_t)N * 12})) return E2F_ERR_ALIAS;
  if (proj) {
    st = check_proj(lmax, C, dtype, w_q, w_k, w_v, workspace, need);
    if (st != E2F_OK) return st;
    st = precouple_proj_impl(stream, N, lmax, C, dtype, pos, h, w_q, w_k, w_v, path_w,
                             workspace);
  } else {
    st = precouple_impl(stream, N, lmax, C, dtype, pos, h, path_w, workspace, ws_bytes);
  }
  if (st != E2F_OK) return st;
  return aggregate_impl(stream, N, K, lmax, C, H, dtype, pos, nbr_idx, nbr_mask, scale,
                        env_cutoff, path_w, workspace, out, out_msg, lse, flags);
}

}  // namespace

namespace e2f {

int runtime_status() { return check_runtime(); }

int hip_error_status(int err) { return hip_status(err); }

}  // namespace e2f

extern "C" {

int e2f_attn_forward(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                     const float* pos, const void* h, const int32_t* nbr_idx,
                     const uint8_t* nbr_mask, float scale, float env_cutoff,
                     const float* path_w, void* workspace, size_t ws_bytes, void* out,
                     void* out_msg, float* lse, uint32_t flags) {
  return forward_impl(stream, N, K, lmax, C, H, dtype, pos, h, nullptr, nullptr, nullptr,
                      nbr_idx, nbr_mask, scale, env_cutoff, path_w, workspace, ws_bytes, out,
                      out_msg, lse, flags, false);
}

int e2f_attn_forward_proj(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                          const float* pos, const void* h, const void* w_q, const void* w_k,
                          const void* w_v, const int32_t* nbr_idx, const uint8_t* nbr_mask,
                          float scale, float env_cutoff, const float* path_w, void* workspace,
                          size_t ws_bytes, void* out, void* out_msg, float* lse, uint32_t flags) {
  return forward_impl(stream, N, K, lmax, C, H, dtype, pos, h, w_q, w_k, w_v, nbr_idx, nbr_mask,
                      scale, env_cutoff, path_w, workspace, ws_bytes, out, out_msg, lse, flags,
                      true);
}

int e2f_attn_precouple_proj(hipStream_t stream, int64_t N, int lmax, int C, int dtype,
                            const float* pos, const void* h, const void* w_q, const void* w_k,
                            const void* w_v, const float* path_w, void* workspace,
                            size_t ws_bytes) {
  if (const int rt = check_runtime()) return rt;
  int st = check_shape_common(N, lmax, C, dtype);
  if (st != E2F_OK) return st;
  if (N == 0) return E2F_OK;
  if (!pos || !h || !workspace) return E2F_ERR_NULL;
  if (!aligned(pos, 4) || !aligned(h, 16) || !aligned(workspace, 16) ||
      (path_w && !aligned(path_w, 4)))
    return E2F_ERR_ALIGN;
  const size_t need = e2f_attn_workspace_bytes(N, lmax, C, dtype);
  if (ws_bytes < need) return E2F_ERR_WORKSPACE;
  const size_t hb = (size_t)N * ncomp(lmax) * C * esize(dtype);
  if (overlap({workspace, need}, {h, hb}) || overlap({workspace, need}, {pos, (size_t)N * 12}))
    return E2F_ERR_ALIAS;
  st = check_proj(lmax, C, dtype, w_q, w_k, w_v, workspace, need);
  if (st != E2F_OK) return st;
  return precouple_proj_impl(stream, N, lmax, C, dtype, pos, h, w_q, w_k, w_v, path_w,
                             workspace);
}

size_t e2f_attn_backward_workspace_bytes(int64_t N, int K, int lmax, int C, int H, int dtype) {
  if (check_bwd_shape(N, K, lmax, C, H, dtype, 0) != E2F_OK) return 0;
  return bwd_layout(N, K, lmax, C, H, dtype, false).total;
}

size_t e2f_attn_backward_proj_workspace_bytes(int64_t N, int K, int lmax, int C, int H,
                                              int dtype) {
  if (check_bwd_shape(N, K, lmax, C, H, dtype, 0) != E2F_OK) return 0;
  if (!e2f::proj_supported(C, dtype)) return 0;
  return bwd_layout(N, K, lmax, C, H, dtype, true).total;
}

}  // extern "C"

namespace {

// e2f_attn_backward and e2f_attn_backward_proj (proj: through the learned projections)
int backward_impl(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                  const float* pos, const void* h, const void* w_q, const void* w_k,
                  const void* w_v, const int32_t* nbr_idx, const uint8_t* nbr_mask, float scale,
                  float env_cutoff, const float* path_w, const void* workspace, size_t ws_bytes,
                  const void* msg, const float* lse, const void* grad_out, void* grad_h,
                  float* grad_pos, float* grad_w_q, float* grad_w_k, float* grad_w_v,
                  void* bwd_workspace, size_t bwd_ws_bytes, uint32_t flags, bool proj) {
  if (const int rt = check_runtime()) return rt;
  int st = check_bwd_shape(N, K, lmax, C, H, dtype, flags);
  if (st != E2F_OK) return st;
  if (bad_env(env_cutoff)) return E2F_ERR_SHAPE;
  if (flags & (E2F_VALIDATE_INDICES | E2F_MSG_F32)) return E2F_ERR_SHAPE;  // forward-only flags
  if (proj && !e2f::proj_supported(C, dtype)) return E2F_ERR_UNSUPPORTED;
  if (N == 0) return E2F_OK;
  if (N > (int64_t)e2f::kScanTile * e2f::kScanTile || N * (int64_t)K >= ((int64_t)1 << 31) ||
      K > e2f::kRevMaxK)
    return E2F_ERR_UNSUPPORTED;
  const bool recompute = dtype == E2F_BF16;   // msg and lse are recomputed in fp32 (may be NULL)
  if (!pos || !h || !nbr_idx || !nbr_mask || !workspace || (!recompute && (!msg || !lse)) ||
      !grad_out || !grad_h || !grad_pos || !bwd_workspace)
    return E2F_ERR_NULL;
  if (proj && (!w_q || !w_k || !w_v || !grad_w_q || !grad_w_k || !grad_w_v)) return E2F_ERR_NULL;
  if (!aligned(pos, 4) || !aligned(h, 16) || !aligned(nbr_idx, 4) || !aligned(workspace, 16) ||
      (msg && !aligned(msg, 16)) || (lse && !aligned(lse, 4)) || !aligned(grad_out, 16) ||
      !aligned(grad_h, 16) ||
      !aligned(grad_pos, 4) || !aligned(bwd_workspace, 16) || (path_w && !aligned(path_w, 4)))
    return E2F_ERR_ALIGN;
  if (proj && (!aligned(w_q, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) ||
               !aligned(grad_w_q, 4) || !aligned(grad_w_k, 4) || !aligned(grad_w_v, 4)))
    return E2F_ERR_ALIGN;
  const size_t need = e2f_attn_workspace_bytes(N, lmax, C, dtype);
  if (ws_bytes < need) return E2F_ERR_WORKSPACE;
  const BwdLayout L = bwd_layout(N, K, lmax, C, H, dtype, proj);
  if (bwd_ws_bytes < L.total) return E2F_ERR_WORKSPACE;
  const size_t hb = (size_t)N * ncomp(lmax) * C * esize(dtype);
  const size_t mb = recompute ? 0 : hb;   // unused with bf16 storage
  const size_t wb = proj ? (size_t)C * C * esize(dtype) : 0;
  const size_t gwb = proj ? (size_t)C * C * 4 : 0;
  const Range ins[11] = {{pos, (size_t)N * 12}, {h, hb},       {nbr_idx, (size_t)N * K * 4},
                         {nbr_mask, (size_t)N * K}, {workspace, need}, {msg, mb},
                         {lse, (size_t)N * H * 4}, {grad_out, hb}, {w_q, wb}, {w_k, wb},
                         {w_v, (size_t)(lmax + 1) * wb}};
  const Range outs[6] = {{grad_h, hb},        {grad_pos, (size_t)N * 12},
                         {bwd_workspace, L.total}, {grad_w_q, gwb},
                         {grad_w_k, gwb},     {grad_w_v, (size_t)(lmax + 1) * gwb}};
  for (const Range& o : outs)
    for (const Range& r : ins)
      if (overlap(o, r)) return E2F_ERR_ALIAS;
  for (int x = 0; x < 6; ++x)
    for (int y = x + 1; y < 6; ++y)
      if (overlap(outs[x], outs[y])) return E2F_ERR_ALIAS;

  char* b = static_cast<char*>(bwd_workspace);
  e2f::BwdArgs a;
  a.pos = pos;
  a.h = static_cast<const float*>(h);
  a.idx = nbr_idx;
  a.mask = nbr_mask;
  a.ws = static_cast<const float*>(workspace);
  a.q = static_cast<const float*>(ws_query_rows(const_cast<void*>(workspace), N, lmax, C, dtype));
  a.dk = nullptr;
  a.msg = static_cast<const float*>(msg);
  a.lse = lse;
  a.gout = static_cast<const float*>(grad_out);
  a.grad_h = static_cast<float*>(grad_h);
  a.grad_pos = grad_pos;
  const bool wide = dtype == E2F_BF16;
  const int64_t n_feat = N * (int64_t)ncomp(lmax) * C;
  const int64_t cc = (int64_t)C * C;
  // fp32 weights (the caller's, or exact copies of the bf16 ones)
  const float* wq32 = static_cast<const float*>(w_q);
  const float* wk32 = static_cast<const float*>(w_k);
  const float* wv32 = static_cast<const float*>(w_v);
  float* dv32 = proj ? reinterpret_cast<float*>(b + L.dv32) : nullptr;
  if (wide) {
    // exact fp32 copies of h and G, and the forward recomputed from them in fp32: the
    // gradients of the layer at the bf16 inputs, without the rounding of the stored
    // workspace and message (the softmax backward's <dm_i, h'_j> - <dm_i, m_i> cancels)
    float* h32 = reinterpret_cast<float*>(b + L.h32);
    void* ws32 = b + L.ws32;
    float* msg32 = reinterpret_cast<float*>(b + L.msg32);
    float* lse32 = reinterpret_cast<float*>(b + L.lse32);
    float* g32 = reinterpret_cast<float*>(b + L.g32);
    // the aggregate's out is scratch here: the buffer it lands in is overwritten later
    float* out32 = proj ? dv32 : reinterpret_cast<float*>(b + L.gh32);
    st = hip_status(e2f::launch_widen_bf16(n_feat, static_cast<const uint16_t*>(h), h32, stream));
    if (st == E2F_OK)
      st = hip_status(
          e2f::launch_widen_bf16(n_feat, static_cast<const uint16_t*>(grad_out), g32, stream));
    const size_t ws32_bytes = e2f_attn_workspace_bytes(N, lmax, C, E2F_F32);
    if (proj) {
      float* w32 = reinterpret_cast<float*>(b + L.w32);
      if (st == E2F_OK)
        st = hip_status(e2f::launch_widen_bf16(cc, static_cast<const uint16_t*>(w_q), w32, stream));
      if (st == E2F_OK)
        st = hip_status(
            e2f::launch_widen_bf16(cc, static_cast<const uint16_t*>(w_k), w32 + cc, stream));
      if (st == E2F_OK)
        st = hip_status(e2f::launch_widen_bf16((lmax + 1) * cc,
                                               static_cast<const uint16_t*>(w_v), w32 + 2 * cc,
                                               stream));
      wq32 = w32;
      wk32 = w32 + cc;
      wv32 = w32 + 2 * cc;
      if (st == E2F_OK)
        st = precouple_proj_impl(stream, N, lmax, C, E2F_F32, pos, h32, wq32, wk32, wv32, path_w,
                                 ws32);
    } else if (st == E2F_OK) {
      st = precouple_impl(stream, N, lmax, C, E2F_F32, pos, h32, path_w, ws32, ws32_bytes);
    }
    if (st == E2F_OK)
      st = aggregate_impl(stream, N, K, lmax, C, H, E2F_F32, pos, nbr_idx, nbr_mask, scale,
                          env_cutoff, path_w, ws32, out32, msg32, lse32,
                          flags & (E2F_TARGETS_IN_ORDER | E2F_SHARED_ROWS | E2F_MATRIX_TILES));
    if (st != E2F_OK) return st;
    a.h = h32;
    a.ws = static_cast<const float*>(ws32);
    a.q = static_cast<const float*>(ws_query_rows(ws32, N, lmax, C, E2F_F32));
    a.msg = msg32;
    a.lse = lse32;
    a.gout = g32;
    a.grad_h = out32;
  }
  const float* h_in = a.h;   // fp32 h: the caller's, or its exact copy
  if (proj) {
    // the passes differentiate the pre-coupling of v = h W_V: recompute v, take dv and
    // dk apart, and finish through the projections afterwards
    float* v32 = reinterpret_cast<float*>(b + L.v32);
    e2f::RowsArgs r;
    r.x = h_in;
    r.dq = nullptr;
    r.dk = nullptr;
    r.w_q = wq32;
    r.w_k = wk32;
    r.w_v = wv32;
    r.out = v32;
    r.n = N;
    st = hip_status(e2f::launch_value_rows(lmax, C, r, stream));
    if (st != E2F_OK) return st;
    a.h = v32;
    a.dk = reinterpret_cast<float*>(b + L.dk32);
    a.grad_h = dv32;
  }
  a.brows = reinterpret_cast<float*>(b + L.brows);
  a.dq = reinterpret_cast<float*>(b + L.dq);
  a.dh = reinterpret_cast<float*>(b + L.dh);
  int32_t* off = reinterpret_cast<int32_t*>(b + L.off);
  int32_t* cur = reinterpret_cast<int32_t*>(b + L.cur);
  int32_t* tiles = reinterpret_cast<int32_t*>(b + L.tiles);
  int32_t* entries = reinterpret_cast<int32_t*>(b + L.entries);
  a.rev_off = off;
  a.rev_idx = entries;
  a.sched = nullptr;
  if (!(flags & E2F_TARGETS_IN_ORDER) && N > kSchedMinAtoms) {
    e2f::SchedScratch sc;
    sc.bits = sched_bits(N);
    sc.sched = reinterpret_cast<int32_t*>(b + L.sched);
    sc.cell = reinterpret_cast<int32_t*>(b + L.cell);
    sc.counts = reinterpret_cast<int32_t*>(b + L.counts);
    sc.partial = reinterpret_cast<float*>(b + L.partial);
    st = hip_status(e2f::launch_schedule(N, pos, sc, stream));
    if (st != E2F_OK) return st;
    a.sched = sc.sched;
  }
  st = hip_status(e2f::launch_reverse_list(N, K, nbr_idx, nbr_mask, a.sched, off, cur, tiles,
                                           entries, stream));
  if (st != E2F_OK) return st;
  const int V = attn_width(C, H, E2F_F32);   // the fp32 passes' lane mapping
  const int d = C / H;
  a.N = N;
  a.K = K;
  a.C = C;
  a.heads = H;
  a.lane_log = ceil_log2(C / V);
  a.head_lanes = d / V;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)d);
  a.scale = (float)sc;
  a.scale_log2e = (float)(sc * 1.4426950408889634);
  a.env_inv_rc = env_inv(env_cutoff);
  a.env_rc = env_cutoff > 0.0f ? env_cutoff : 0.0f;
  a.shared = (flags & E2F_SHARED_ROWS) ? 1 : 0;
  const EaasCoef cf = make_coef(lmax, path_w);
  st = hip_status(e2f::launch_backward(lmax, V, a, cf, stream));
  if (st != E2F_OK) return st;
  if (!proj) {
    if (!wide) return E2F_OK;
    return hip_status(e2f::launch_narrow_bf16(n_feat, a.grad_h, static_cast<uint16_t*>(grad_h),
                                              stream));
  }
  // dL/dh through the projections, in the storage type
  e2f::RowsArgs r;
  r.x = dv32;
  r.dq = a.dq;
  r.dk = a.dk;
  r.w_q = wq32;
  r.w_k = wk32;
  r.w_v = wv32;
  r.out = grad_h;
  r.n = N;
  st = hip_status(e2f::launch_grad_rows(lmax, C, dtype, r, stream));
  if (st != E2F_OK) return st;
  // weight gradients: X = h rows, dY = dq, dk, dv rows
  const DwPlan P = dw_plan(N, lmax, C);
  e2f::DwArgs w;
  w.partial = reinterpret_cast<float*>(b + L.wpart);
  w.njobs = P.njobs;
  w.C = C;
  const int64_t row = (int64_t)ncomp(lmax) * C;
  for (int j = 0; j < P.njobs; ++j) {
    e2f::DwJob& J = w.job[j];
    const int l = j - 2;
    J.x = j < 2 ? h_in : h_in + (int64_t)l * l * C;
    J.xs = row;
    J.dy = j == 0 ? a.dq : (j == 1 ? a.dk : dv32 + (int64_t)l * l * C);
    J.ys = j < 2 ? C : row;
    J.rows = P.rows[j];
    J.chunk_rows = P.chunk_rows[j];
    J.part_off = P.part_off[j];
    J.out = j == 0 ? grad_w_q : (j == 1 ? grad_w_k : grad_w_v + (int64_t)l * cc);
    J.mult = P.mult[j];
    J.C = C;
    J.chunks = P.chunks[j];
  }
  return hip_status(e2f::launch_weight_grads(w, stream));
}

}  // namespace

extern "C" {

int e2f_attn_backward(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                      const float* pos, const void* h, const int32_t* nbr_idx,
                      const uint8_t* nbr_mask, float scale, float env_cutoff,
                      const float* path_w, const void* workspace, size_t ws_bytes,
                      const void* msg, const float* lse, const void* grad_out, void* grad_h,
                      float* grad_pos, void* bwd_workspace, size_t bwd_ws_bytes,
                      uint32_t flags) {
  return backward_impl(stream, N, K, lmax, C, H, dtype, pos, h, nullptr, nullptr, nullptr,
                       nbr_idx, nbr_mask, scale, env_cutoff, path_w, workspace, ws_bytes, msg,
                       lse, grad_out, grad_h, grad_pos, nullptr, nullptr, nullptr, bwd_workspace,
                       bwd_ws_bytes, flags, false);
}

int e2f_attn_backward_proj(hipStream_t stream, int64_t N, int K, int lmax, int C, int H,
                           int dtype, const float* pos, const void* h, const void* w_q,
                           const void* w_k, const void* w_v, const int32_t* nbr_idx,
                           const uint8_t* nbr_mask, float scale, float env_cutoff,
                           const float* path_w, const void* workspace, size_t ws_bytes,
                           const void* msg, const float* lse, const void* grad_out, void* grad_h,
                           float* grad_pos, float* grad_w_q, float* grad_w_k, float* grad_w_v,
                           void* bwd_workspace, size_t bwd_ws_bytes, uint32_t flags) {
  return backward_impl(stream, N, K, lmax, C, H, dtype, pos, h, w_q, w_k, w_v, nbr_idx, nbr_mask,
                       scale, env_cutoff, path_w, workspace, ws_bytes, msg, lse, grad_out, grad_h,
                       grad_pos, grad_w_q, grad_w_k, grad_w_v, bwd_workspace, bwd_ws_bytes, flags,
                       true);
}

size_t e2f_neighbour_workspace_bytes(int64_t N) {
  if (N < 0 || N > kNlMaxAtoms) return 0;
  return nl_layout(N).total;
}

int e2f_neighbour_list(hipStream_t stream, int64_t N, int K, double cutoff, const float* pos,
                       int32_t* nbr_idx, uint8_t* nbr_mask, int32_t* n_within, int32_t* order,
                       void* workspace, size_t ws_bytes) {
  if (const int rt = check_runtime()) return rt;
  if (N < 0 || K < 1 || !(cutoff > 0.0) || !isfinite(cutoff)) return E2F_ERR_SHAPE;
  if (N > kNlMaxAtoms || K > e2f::kNlMaxK) return E2F_ERR_UNSUPPORTED;
  if (N == 0) return E2F_OK;
  if (!pos || !nbr_idx || !nbr_mask || !workspace) return E2F_ERR_NULL;
  if (!aligned(pos, 4) || !aligned(nbr_idx, 4) || !aligned(workspace, 16) ||
      (n_within && !aligned(n_within, 4)) || (order && !aligned(order, 4)))
    return E2F_ERR_ALIGN;
  const NlLayout L = nl_layout(N);
  if (ws_bytes < L.total) return E2F_ERR_WORKSPACE;
  const Range outs[5] = {{nbr_idx, (size_t)N * K * 4},
                         {nbr_mask, (size_t)N * K},
                         {n_within, (size_t)N * 4},
                         {order, (size_t)N * 4},
                         {workspace, L.total}};
  const Range in = {pos, (size_t)N * 12};
  for (int a = 0; a < 5; ++a) {
    if (overlap(outs[a], in)) return E2F_ERR_ALIAS;
    for (int b = a + 1; b < 5; ++b)
      if (overlap(outs[a], outs[b])) return E2F_ERR_ALIAS;
  }
  char* w = static_cast<char*>(workspace);
  e2f::NlArgs a;
  a.pos = pos;
  a.N = N;
  a.K = K;
  a.rc = cutoff;
  a.bmax = L.bits;
  a.idx = nbr_idx;
  a.mask = nbr_mask;
  a.n_within = n_within;
  a.order = order;
  a.partial = reinterpret_cast<float*>(w + L.partial);
  a.grid = w + L.grid;
  a.cell = reinterpret_cast<int32_t*>(w + L.cell);
  a.starts = reinterpret_cast<int32_t*>(w + L.starts);
  a.cursor = reinterpret_cast<int32_t*>(w + L.cursor);
  a.tile_sums = reinterpret_cast<int32_t*>(w + L.tiles);
  a.sorted_idx = reinterpret_cast<int32_t*>(w + L.sorted_idx);
  a.sorted_pos = reinterpret_cast<float*>(w + L.sorted_pos);
  return hip_status(e2f::launch_neighbours(a, stream));
}

int e2f_frames(hipStream_t stream, int64_t n, int lmax, const float* r, float* Q, float* D) {
  if (const int rt = check_runtime()) return rt;
  if (n < 0 || lmax < 0 || lmax > e2f::kMaxLmax) return E2F_ERR_SHAPE;
  if (n == 0) return E2F_OK;
  if (!r || !Q || !D) return E2F_ERR_NULL;
  if (!aligned(r, 4) || !aligned(Q, 4) || !aligned(D, 4)) return E2F_ERR_ALIGN;
  if (overlap({Q, (size_t)n * 36}, {r, (size_t)n * 12}) ||
      overlap({D, (size_t)n * 140}, {r, (size_t)n * 12}) ||
      overlap({Q, (size_t)n * 36}, {D, (size_t)n * 140}))
    return E2F_ERR_ALIAS;
  return hip_status(e2f::launch_frames(lmax, n, r, Q, D, stream));
}

}  // extern "C"
