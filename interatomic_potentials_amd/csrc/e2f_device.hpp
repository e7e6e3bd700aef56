// e2f_device.hpp -- device-side building blocks of the EAAS tensor product
// and the fused attention stream for gfx950 (wave64).
//
// EAAS (E2Former-V2 write-up on stapisi.com, section 2; Proposition 4.3):
// for a vector r with polar angle t and azimuth p, the alignment rotation
// Q = R_y(-t) R_z(-p) maps r_hat to z_hat.  The Wigner-D matrix of Q in the
// real harmonic basis factorises the same way, D(Q) = D_y(-t) D_z(-p), and
// both factors are sparse:
//   * D_z(a) rotates each (m, -m) pair by the angle m a;
//   * D_y(b) keeps the m < 0 and the m >= 0 components apart (a rotation
//     about y preserves parity in y): a 1x1 + 2x2 block at l = 1 and a
//     2x2 + 3x3 block at l = 2.
// The l = 2 entries below were derived by substituting the rotated
// coordinates into the l = 2 real solid harmonics
//   (sqrt3 xy, sqrt3 yz, (3z^2 - r^2)/2, sqrt3 xz, sqrt3/2 (x^2 - y^2))
// and re-expanding; with c = cos b, s = sin b the m >= 0 block is
//   [ (3c^2-1)/2     -sqrt3 s c     sqrt3/2 s^2 ]
//   [  sqrt3 s c      c^2 - s^2    -s c         ]
//   [  sqrt3/2 s^2    s c          (1 + c^2)/2  ]
// and the m < 0 block is [[c, s], [-s, c]].  In the aligned frame the
// harmonics are |r|^lf at m_f = 0 only (Lemma 4.1 of the gist.science
// summary, section 2.1), so the product reduces to the sparse reindex of
// write-up section 2.2; its weights <li m lf 0 | lo m> arrive from the host.
// All angles are handled through cosines and sines built from the
// coordinates; no trigonometric function is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e2f_internal.hpp"

namespace e2f {

__host__ __device__ constexpr int ncomp(int lmax) { return (lmax + 1) * (lmax + 1); }
__host__ __device__ constexpr int flat(int l, int m) { return l * l + l + m; }

// ---------------------------------------------------------------- frame

struct Frame {
  float ct, st;   // cos, sin of the polar angle
  float c1, s1;   // cos, sin of the azimuth
  float c2, s2;   // cos, sin of twice the azimuth
  float r1, r2;   // |r|, |r|^2
};

__device__ inline Frame make_frame(float x, float y, float z) {
  // Angles come from components scaled by the largest magnitude, so that
  // squares of tiny components cannot lose precision in the denormal range
  // (that would leave Q measurably non-orthogonal).
  Frame f;
  const float ax = fabsf(x), ay = fabsf(y), az = fabsf(z);
  const float mxy = fmaxf(ax, ay);
  const float m = fmaxf(mxy, az);
  if (m > 0.0f) {
    const float im = 1.0f / m;
    const float xs = x * im, ys = y * im, zs = z * im;
    const float rs = sqrtf(xs * xs + ys * ys + zs * zs);   // in [1, sqrt 3]
    const float rhos = sqrtf(xs * xs + ys * ys);
    const float irs = 1.0f / rs;
    f.ct = zs * irs;
    f.st = rhos * irs;
    f.r1 = m * rs;
  } else {  // r = 0: Q = identity; only lf = 0 paths survive since |r|^lf = 0
    f.ct = 1.0f;
    f.st = 0.0f;
    f.r1 = 0.0f;
  }
  if (mxy > 0.0f) {
    const float im = 1.0f / mxy;
    const float xs = x * im, ys = y * im;
    const float irho = 1.0f / sqrtf(xs * xs + ys * ys);
    f.c1 = xs * irho;
    f.s1 = ys * irho;
  } else {  // on the z axis the azimuth is free; take 0
    f.c1 = 1.0f;
    f.s1 = 0.0f;
  }
  f.c2 = f.c1 * f.c1 - f.s1 * f.s1;
  f.s2 = 2.0f * f.s1 * f.c1;
  f.r2 = f.r1 * f.r1;
  return f;
}

// entries of the l = 2, m >= 0 block of D_y(+t) (see the header comment)
struct Dy2 {
  float d00, d01, d02, d11, d12, d22;
};

__device__ inline Dy2 make_dy2(const Frame& f) {
  const float k3 = 1.7320508075688772f;  // sqrt(3)
  Dy2 d;
  const float cc = f.ct * f.ct, ss = f.st * f.st, sc = f.st * f.ct;
  d.d00 = 0.5f * (3.0f * cc - 1.0f);
  d.d01 = k3 * sc;
  d.d02 = 0.5f * k3 * ss;
  d.d11 = cc - ss;
  d.d12 = sc;
  d.d22 = 0.5f * (1.0f + cc);
  return d;
}

// x <- D(Q) x = D_y(-t) D_z(-p) x   (global frame -> aligned frame)
template <int LMAX>
__device__ inline void rotate_in(float* x, const Frame& f, const Dy2& d) {
  if constexpr (LMAX >= 1) {
    // D_z(-p) on the (m=1, m=-1) = (x, y) pair
    const float a = x[flat(1, 1)], b = x[flat(1, -1)];
    const float xp = f.c1 * a + f.s1 * b;
    x[flat(1, -1)] = -f.s1 * a + f.c1 * b;
    // D_y(-t): (z, x) block
    const float zz = x[flat(1, 0)];
    x[flat(1, 0)] = f.ct * zz + f.st * xp;
    x[flat(1, 1)] = -f.st * zz + f.ct * xp;
  }
  if constexpr (LMAX >= 2) {
    // D_z(-p): pairs (m=1, -1) with angle p and (m=2, -2) with angle 2p
    const float a1 = x[flat(2, 1)], b1 = x[flat(2, -1)];
    const float a2 = x[flat(2, 2)], b2 = x[flat(2, -2)];
    const float p1 = f.c1 * a1 + f.s1 * b1;
    const float n1 = -f.s1 * a1 + f.c1 * b1;
    const float p2 = f.c2 * a2 + f.s2 * b2;
    const float n2 = -f.s2 * a2 + f.c2 * b2;
    // D_y(-t): m < 0 block [[c, -s], [s, c]] on (m=-2, m=-1)
    x[flat(2, -2)] = f.ct * n2 - f.st * n1;
    x[flat(2, -1)] = f.st * n2 + f.ct * n1;
    // m >= 0 block of D_y(-t) = transpose of the D_y(+t) block
    const float z0 = x[flat(2, 0)];
    x[flat(2, 0)] = d.d00 * z0 + d.d01 * p1 + d.d02 * p2;
    x[flat(2, 1)] = -d.d01 * z0 + d.d11 * p1 + d.d12 * p2;
    x[flat(2, 2)] = d.d02 * z0 - d.d12 * p1 + d.d22 * p2;
  }
}

// x <- D(Q)^T x = D_z(p) D_y(t) x   (aligned frame -> global frame)
template <int LMAX>
__device__ inline void rotate_out(float* x, const Frame& f, const Dy2& d) {
  if constexpr (LMAX >= 1) {
    const float zz = x[flat(1, 0)], xx = x[flat(1, 1)];
    // D_y(t)
    x[flat(1, 0)] = f.ct * zz - f.st * xx;
    const float xp = f.st * zz + f.ct * xx;
    // D_z(p)
    const float b = x[flat(1, -1)];
    x[flat(1, 1)] = f.c1 * xp - f.s1 * b;
    x[flat(1, -1)] = f.s1 * xp + f.c1 * b;
  }
  if constexpr (LMAX >= 2) {
    const float n2 = x[flat(2, -2)], n1 = x[flat(2, -1)];
    const float z0 = x[flat(2, 0)], p1 = x[flat(2, 1)], p2 = x[flat(2, 2)];
    // D_y(t): m < 0 block [[c, s], [-s, c]]
    const float m2 = f.ct * n2 + f.st * n1;
    const float m1 = -f.st * n2 + f.ct * n1;
    // D_y(t): m >= 0 block
    const float q0 = d.d00 * z0 - d.d01 * p1 + d.d02 * p2;
    const float q1 = d.d01 * z0 + d.d11 * p1 - d.d12 * p2;
    const float q2 = d.d02 * z0 + d.d12 * p1 + d.d22 * p2;
    x[flat(2, 0)] = q0;
    // D_z(p) on the pairs
    x[flat(2, 1)] = f.c1 * q1 - f.s1 * m1;
    x[flat(2, -1)] = f.s1 * q1 + f.c1 * m1;
    x[flat(2, 2)] = f.c2 * q2 - f.s2 * m2;
    x[flat(2, -2)] = f.s2 * q2 + f.c2 * m2;
  }
}

// Per-atom reindex weights: k[p][m] = w_p <li m lf 0 | lo m> |r|^lf.
template <int LMAX>
struct Reindex {
  float k[kMaxPaths][LMAX + 1];
};

template <int LMAX>
__device__ inline Reindex<LMAX> make_reindex(const EaasCoef& cf, const Frame& f) {
  Reindex<LMAX> R;
  int p = 0;
#pragma unroll
  for (int li = 0; li <= LMAX; ++li)
#pragma unroll
    for (int lf = 0; lf <= LMAX; ++lf)
#pragma unroll
      for (int lo = 0; lo <= LMAX; ++lo) {
        if (lo < (li > lf ? li - lf : lf - li) || lo > li + lf) continue;
        const float rl = lf == 0 ? 1.0f : (lf == 1 ? f.r1 : f.r2);
#pragma unroll
        for (int m = 0; m <= LMAX; ++m) R.k[p][m] = cf.c[p][m] * rl;
        ++p;
      }
  return R;
}

// y = P(x) in the aligned frame: even li+lf+lo keeps m_i = m_o, odd maps
// m_i = -m_o with the sign (+ for m_o > 0, - for m_o < 0); y[lo, 0] gets
// nothing from odd paths.
template <int LMAX>
__device__ inline void reindex(const float* x, float* y, const Reindex<LMAX>& R) {
#pragma unroll
  for (int s = 0; s < ncomp(LMAX); ++s) y[s] = 0.0f;
  int p = 0;
#pragma unroll
  for (int li = 0; li <= LMAX; ++li)
#pragma unroll
    for (int lf = 0; lf <= LMAX; ++lf)
#pragma unroll
      for (int lo = 0; lo <= LMAX; ++lo) {
        if (lo < (li > lf ? li - lf : lf - li) || lo > li + lf) continue;
        const int mmax = li < lo ? li : lo;
        if (((li + lf + lo) & 1) == 0) {
#pragma unroll
          for (int m = 0; m <= mmax; ++m) {
            y[flat(lo, m)] += R.k[p][m] * x[flat(li, m)];
            if (m > 0) y[flat(lo, -m)] += R.k[p][m] * x[flat(li, -m)];
          }
        } else {
#pragma unroll
          for (int m = 1; m <= mmax; ++m) {
            y[flat(lo, m)] += R.k[p][m] * x[flat(li, -m)];
            y[flat(lo, -m)] -= R.k[p][m] * x[flat(li, m)];
          }
        }
        ++p;
      }
}

// x = P^T(y): the transpose of the reindex (adjoint of the aligned-frame map)
template <int LMAX>
__device__ inline void reindex_t(const float* y, float* x, const Reindex<LMAX>& R) {
#pragma unroll
  for (int s = 0; s < ncomp(LMAX); ++s) x[s] = 0.0f;
  int p = 0;
#pragma unroll
  for (int li = 0; li <= LMAX; ++li)
#pragma unroll
    for (int lf = 0; lf <= LMAX; ++lf)
#pragma unroll
      for (int lo = 0; lo <= LMAX; ++lo) {
        if (lo < (li > lf ? li - lf : lf - li) || lo > li + lf) continue;
        const int mmax = li < lo ? li : lo;
        if (((li + lf + lo) & 1) == 0) {
#pragma unroll
          for (int m = 0; m <= mmax; ++m) {
            x[flat(li, m)] += R.k[p][m] * y[flat(lo, m)];
            if (m > 0) x[flat(li, -m)] += R.k[p][m] * y[flat(lo, -m)];
          }
        } else {
#pragma unroll
          for (int m = 1; m <= mmax; ++m) {
            x[flat(li, -m)] += R.k[p][m] * y[flat(lo, m)];
            x[flat(li, m)] -= R.k[p][m] * y[flat(lo, -m)];
          }
        }
        ++p;
      }
}

// Reindex weights for the position gradient (no path to l_f = 0 moves with r):
//   radial: w_p c_m l_f |r|^(l_f - 1)   (d/d|r| of the value weights)
//   hat:    w_p c_m |r|^(l_f - 1)       (value weights over |r|, for the torque terms)
template <int LMAX>
__device__ inline void make_grad_reindex(const EaasCoef& cf, const Frame& f, Reindex<LMAX>& rad,
                                         Reindex<LMAX>& hat) {
  int p = 0;
#pragma unroll
  for (int li = 0; li <= LMAX; ++li)
#pragma unroll
    for (int lf = 0; lf <= LMAX; ++lf)
#pragma unroll
      for (int lo = 0; lo <= LMAX; ++lo) {
        if (lo < (li > lf ? li - lf : lf - li) || lo > li + lf) continue;
        const float rl1 = lf == 2 ? f.r1 : 1.0f;  // |r|^(l_f - 1) for l_f = 1, 2
#pragma unroll
        for (int m = 0; m <= LMAX; ++m) {
          hat.k[p][m] = lf == 0 ? 0.0f : cf.c[p][m] * rl1;
          rad.k[p][m] = hat.k[p][m] * (float)lf;
        }
        ++p;
      }
}

// Generators of rotations about the x and y axes in the real harmonic basis
// (D(R_a(e)) = 1 + e J_a + O(e^2)); at l = 1 the basis is (y, z, x), at l = 2
// the entries follow from differentiating the D_y blocks above at zero angle
// and J_x = J_y J_z - J_z J_y.
template <int LMAX>
__device__ inline void apply_jx(const float* x, float* y) {
  y[0] = 0.0f;
  if constexpr (LMAX >= 1) {
    y[flat(1, -1)] = -x[flat(1, 0)];
    y[flat(1, 0)] = x[flat(1, -1)];
    y[flat(1, 1)] = 0.0f;
  }
  if constexpr (LMAX >= 2) {
    const float k3 = 1.7320508075688772f;
    y[flat(2, -2)] = -x[flat(2, 1)];
    y[flat(2, -1)] = -k3 * x[flat(2, 0)] - x[flat(2, 2)];
    y[flat(2, 0)] = k3 * x[flat(2, -1)];
    y[flat(2, 1)] = x[flat(2, -2)];
    y[flat(2, 2)] = x[flat(2, -1)];
  }
}

template <int LMAX>
__device__ inline void apply_jy(const float* x, float* y) {
  y[0] = 0.0f;
  if constexpr (LMAX >= 1) {
    y[flat(1, -1)] = 0.0f;
    y[flat(1, 0)] = -x[flat(1, 1)];
    y[flat(1, 1)] = x[flat(1, 0)];
  }
  if constexpr (LMAX >= 2) {
    const float k3 = 1.7320508075688772f;
    y[flat(2, -2)] = x[flat(2, -1)];
    y[flat(2, -1)] = -x[flat(2, -2)];
    y[flat(2, 0)] = -k3 * x[flat(2, 1)];
    y[flat(2, 1)] = k3 * x[flat(2, 0)] - x[flat(2, 2)];
    y[flat(2, 2)] = x[flat(2, 1)];
  }
}

// Position gradient of f(r) = <g, x (x) R(r)> for one channel, in the aligned
// frame.  With xt = D(Q) x and gt = D(Q) g the product is <gt, P xt>:
//   * moving r along r_hat changes only |r|:        df/d|r| = <gt, P_rad xt>;
//   * rotating r about a local axis a (a = x, y) conjugates the map by that
//     rotation, so its derivative is the torque <gt, [J_a, P] xt>; rotating about
//     r itself changes nothing.  Torque about local a = (r' x grad')_a with
//     r' = |r| z, which gives grad'_x = t_y / |r| and grad'_y = -t_x / |r|.
// `hat` already carries the 1/|r|, so no division happens (also fine at r = 0).
// Adds (grad'_x, grad'_y, grad'_z) of this channel to acc; the caller rotates
// the channel sum back with Q^T.
template <int LMAX>
__device__ inline void pos_grad_channel(float* xt, float* gt, const Reindex<LMAX>& rad,
                                        const Reindex<LMAX>& hat, float* acc) {
  constexpr int S = ncomp(LMAX);
  float t[S], u[S], v[S];
  reindex<LMAX>(xt, t, rad);
  float dr = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) dr = fmaf(gt[s], t[s], dr);
  reindex<LMAX>(xt, t, hat);  // P_hat xt
  // t_a = -<J_a gt, P_hat xt> - <gt, P_hat J_a xt>
  float tx = 0.0f, ty = 0.0f;
  apply_jx<LMAX>(gt, u);
#pragma unroll
  for (int s = 0; s < S; ++s) tx = fmaf(-u[s], t[s], tx);
  apply_jx<LMAX>(xt, u);
  reindex<LMAX>(u, v, hat);
#pragma unroll
  for (int s = 0; s < S; ++s) tx = fmaf(-gt[s], v[s], tx);
  apply_jy<LMAX>(gt, u);
#pragma unroll
  for (int s = 0; s < S; ++s) ty = fmaf(-u[s], t[s], ty);
  apply_jy<LMAX>(xt, u);
  reindex<LMAX>(u, v, hat);
#pragma unroll
  for (int s = 0; s < S; ++s) ty = fmaf(-gt[s], v[s], ty);
  acc[0] += ty;
  acc[1] -= tx;
  acc[2] += dr;
}

// v = Q^T v' for the alignment rotation of the frame (local -> global vector)
__device__ inline void frame_to_global(const Frame& f, const float* l, float* g) {
  // rows of Q = R_y(-t) R_z(-p)
  g[0] = f.ct * f.c1 * l[0] - f.s1 * l[1] + f.st * f.c1 * l[2];
  g[1] = f.ct * f.s1 * l[0] + f.c1 * l[1] + f.st * f.s1 * l[2];
  g[2] = -f.st * l[0] + f.ct * l[2];
}

// full EAAS on one channel: x (global) -> y (global)
template <int LMAX>
__device__ inline void eaas_channel(float* x, float* y, const Frame& f, const Dy2& d,
                                    const Reindex<LMAX>& R) {
  rotate_in<LMAX>(x, f, d);
  reindex<LMAX>(x, y, R);
  rotate_out<LMAX>(y, f, d);
}

// adjoint EAAS on one channel: x = D^T P^T D y (y is overwritten)
template <int LMAX>
__device__ inline void eaas_channel_t(float* y, float* x, const Frame& f, const Dy2& d,
                                      const Reindex<LMAX>& R) {
  rotate_in<LMAX>(y, f, d);
  reindex_t<LMAX>(y, x, R);
  rotate_out<LMAX>(x, f, d);
}

// ------------------------------------------------ work units of the shared-row kernels
//
// One wave a unit.  XCD x takes the x-th contiguous stretch of sx schedule slots
// (workgroups are dealt to the XCDs round-robin, so XCD x runs blocks x, x + 8,
// ... in order), in `head` units of T slots and then, with tail_den > 0, units
// of tail_t slots for the last 1/tail_den of the stretch: a wave's time grows
// with its slots, so short closing units let the XCD's waves run out closer
// together.  Every slot lands in exactly one unit; a unit's slots past the
// stretch or N are empty.
struct UnitMap {
  int64_t sx;        // schedule slots per XCD
  int64_t head;      // units of T slots per XCD
  int64_t per_xcd;   // units per XCD (grid = kXcds * per_xcd)
};

__host__ __device__ inline UnitMap unit_map(int64_t N, int T, int tail_den, int tail_t) {
  const int64_t base = (N + T - 1) / T;
  const int64_t per0 = (base + kXcds - 1) / kXcds;
  UnitMap u;
  u.sx = per0 * T;
  const int64_t q = (int64_t)T * tail_t;   // the closing part holds whole units of both sizes
  const int64_t tl = tail_den > 0 ? u.sx / tail_den / q * q : 0;
  u.head = (u.sx - tl) / T;
  u.per_xcd = u.head + tl / tail_t;
  return u;
}

// block `blk`'s unit: its first slot, its number of slots, the end of its stretch
__host__ __device__ inline void unit_of_block(const UnitMap& u, int64_t blk, int T, int tail_t,
                                              int64_t& slot0, int& cnt, int64_t& xend) {
  const int64_t xcd = blk % kXcds, b = blk / kXcds;
  xend = (xcd + 1) * u.sx;
  if (b < u.head) {
    slot0 = xcd * u.sx + b * T;
    cnt = T;
  } else {
    slot0 = xcd * u.sx + u.head * T + (b - u.head) * tail_t;
    cnt = tail_t;
  }
}

// ------------------------------------------------------ storage types

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two fp32 values rounded to bf16 (nearest, ties to even; NaN stays a quiet NaN)
// by gfx950's packed conversion, one instruction for the pair; a in the low half.
__device__ inline uint32_t f32x2_to_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ inline uint16_t f32_to_bf16(float f) { return uint16_t(f32x2_to_bf16x2(f, 0.0f)); }

// One lane's V elements of a row exactly as loaded (fp32, or bf16 pairs packed
// in 32-bit words), widened to fp32 only where they are used.
template <typename T, int V>
struct Raw;

template <int V>
struct Raw<float, V> {
  float f[V];
  __device__ inline float get(int v) const { return f[v]; }
  __device__ inline void zero() {
#pragma unroll
    for (int v = 0; v < V; ++v) f[v] = 0.0f;
  }
};

template <int V>
struct Raw<uint16_t, V> {
  uint32_t w[(V + 1) / 2];
  __device__ inline float get(int v) const {
    const uint32_t x = w[v >> 1];
    return __uint_as_float((v & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  __device__ inline void zero() {
#pragma unroll
    for (int k = 0; k < (V + 1) / 2; ++k) w[k] = 0u;
  }
};

// Raw loads through a buffer resource: the row offset goes in an SGPR, so a
// neighbour's S + 1 rows cost one address computation (32-bit byte offsets).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <typename T, int V>
__device__ inline void buffer_load_raw(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                       Raw<T, V>& r) {
  constexpr int bytes = V * (int)sizeof(T);
  uint32_t* w;
  if constexpr (sizeof(T) == 4) {
    w = reinterpret_cast<uint32_t*>(r.f);
  } else {
    w = r.w;
  }
  if constexpr (bytes == 16) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (bytes == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, (int)soff, 0);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (bytes == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)voff, (int)soff, 0);
  } else {
    static_assert(bytes == 2, "row chunk size");
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)voff, (int)soff, 0);
  }
}

template <typename T, int V>
struct VecIO;

template <int V>
struct VecIO<float, V> {
  static __device__ inline void load_raw(const float* p, Raw<float, V>& r) { load(p, r.f); }
  static __device__ inline void load(const float* p, float* o) {
    if constexpr (V == 4) {
      const float4 v = *reinterpret_cast<const float4*>(p);
      o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (V == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      o[0] = v.x; o[1] = v.y;
    } else {
      static_assert(V == 1, "fp32 vector width");
      o[0] = *p;
    }
  }
  static __device__ inline void store(float* p, const float* o) {
    if constexpr (V == 8) {   // fp32 copies of 8-channel bf16 lanes (the fp32 message)
      *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(p + 4) = make_float4(o[4], o[5], o[6], o[7]);
    } else if constexpr (V == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
    } else if constexpr (V == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(o[0], o[1]);
    } else {
      static_assert(V == 1, "fp32 vector width");
      *p = o[0];
    }
  }
};

template <int V>
struct VecIO<uint16_t, V> {
  static __device__ inline void unpack(uint32_t w, float* o) {
    o[0] = __uint_as_float(w << 16);
    o[1] = __uint_as_float(w & 0xffff0000u);
  }
  static __device__ inline uint32_t pack(float a, float b) { return f32x2_to_bf16x2(a, b); }
  static __device__ inline void load_raw(const uint16_t* p, Raw<uint16_t, V>& r) {
    if constexpr (V == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (V == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      r.w[0] = v.x; r.w[1] = v.y;
    } else if constexpr (V == 2) {
      r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      r.w[0] = *p;
    }
  }
  static __device__ inline void load(const uint16_t* p, float* o) {
    if constexpr (V == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      unpack(v.x, o); unpack(v.y, o + 2); unpack(v.z, o + 4); unpack(v.w, o + 6);
    } else if constexpr (V == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      unpack(v.x, o); unpack(v.y, o + 2);
    } else if constexpr (V == 2) {
      unpack(*reinterpret_cast<const uint32_t*>(p), o);
    } else {
      static_assert(V == 1, "bf16 vector width");
      o[0] = bf16_to_f32(*p);
    }
  }
  static __device__ inline void store(uint16_t* p, const float* o) {
    if constexpr (V == 8) {
      *reinterpret_cast<uint4*>(p) =
          make_uint4(pack(o[0], o[1]), pack(o[2], o[3]), pack(o[4], o[5]), pack(o[6], o[7]));
    } else if constexpr (V == 4) {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack(o[0], o[1]), pack(o[2], o[3]));
    } else if constexpr (V == 2) {
      *reinterpret_cast<uint32_t*>(p) = pack(o[0], o[1]);
    } else {
      *p = f32_to_bf16(o[0]);
    }
  }
};

// Smooth distance envelope of the attention weights (EquiformerV3 page, method
// details: an envelope of the pair distance multiplies the softmax numerator
// and denominator).  u(x) = 1 - 21 x^5 + 35 x^6 - 15 x^7 for x = d / r_env < 1,
// 0 beyond, evaluated in its factored form (1 - x)^3 (1 + 3x + 6x^2 + 10x^3 +
// 15x^4), whose factors are all positive.  1 - x itself is ill-conditioned near
// the cutoff: from an fp32 distance its relative error grows as 2^-24 / (1 - x),
// and the cube triples it (3e-3 in u at 1 - x = 1e-4).  So the squared distance
// and r_env^2 - d^2 are taken in float64, where the difference of two fp32
// coordinates is exact; the rest is fp32.
struct EnvTerm {
  float log2u;   // log2 u(x); -inf at or beyond the cutoff
  float dlog;    // (d ln u / d r_i) = dlog * (r_i - r_j); 0 at or beyond the cutoff
};

// pi = r_i, pj = r_j (fp32 positions as given), rc = r_env.  d^2 and r_env^2 - d^2
// in float64 (exact differences, no cancellation left in 1 - x = (r_env^2 - d^2) /
// (r_env (r_env + d))); the denominator, x and the polynomial in fp32.
__device__ inline EnvTerm envelope_term(float xi, float yi, float zi, float xj, float yj, float zj,
                                        float rc) {
  const double dx = (double)xi - (double)xj;
  const double dy = (double)yi - (double)yj;
  const double dz = (double)zi - (double)zj;
  const double d2 = fma(dx, dx, fma(dy, dy, dz * dz));
  const double rc2 = (double)rc * (double)rc;
  EnvTerm e;
  if (!(d2 < rc2)) {
    e.log2u = -INFINITY;
    e.dlog = 0.0f;
    return e;
  }
  const float d = sqrtf((float)d2);
  const float inv_rc = 1.0f / rc;
  const float y = (float)(rc2 - d2) / (rc * (rc + d));
  const float x = d * inv_rc;
  const float q = fmaf(x, fmaf(x, fmaf(x, fmaf(x, 15.0f, 10.0f), 6.0f), 3.0f), 1.0f);
  e.log2u = __log2f(y * y * y * q);
  // u'(x) = -105 x^4 (1 - x)^2, so d ln u / dd = -105 x^4 / ((1 - x) q) / r_env and
  // the gradient along r_i - r_j divides by d = x r_env once more
  e.dlog = -105.0f * x * x * x / (y * q) * (inv_rc * inv_rc);
  return e;
}

// Exclusive prefix of v over the 1024 threads of a workgroup, in thread order,
// and the workgroup's total: a shuffle scan within each wave, then the 16 wave
// totals through `part` (16 ints of LDS).  One workgroup barrier; call once.
__device__ inline int32_t block_exclusive_scan_1024(int32_t v, int32_t* part, int32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t up = __shfl_up(inc, o);
    if (lane >= o) inc += up;
  }
  if (lane == 63) part[wv] = inc;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    before += k < wv ? part[k] : 0;
    all += part[k];
  }
  *total = all;
  return before + inc - v;
}

// ------------------------------------------------------------------------
// Union of several targets' neighbour lists, for kernels in which the targets
// of one wavefront share every source row they read.  The valid slots of the
// T lists (of at most MAXL slots each, kShareMaxK by default) are merged into
// 32-bit keys (bucket j mod P in the top lgp bits, then j / P, then the target),
// sorted in registers (wave_sort), and turned into the union of distinct
// sources, bucket by bucket and in increasing j within a bucket, with each source's
// slot count per target (16 bits per target) and each bucket's size and start.
// Subgroup g of the wave then streams bucket g.  hook(t, u, j) runs once per
// valid slot after the counts are cleared (e.g. to tabulate per-pair data).
constexpr int kShareMaxK = 256;

constexpr int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <int T, int MAXL = kShareMaxK>
struct ShareLds {
  static constexpr int EN = T * MAXL;         // merged slots, at most
  static constexpr int EN2 = pow2_ceil(EN);   // the sort pads to a power of two
  static constexpr int CW = (T + 1) / 2;      // count words per source
  uint32_t key[EN2];                          // merge keys, sorted
  int32_t uj[EN];                             // union sources, bucket by bucket
  uint32_t cnt[CW][EN];                       // slot counts per target, 16 bits each
  int32_t bcnt[64];                           // per bucket: union sources
  int32_t bstart[64];                         // per bucket: first union entry
};

__device__ inline void share_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline uint32_t share_key(uint32_t j, uint32_t t, int lgp) {
  const uint32_t hi = lgp ? (j & ((1u << lgp) - 1u)) << (32 - lgp) : 0u;
  return hi | ((j >> lgp) << 2) | t;
}

__device__ inline int32_t share_key_source(uint32_t k, int lgp) {
  const uint32_t b = lgp ? k >> (32 - lgp) : 0u;
  const uint32_t q = (k & (lgp ? (~0u >> lgp) : ~0u)) >> 2;
  return (int32_t)((q << lgp) | b);
}

// Bitonic sort of 64·R keys, R a lane in registers (element lane·R + r): the
// stages of stride below R compare within a lane, the others across lanes
// through a shuffle, so no stage waits on LDS.
template <int R>
__device__ inline void share_sort_regs(uint32_t* key, int lane) {
  uint32_t k[R];
#pragma unroll
  for (int r = 0; r < R; ++r) k[r] = key[lane * R + r];
#pragma unroll
  for (int kk = 2; kk <= 64 * R; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj >= R) {
        const int dl = jj / R;                       // partner lane: lane ^ dl
        const bool up = ((lane * R) & kk) == 0;      // ascending run
        const bool keep_min = ((lane & dl) == 0) == up;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t p = (uint32_t)__shfl_xor((int)k[r], dl);
          k[r] = keep_min ? min(k[r], p) : max(k[r], p);
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r & jj) continue;
          const int r2 = r + jj;
          const bool up = ((lane * R + r) & kk) == 0;
          const uint32_t lo = min(k[r], k[r2]), hi = max(k[r], k[r2]);
          k[r] = up ? lo : hi;
          k[r2] = up ? hi : lo;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) key[lane * R + r] = k[r];
}

// Ascending sort of key[0..cnt) by one wave (cnt <= MAXN, MAXN a power of two
// in [64, 1024]): padded with `pad`, which sorts after every key, to a power of
// two of at least 64, then sorted in registers.  Ends with a wave-wide LDS sync.
template <int MAXN>
__device__ inline void wave_sort(uint32_t* key, int cnt, int lane, uint32_t pad) {
  static_assert(MAXN >= 64 && MAXN <= 1024 && (MAXN & (MAXN - 1)) == 0, "sort sizes");
  int n2 = 64;
  while (n2 < cnt) n2 <<= 1;
  for (int e = cnt + lane; e < n2; e += 64) key[e] = pad;
  share_wave_sync();
  if (n2 == 64) {
    share_sort_regs<1>(key, lane);
  } else if (n2 == 128) {
    if constexpr (MAXN >= 128) share_sort_regs<2>(key, lane);
  } else if (n2 == 256) {
    if constexpr (MAXN >= 256) share_sort_regs<4>(key, lane);
  } else if (n2 == 512) {
    if constexpr (MAXN >= 512) share_sort_regs<8>(key, lane);
  } else {
    if constexpr (MAXN >= 1024) share_sort_regs<16>(key, lane);
  }
  share_wave_sync();
}

// Build the union of T lists: list t has len[t] <= MAXL slots and
// slot(t, sl) returns the source of its slot sl, or -1 for an empty slot;
// sources need j < 2^30.  Returns the number of union sources.  Ends with a
// wave-wide LDS sync.
template <int T, int MAXL, typename Slot, typename Hook>
__device__ inline int share_union(ShareLds<T, MAXL>& L, const int (&len)[T], Slot slot, int lgp,
                                  int lane, Hook hook) {
  static_assert(T >= 1 && T <= 4, "two bits of target index in the merge key");
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int P = 1 << lgp;
  // merge the lists' valid slots; every chunk's loads are issued before the first is used
  constexpr int NS = (MAXL + 63) / 64;   // 64-slot chunks a list
  int jv[T][NS];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const int sl = c * 64 + lane;
      jv[t][c] = sl < len[t] ? slot(t, sl) : -1;
    }
  int cnt = 0;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      if (c * 64 >= len[t]) break;   // uniform
      const bool ok = jv[t][c] >= 0;
      const uint64_t b = __ballot(ok);
      if (ok) L.key[cnt + __popcll(b & below)] = share_key((uint32_t)jv[t][c], (uint32_t)t, lgp);
      cnt += __popcll(b);
    }
  L.bcnt[lane] = 0;
  // sort the keys (the largest key pads)
  wave_sort<ShareLds<T, MAXL>::EN2>(L.key, cnt, lane, 0xffffffffu);
  // the union: one entry per distinct source, bucket sizes
  int nu = 0;
  for (int e0 = 0; e0 < cnt; e0 += 64) {
    const int e = e0 + lane;
    const bool in = e < cnt;
    const uint32_t kk = in ? L.key[e] : 0u;
    const bool head = in && (e == 0 || (L.key[e - 1] >> 2) != (kk >> 2));
    const uint64_t b = __ballot(head);
    if (head) {
      const int u = nu + __popcll(b & below);
      const int32_t j = share_key_source(kk, lgp);
      L.uj[u] = j;
#pragma unroll
      for (int c = 0; c < ShareLds<T, MAXL>::CW; ++c) L.cnt[c][u] = 0u;
      atomicAdd(&L.bcnt[j & (P - 1)], 1);
    }
    nu += __popcll(b);
  }
  share_wave_sync();
  // slot counts per (source, target)
  {
    int run = 0;  // heads before this chunk
    for (int e0 = 0; e0 < cnt; e0 += 64) {
      const int e = e0 + lane;
      const bool in = e < cnt;
      const uint32_t kk = in ? L.key[e] : 0u;
      const bool head = in && (e == 0 || (L.key[e - 1] >> 2) != (kk >> 2));
      const uint64_t b = __ballot(head);
      if (in) {
        const int u = run + __popcll(b & (below | (1ull << lane))) - 1;
        const int t = (int)(kk & 3u);
        atomicAdd(&L.cnt[t >> 1][u], 1u << (16 * (t & 1)));
        hook(t, u, share_key_source(kk, lgp));
      }
      run += __popcll(b);
    }
  }
  // bucket starts: buckets follow each other in the sorted union
  if (lane == 0) {
    int acc0 = 0;
    for (int g = 0; g < P; ++g) {
      L.bstart[g] = acc0;
      acc0 += L.bcnt[g];
    }
  }
  share_wave_sync();
  return nu;
}

// The union of T targets' padded neighbour rows (idx + mask, K slots each; an
// index outside [0, N) at a valid slot is skipped like a masked slot).
template <int T, typename Hook>
__device__ inline int share_union_rows(ShareLds<T>& L, const int32_t* idx, const uint8_t* mask,
                                       int64_t N, int K, const int64_t (&tg)[T], int lgp,
                                       int lane, Hook hook) {
  int len[T];
#pragma unroll
  for (int t = 0; t < T; ++t) len[t] = tg[t] >= 0 ? K : 0;
  return share_union<T, kShareMaxK>(L, len,
                        [&](int t, int sl) -> int {
                          int64_t i = tg[0];
#pragma unroll
                          for (int tt = 1; tt < T; ++tt)
                            if (t == tt) i = tg[tt];
                          // both loads independent of each other
                          const uint8_t m = mask[i * K + sl];
                          const int j = idx[i * K + sl];
                          return (m != 0 && j >= 0 && (int64_t)j < N) ? j : -1;
                        },
                        lgp, lane, hook);
}

// slot count of target t in the packed count words of one union source
template <int CW>
__device__ inline uint32_t share_count(const uint32_t (&cw)[CW], int t) {
  return (cw[t >> 1] >> (16 * (t & 1))) & 0xffffu;
}

}  // namespace e2f
