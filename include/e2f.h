/*
 * e2f.h -- C ABI of libe2f: E2Former-V2's on-the-fly equivariant attention
 * (forward pass) on AMD Instinct MI355X (gfx950).
 *
 * Method (E2Former-V2 news write-up on stapisi.com, sections 2 and 3; the
 * gist.science technical summary of arXiv 2601.16622, sections 2.1-2.2):
 *
 *   step 1  h'_j  = h_j (x) R(r_j)            EAAS tensor product per source atom
 *   step 2  m_i   = sum_j alpha_ij h'_j       streamed over i's padded neighbour
 *                                             list with an online softmax
 *   step 3  out_i = m_i (x) R(r_i)            EAAS tensor product per target atom
 *
 * "(x) R(r)" couples each irrep block of a feature with the real solid
 * harmonics R_lf(r) = |r|^lf C_lf(r_hat) (Racah normalisation, components
 * m = -l..l at flat index l*l + l + m, l = 1 ordered (y, z, x)) over every
 * path (li, lf, lo) with li, lf, lo <= lmax and |li - lf| <= lo <= li + lf,
 * channel-wise, summed per lo.  EAAS (write-up section 2, Proposition 4.3)
 * evaluates it exactly as: rotate the feature into the frame whose z axis
 * lies along r, apply the sparse reindex (li + lf + lo even: m_i = m_o;
 * odd: m_i = -m_o with a sign), rotate back.
 *
 * The attention logits use SO(3)-invariant scalars only (gist.science
 * summary 2.2): q_i = h_i[l=0, :], k_j = h_j[l=0, :]; head h owns channels
 * [h*d, (h+1)*d), d = C / H, for Q, K and V; logit = scale * <q_i, k_j>.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Buffers are device memory owned by the caller (path_w excepted: it is a
 *   small host array folded into the kernel arguments); the library
 *   allocates nothing and keeps no mutable global state beyond a
 *   mutex-guarded count of the HIP runtimes mapped (E2F_ERR_RUNTIME);
 *   entry points are reentrant and thread-safe.
 * - Layouts are dense row-major with channels innermost:
 *     positions   float  [n, 3]          (always fp32, angstrom, as given)
 *     features    T      [n, S, C]       S = (lmax + 1)^2, T per `dtype`
 *     nbr_idx     int32  [N, K]          padded neighbour list
 *     nbr_mask    uint8  [N, K]          1 = valid slot, 0 = padded
 *     path_w      float  [P] or NULL     HOST memory: per-path weight, NULL =
 *                                        all 1; P = e2f_path_count(lmax),
 *                                        paths in lexicographic (li, lf, lo)
 *                                        order; read during the call only
 * - `dtype` is E2F_F32 or E2F_BF16 and applies to features, workspace and
 *   outputs; bf16 is stored round-to-nearest-even, all arithmetic is fp32.
 * - Feature, workspace and output pointers must be 16-byte aligned;
 *   positions, path_w and nbr_idx 4-byte aligned.
 * - Argument errors are returned synchronously, before anything is enqueued.
 *   Work is enqueued on `stream` and the call returns without waiting, except
 *   under E2F_VALIDATE_INDICES.  Device faults surface at the caller's next
 *   synchronisation, as usual for HIP.
 * - n = 0 (or N = 0) is a successful no-op.
 * - Supported sizes: lmax in {0, 1, 2}; C >= 1, H >= 1, C % H == 0.  The
 *   attention forward serves every such layout up to C = 512 (wider rows:
 *   E2F_ERR_UNSUPPORTED): layouts with a per-lane channel count V in {1, 2,
 *   4} (fp32) or {1, 2, 4, 8} (bf16) with V | d, d / V a power of two and
 *   C / V <= 64 take the vectorised kernels, every other one (head widths
 *   d = 3, 5, 6, 12, ..., fp32 rows above 256 channels) a general kernel with
 *   one channel a lane.  The backward needs such a V (E2F_ERR_UNSUPPORTED
 *   otherwise).
 */
#ifndef E2F_H_
#define E2F_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage type of features, workspace and outputs */
typedef enum e2f_dtype {
  E2F_F32 = 0,
  E2F_BF16 = 1
} e2f_dtype;

/* status codes */
#define E2F_OK 0
#define E2F_ERR_NULL (-1)        /* a required pointer is NULL */
#define E2F_ERR_SHAPE (-2)       /* n < 0, K < 1, C < 1, H < 1, C % H != 0, lmax not in 0..2 */
#define E2F_ERR_DTYPE (-3)       /* dtype is not an e2f_dtype value */
#define E2F_ERR_ALIGN (-4)       /* a pointer breaks its alignment rule */
#define E2F_ERR_WORKSPACE (-5)   /* ws_bytes < e2f_attn_workspace_bytes(...) */
#define E2F_ERR_ALIAS (-6)       /* an output overlaps an input or another output */
#define E2F_ERR_HIP (-7)         /* the HIP runtime reported an error at launch */
#define E2F_ERR_INDEX (-8)       /* a valid slot holds an index outside [0, N) (validation only) */
#define E2F_ERR_UNSUPPORTED (-9) /* channel / head layout outside the kernels' lane mapping */
#define E2F_ERR_RUNTIME (-10)    /* two HIP runtimes are mapped into the process (e.g. this
                                    library's libamdhip64.so.7 and a framework's own copy):
                                    pointers and streams of one are invalid in the other; every
                                    entry point that launches returns this before touching HIP */

/* flags of the attention entry points (any other bit: E2F_ERR_SHAPE) */
#define E2F_VALIDATE_INDICES 1u  /* check every valid slot's index before running; synchronises */
#define E2F_TARGETS_IN_ORDER 2u  /* visit targets in index order: skip the spatial schedule, for
                                    atoms already stored in a spatially coherent order */
#define E2F_MSG_F32 4u           /* out_msg is stored fp32 whatever the dtype (the message
                                    before any rounding to the storage type) */
#define E2F_SHARED_ROWS 8u       /* fp32 layouts: run the kernels in which several atoms of a
                                    wave share the rows they read whatever N.  Without it they
                                    run above 4,096 atoms only, where N/3 waves fill the chip;
                                    below, one atom a wave is faster.  Either way the result is
                                    the same function, rounded in another order. */
#define E2F_MATRIX_TILES 16u     /* run the aggregate on the matrix cores, 16 atoms a
                                    workgroup sharing the rows they read, where that kernel
                                    serves the layout (fp32, C = 128, H = 16, K <= 256, no
                                    envelope); ignored elsewhere and under E2F_SHARED_ROWS.
                                    Opt-in: slower than the default kernels at the measured
                                    sizes.  The same function, rounded in another order; each
                                    atom's result does not depend on the atoms sharing its
                                    workgroup. */

/* Name of a status code ("E2F_OK", "E2F_ERR_SHAPE", ...); never NULL. */
const char* e2f_status_string(int status);

/* Number of coupling paths at this lmax (1, 5 or 15), or E2F_ERR_SHAPE. */
int e2f_path_count(int lmax);

/* The hipError_t value behind the calling thread's most recent E2F_ERR_HIP
 * (0 if none yet); e2f_last_hip_error_name gives its HIP name. */
int e2f_last_hip_error(void);
const char* e2f_last_hip_error_name(void);

/*
 * e2f_eaas_couple -- the EAAS tensor product h_out_a = h_in_a (x) R(r_a).
 * Write-up section 2 (alignment rotation, feature rotation, sparse
 * reindex, inverse rotation; Proposition 4.3).
 *   r      [n, 3] fp32     vectors (any length, including 0)
 *   h_in   [n, S, C] T     features
 *   path_w [P] fp32|NULL   host array of per-path weights (one-hot isolates a path)
 *   h_out  [n, S, C] T     result; may equal h_in exactly (in place), must
 *                          not overlap it otherwise
 */
int e2f_eaas_couple(hipStream_t stream, int64_t n, int lmax, int C, int dtype,
                    const float* r, const void* h_in, const float* path_w, void* h_out);

/*
 * e2f_dense_couple -- the same product h_out_a = h_in_a (x) R(r_a) as
 * e2f_eaas_couple, computed the way EAAS avoids: for every path the full real
 * Clebsch-Gordan tensor C_p[mi, mf, mo] (zeros included) is contracted with
 * the feature block and the solid harmonics,
 *   y[lo, mo] = sum_p w_p sum_{mi, mf} C_p[mi, mf, mo] h[li, mi] R_lf(r)[mf],
 * 615 multiply-adds per channel at lmax = 2 (write-up section 2.2, Fig. 3:
 * the dense baseline of the EAAS speed-up; gist.science summary 2.1: dense
 * CG at O(L^6)).  Real basis: spherical components T_0 = x_0,
 * T_{+m} = (-1)^m (x_m + i x_{-m}) / sqrt2, T_{-m} = (x_m - i x_{-m}) / sqrt2,
 * Condon-Shortley coefficients, odd li + lf + lo tensors times -i.  By
 * Proposition 4.3 the result equals e2f_eaas_couple's up to rounding.
 * Arguments, layouts, in-place use and errors as for e2f_eaas_couple.
 */
int e2f_dense_couple(hipStream_t stream, int64_t n, int lmax, int C, int dtype,
                     const float* r, const void* h_in, const float* path_w, void* h_out);

/*
 * Workspace bytes that e2f_attn_precouple / _aggregate / _forward need for
 * N atoms, 0 on bad arguments.  Layout, each part 256-byte aligned:
 *   - the pre-coupled values of step 1, stored per atom as S + 1 rows of C
 *     elements (row 0 = k_j = h_j[l=0, :], rows 1..S = h'_j), so that each
 *     neighbour's K and V are one contiguous (S + 1) * C * sizeof(T) block;
 *   - the query rows q_i, N rows of C elements (h_i[l=0, :]);
 *   - 256 bytes for the validation flag;
 *   - the target schedule scratch (order and cell per atom, 2^15 cell
 *     counts, bounding-box partials): 8 N bytes plus about 140 KiB.
 */
size_t e2f_attn_workspace_bytes(int64_t N, int lmax, int C, int dtype);

/*
 * e2f_attn_precouple -- step 1 (write-up section 3.1): fills the workspace
 * with k_j and h'_j = h_j (x) R(pos_j) for every atom.
 *   pos [N, 3] fp32, h [N, S, C] T, workspace as above (written).
 */
int e2f_attn_precouple(hipStream_t stream, int64_t N, int lmax, int C, int dtype,
                       const float* pos, const void* h, const float* path_w,
                       void* workspace, size_t ws_bytes);

/*
 * e2f_attn_precouple_proj -- step 1 with learned projections, the queries and
 * keys as invariant scalar projections (gist.science summary of arXiv
 * 2601.16622, technical summary 2.2, Eq. 6) and the values mixed per degree:
 *   q_i = h_i[l=0] W_Q,  k_i = h_i[l=0] W_K,  v_i[l] = h_i[l] W_V[l],
 *   h'_i = v_i (x) R(pos_i)   (EAAS, write-up section 2),
 * written to the same workspace layout, so e2f_attn_aggregate follows as
 * without projections.  The products run on the matrix cores (MFMA) with
 * fp32 accumulation.
 *   w_q, w_k  [C, C] device arrays of the storage type, row-major
 *             [C_in, C_out], applied from the right
 *   w_v       [lmax + 1, C, C] device array, one matrix per degree
 * C = 16, 32, 64, 128 (fp32) and 32, 64, 128 (bf16) run on the matrix cores;
 * any other C up to 1024 on the vector ALUs (same products, fp32 accumulation,
 * input channels summed in order); above 1024: E2F_ERR_UNSUPPORTED.
 * Weights must be 16-byte aligned and must not overlap
 * the workspace.
 */
int e2f_attn_precouple_proj(hipStream_t stream, int64_t N, int lmax, int C, int dtype,
                            const float* pos, const void* h, const void* w_q, const void* w_k,
                            const void* w_v, const float* path_w, void* workspace,
                            size_t ws_bytes);

/*
 * e2f_attn_aggregate -- steps 2 and 3 (write-up sections 3.1-3.2): one
 * wavefront per target streams its valid slots once, computes the per-head
 * logits, keeps a running max and normaliser (online softmax) and fp32
 * accumulators on chip, divides, and couples the result with the target's
 * own harmonics.  No per-edge tensor is written.
 *   pos       [N, 3] fp32
 *   nbr_idx   [N, K] int32   index of the source atom at each slot; read only
 *                            at mask = 1 slots; an index outside [0, N) at a
 *                            valid slot is skipped like a masked slot, or
 *                            reported as E2F_ERR_INDEX under
 *                            E2F_VALIDATE_INDICES
 *   nbr_mask  [N, K] uint8   any pattern; valid slots need not come first;
 *                            repeated indices count once per slot
 *   scale     logit scale; <= 0 selects 1 / sqrt(C / H)
 *   env_cutoff  0: plain softmax.  r_env > 0 (finite): smooth distance
 *             envelope (EquiformerV3 page, method details, attention: an
 *             envelope of the pair distance multiplies the softmax numerator
 *             and denominator); the weights become
 *               e_ij exp(s_ijh) / sum_k e_ik exp(s_ikh),  e_ij = u(|pos_i - pos_j| / r_env),
 *               u(x) = 1 - 21 x^5 + 35 x^6 - 15 x^7 = (1-x)^3 (1+3x+6x^2+10x^3+15x^4)
 *             for x < 1 and 0 beyond (u, u' and u'' vanish at the cutoff).
 *             The squared distance and r_env^2 - d^2 are taken in fp64 from
 *             the fp32 positions (1 - x is ill-conditioned near the cutoff),
 *             the rest of u in fp32.  A slot at or beyond r_env weighs
 *             nothing; a target whose every slot does gives 0 like an empty
 *             row; lse then includes ln e.  Negative, infinite or NaN:
 *             E2F_ERR_SHAPE.
 *   workspace filled by e2f_attn_precouple (or _proj); its schedule scratch (and, under
 *             E2F_VALIDATE_INDICES, its flag) is rewritten here, hence not
 *             const.  Targets are visited in Hilbert-curve order of
 *             their cells on a grid over the positions' bounding box (built
 *             on the GPU each call unless
 *             E2F_TARGETS_IN_ORDER or N <= 2048), each XCD taking one contiguous
 *             stretch, so that waves sharing an L2 share neighbours; the
 *             visiting order never changes any target's result.
 *   out       [N, S, C] T    out_i; exactly 0 for a target with no valid slot
 *   out_msg   [N, S, C] T (fp32 under E2F_MSG_F32) or NULL: also store the
 *             normalised message m_i
 *   lse       [N, H] fp32 or NULL: also store each head's natural log-sum-exp
 *             of the logits over the valid slots (-inf with no valid slot);
 *             with out_msg, this is what e2f_attn_backward needs
 *   flags     0 or E2F_VALIDATE_INDICES | E2F_TARGETS_IN_ORDER | E2F_MSG_F32 |
 *             E2F_SHARED_ROWS | E2F_MATRIX_TILES
 */
int e2f_attn_aggregate(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                       const float* pos, const int32_t* nbr_idx, const uint8_t* nbr_mask,
                       float scale, float env_cutoff, const float* path_w, void* workspace,
                       size_t ws_bytes, void* out, void* out_msg, float* lse, uint32_t flags);

/* e2f_attn_forward -- e2f_attn_precouple then e2f_attn_aggregate on one stream. */
int e2f_attn_forward(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                     const float* pos, const void* h, const int32_t* nbr_idx,
                     const uint8_t* nbr_mask, float scale, float env_cutoff,
                     const float* path_w, void* workspace, size_t ws_bytes, void* out,
                     void* out_msg, float* lse, uint32_t flags);

/* e2f_attn_forward_proj -- e2f_attn_precouple_proj then e2f_attn_aggregate. */
int e2f_attn_forward_proj(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                          const float* pos, const void* h, const void* w_q, const void* w_k,
                          const void* w_v, const int32_t* nbr_idx, const uint8_t* nbr_mask,
                          float scale, float env_cutoff, const float* path_w, void* workspace,
                          size_t ws_bytes, void* out, void* out_msg, float* lse, uint32_t flags);

/*
 * e2f_attn_forward_noalloc -- e2f_attn_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument; the workspace is
 * the library's own static device array of e2f_attn_noalloc_max_bytes()
 * bytes (64 MiB), one per GPU, created when the library's code is loaded on
 * that GPU and held until the process ends.  The call allocates nothing.
 *   - Arguments, outputs, flags and errors as for e2f_attn_forward; N with
 *     e2f_attn_workspace_bytes(N, lmax, C, dtype) above the array's size gives
 *     E2F_ERR_WORKSPACE (at lmax 2, C 128: about 10,900 atoms at fp32,
 *     21,800 at bf16).
 *   - Every call on one GPU uses that GPU's one array, which keeps the last
 *     call's contents: calls that overlap on one GPU (other streams, other
 *     threads) race on it and must be serialised by the caller.
 *   - The array's device address is looked up on the first call on each
 *     device (the stream's device); that first call is not capturable.
 */
int e2f_attn_forward_noalloc(hipStream_t stream, int64_t N, int K, int lmax, int C, int H,
                             int dtype, const float* pos, const void* h, const int32_t* nbr_idx,
                             const uint8_t* nbr_mask, float scale, float env_cutoff,
                             const float* path_w, void* out, void* out_msg, float* lse,
                             uint32_t flags);

/* Size in bytes of the static workspace of e2f_attn_forward_noalloc. */
size_t e2f_attn_noalloc_max_bytes(void);

/*
 * Backward pass (vector-Jacobian product) of the attention, for forces as
 * derivatives of an energy with respect to positions (the write-up's
 * "Conservative" variant, section 4.2): given G = dL/d out it returns
 * dL/dh and dL/dpos.  Softmax weights are recomputed from the forward's
 * log-sum-exp (no per-edge tensor is stored); feature gradients use the
 * adjoint EAAS map and position gradients its derivative with respect to
 * r (radial part and rotation generators in the aligned frame).
 *
 * e2f_attn_backward_workspace_bytes -- scratch bytes for N atoms and K slots:
 * (S + 1) C + C + H floats per atom, the reverse neighbour list (8 N + 4 N K
 * bytes) and the target schedule scratch; with bf16 storage also fp32 copies
 * of h, G and dL/dh, the recomputed message and log-sum-exp, and an fp32
 * attention workspace (e2f_attn_workspace_bytes at E2F_F32).  0 on bad
 * arguments.
 */
size_t e2f_attn_backward_workspace_bytes(int64_t N, int K, int lmax, int C, int H, int dtype);

/*
 * e2f_attn_backward -- fp32 or bf16 storage, fp32 arithmetic.  With bf16
 * storage, h and G are widened exactly into fp32 copies in the backward
 * workspace, the forward (step 1, message, log-sum-exp) is recomputed from
 * them in fp32, and the gradients of that are taken; dL/dh is rounded to bf16
 * at the end.  (The stored bf16 workspace and message would carry a 2^-9
 * rounding into the softmax backward's <dm_i, h'_j> - <dm_i, m_i>, which
 * cancels.)  E2F_ERR_UNSUPPORTED for N above 2^24, K above 2048, N K at or
 * above 2^31, or a layout without an fp32 lane width.
 *   pos, h, nbr_idx, nbr_mask, scale, env_cutoff, path_w: as given to the
 *               forward (with an envelope, dL/dpos includes its derivative
 *               through each pair distance)
 *   workspace   the forward's workspace after e2f_attn_precouple (read only;
 *               the layer without projections is differentiated, with q_i read
 *               from the workspace's query rows)
 *   msg, lse    the forward's out_msg ([N, S, C] fp32) and lse ([N, H] fp32)
 *               outputs; with bf16 storage they are recomputed and these are
 *               not read (NULL allowed)
 *   grad_out    [N, S, C] T     dL/d out
 *   grad_h      [N, S, C] T     dL/dh (written)
 *   grad_pos    [N, 3] fp32     dL/dpos (written)
 *   bwd_workspace, bwd_ws_bytes  scratch of e2f_attn_backward_workspace_bytes
 *               (with bf16 storage it also holds the fp32 copies)
 *   flags       0 or E2F_TARGETS_IN_ORDER | E2F_SHARED_ROWS | E2F_MATRIX_TILES (index
 *               order, also taken for N <= 2048; the kernels of a recomputed forward)
 * The result does not depend on the order of a target's slots, nor on the
 * order in which the reverse list is filled for sources listed by at most
 * 16,384 targets (each source's list is sorted before it is summed).
 */
int e2f_attn_backward(hipStream_t stream, int64_t N, int K, int lmax, int C, int H, int dtype,
                      const float* pos, const void* h, const int32_t* nbr_idx,
                      const uint8_t* nbr_mask, float scale, float env_cutoff,
                      const float* path_w, const void* workspace, size_t ws_bytes,
                      const void* msg, const float* lse, const void* grad_out, void* grad_h,
                      float* grad_pos, void* bwd_workspace, size_t bwd_ws_bytes,
                      uint32_t flags);

/*
 * e2f_attn_backward_proj -- the backward pass of the layer with learned
 * projections (e2f_attn_precouple_proj's q, k and v; gist.science summary,
 * technical summary 2.2, Eq. 6): besides dL/dh and dL/dpos it returns the
 * weight gradients
 *   dL/dW_Q = sum_i h_i[0]^T dq_i,  dL/dW_K = sum_i h_i[0]^T dk_i,
 *   dL/dW_V[l] = sum_i sum_m h_i[l, m]^T dv_i[l, m],
 * and dL/dh flows through the projections:
 *   dL/dh_i[0] = dv_i[0] W_V[0]^T + dq_i W_Q^T + dk_i W_K^T,
 *   dL/dh_i[l] = dv_i[l] W_V[l]^T (l > 0),
 * where dq, dk are the logit gradients and dv the adjoint pre-coupling of the
 * value gradients.  The value rows v = h W_V are recomputed (the position
 * gradient of the pre-coupling needs them).  Arguments as e2f_attn_backward,
 * plus:
 *   w_q, w_k, w_v     the forward's weights (storage type, 16-byte aligned);
 *                     workspace must come from e2f_attn_precouple_proj with them
 *   grad_w_q, grad_w_k  [C, C] fp32, written (not accumulated)
 *   grad_w_v          [lmax + 1, C, C] fp32, written
 *   bwd_workspace     e2f_attn_backward_proj_workspace_bytes(...) bytes: that
 *                     of e2f_attn_backward plus v, dv and dk, fp32 weight copies
 *                     (bf16), and the weight gradients' partial sums (one [C, C]
 *                     matrix per chunk of rows, chunks sized for about 4,096
 *                     waves and at least 512 rows, at most 128 MiB in all)
 * The weight gradients are sums over chunks of rows, the chunks added in a
 * fixed order: the same bits on every run.  The products run on the matrix
 * cores for C = 16, 32, 64, 128, on the vector ALUs for other C up to 1024.
 * E2F_ERR_UNSUPPORTED where e2f_attn_backward or the projections are.
 */
size_t e2f_attn_backward_proj_workspace_bytes(int64_t N, int K, int lmax, int C, int H,
                                              int dtype);
int e2f_attn_backward_proj(hipStream_t stream, int64_t N, int K, int lmax, int C, int H,
                           int dtype, const float* pos, const void* h, const void* w_q,
                           const void* w_k, const void* w_v, const int32_t* nbr_idx,
                           const uint8_t* nbr_mask, float scale, float env_cutoff,
                           const float* path_w, const void* workspace, size_t ws_bytes,
                           const void* msg, const float* lse, const void* grad_out, void* grad_h,
                           float* grad_pos, float* grad_w_q, float* grad_w_k, float* grad_w_v,
                           void* bwd_workspace, size_t bwd_ws_bytes, uint32_t flags);

/*
 * Padded neighbour lists, built on the GPU: the list that the attention
 * streams (write-up section 3.2: padded slots plus a mask, masked slots
 * skipped; section 5.1: the edge cutoff).  The pages leave the list itself
 * open; this is the definition the library implements:
 *   - the neighbours of atom i are the atoms j != i with d2_ij < cutoff^2,
 *     where d2_ij = (dx*dx + dy*dy) + dz*dz with (dx, dy, dz) = pos_i - pos_j,
 *     all in float64 from the float32 positions, every operation rounded
 *     once (no fused multiply-add), cutoff^2 = cutoff * cutoff in float64
 *     (a strict cutoff; open boundaries: no periodic images);
 *   - row i lists them by increasing (d2_ij, j) -- nearest first, equal
 *     distances by atom index -- and keeps the first K: slots [0, k_i) hold
 *     them with mask 1, k_i = min(K, count); slots [k_i, K) hold index -1
 *     and mask 0.
 * The rows are therefore unique (bit-reproducible), whatever order the
 * builder meets the candidates in.
 *
 * e2f_neighbour_workspace_bytes -- scratch bytes for N atoms (cell grid,
 * grouped atoms and their positions: about 24 N bytes plus the cell
 * table); 0 when N < 0 or N > 2^30.
 */
size_t e2f_neighbour_workspace_bytes(int64_t N);

/*
 * e2f_neighbour_list -- build the rows above with a cell list: cells no
 * smaller than the cutoff, numbered in Morton order; atoms grouped by cell;
 * one wavefront per target scans the 27 cells around its own.
 *   cutoff     > 0, finite (angstrom, like the positions); E2F_ERR_SHAPE
 *              otherwise
 *   pos        [N, 3] fp32 device array
 *   nbr_idx    [N, K] int32 (written)
 *   nbr_mask   [N, K] uint8 (written)
 *   n_within   [N] int32 or NULL: the count before truncation to K
 *   order      [N] int32 or NULL: every atom once, grouped by cell in
 *              Morton order of the cells (a spatially coherent ordering;
 *              the order within a cell is unspecified)
 *   workspace  device scratch of e2f_neighbour_workspace_bytes(N)
 * K ranges over 1..1984 (E2F_ERR_SHAPE below, E2F_ERR_UNSUPPORTED above);
 * N over 0..2^30.  Outputs may not overlap each other, pos or the workspace.
 */
int e2f_neighbour_list(hipStream_t stream, int64_t N, int K, double cutoff, const float* pos,
                       int32_t* nbr_idx, uint8_t* nbr_mask, int32_t* n_within, int32_t* order,
                       void* workspace, size_t ws_bytes);

/*
 * e2f_frames -- test hook: the alignment rotation Q (Q r_hat = z_hat, write-up
 * section 2.1) and the Wigner-D blocks D^l(Q), l = 0..lmax, exactly as the
 * kernels build them.
 *   r [n, 3] fp32; Q [n, 9] fp32 row-major; D [n, 35] fp32: the blocks
 *   D^0 (1), D^1 (3x3), D^2 (5x5) row-major one after another (blocks
 *   above lmax are left untouched).
 */
int e2f_frames(hipStream_t stream, int64_t n, int lmax, const float* r, float* Q, float* D);

#ifdef __cplusplus
}
#endif

#endif /* E2F_H_ */
