/*
 * addrms.h -- C ABI of the RMSNorm / fused residual-Add + RMSNorm library
 * (with LayerNorm variants) for AMD Instinct MI355X (gfx950).
 *
 * Operations (the pages name them; the formula is the textbook RMSNorm,
 * Zhang & Sennrich 2019, with eps inside the square root):
 *   - RMSNorm, an op of the "Machete" README ("Built-In Areas"), and the
 *     fused residual Add + RMSNorm of KernelAgent-Oink (KernelAgent
 *     repository digest, opening summary):
 *         h      = x                                    (rmsnorm_fwd)
 *         h      = residual_out = round(fp32(x) + fp32(r))   (add_rmsnorm_fwd)
 *         rstd_i = 1 / sqrt(mean_j(h_ij^2) + eps)
 *         y_ij   = round(h_ij * rstd_i * w_j)
 *     The fused op normalises the residual exactly as it is stored, so its y
 *     equals rmsnorm_fwd applied to residual_out, bit for bit (with the
 *     kernel variants the library chooses; the tuning knobs below can force
 *     variants whose sums round differently).
 *   - The backward the Machete README's autograd helpers ("Built-In Areas")
 *     imply, the exact derivative given the saved rstd:
 *         g = dy * w,  xh = x * rstd_i,  c_i = mean_j(g_ij * xh_ij)
 *         dx_ij = round(rstd_i * (g_ij - xh_ij * c_i))
 *         dw_j  = sum_i dy_ij * xh_ij                    (overwritten)
 *
 * Arithmetic: float32 throughout on the GPU; each output is rounded once to
 * its storage type, round-to-nearest-even.  The residual add is a float32 add.
 * A row's sums (and dw's column sums) are float32 sums in an order that
 * follows the launch shape, which the library picks from N and M: the last
 * bit of y, dx, dw and db can differ between batch sizes or tuning knobs,
 * never beyond the tolerances the results are tested to.  The same call on
 * the same shape returns the same bits every time (dw included).
 * Storage types (dtype for the matrices, w_dtype for the weights, chosen
 * independently): ADDRMS_F32, ADDRMS_BF16, ADDRMS_F16.  A float16 result
 * beyond its range (65504) is infinite, as a float16 store rounds it.
 *
 * Layout: every matrix is row-major and contiguous, M rows of N elements
 * (row stride N).  w, dw have N elements; rstd has M.
 *
 * Memory and streams: every pointer argument is a DEVICE pointer.  The
 * caller owns every buffer, including the backward's workspace; the library
 * allocates nothing and keeps no per-call state.  Work is enqueued on
 * `stream` (a hipStream_t; NULL is the null stream) and the call returns
 * without synchronising.  A device fault surfaces at the caller's next
 * synchronisation, not in the return code.
 *
 * Alignment: any.  When every matrix pointer and w are 16-byte aligned and a
 * row is a multiple of 16 bytes, 128-bit vector loads/stores are used;
 * otherwise an element-wise path gives the same results.
 *
 * Aliasing: an output may be exactly the same buffer as an input of the same
 * shape (y == x; residual_out == r or x; dx == dy or x; dh == dy, dres or h).
 * Any other overlap
 * between an output and any other argument is ADDRMS_ERR_ALIAS.
 *
 * Errors: arguments are validated before any HIP call; on error nothing is
 * launched.  M == 0 is valid: the matrices and rstd may then be NULL, the
 * forward launches nothing, and the backward only writes dw = 0.  Calls are
 * thread-safe.
 */
#ifndef ADDRMS_H
#define ADDRMS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define ADDRMS_F32 0  /* IEEE binary32 */
#define ADDRMS_BF16 1 /* bfloat16: the upper 16 bits of a binary32 */
#define ADDRMS_F16 2  /* IEEE binary16 (half precision) */

/* Status codes: 0 on success, negative on error. */
#define ADDRMS_OK 0
#define ADDRMS_ERR_NULL -1      /* a required pointer is NULL */
#define ADDRMS_ERR_SHAPE -2     /* M < 0, N <= 0, or M*N too large */
#define ADDRMS_ERR_DTYPE -3     /* unknown element type code */
#define ADDRMS_ERR_EPS -4       /* eps negative, NaN or infinite */
#define ADDRMS_ERR_ALIAS -5     /* forbidden overlap between buffers */
#define ADDRMS_ERR_WORKSPACE -6 /* workspace NULL or smaller than required */
#define ADDRMS_ERR_HIP -7       /* a HIP call failed; see addrms_last_hip_error() */
#define ADDRMS_ERR_SCRATCH -8   /* a row is wider than rmsnorm_bwd_noalloc's scratch holds */
#define ADDRMS_ERR_KNOB -9      /* unknown tuning knob (addrms_tune) */

/*
 * RMSNorm forward.
 *   x     [M, N] dtype        input
 *   w     [N]    w_dtype      per-column scale, multiplied as stored
 *   y     [M, N] dtype        output; may be x itself
 *   rstd  [M]    float32      optional output (NULL: not written); the
 *                             rstd_i used, for the backward
 *   eps   >= 0, finite
 */
int rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd, int64_t M, int64_t N,
                float eps, int dtype, int w_dtype, void *stream);

/*
 * Fused residual-Add + RMSNorm forward (KernelAgent-Oink's fused op).
 *   x, r          [M, N] dtype  inputs (x may equal r)
 *   w             [N]    w_dtype
 *   y             [M, N] dtype  output RMSNorm(residual_out) * w; may be x or r
 *   residual_out  [M, N] dtype  output round(fp32(x) + fp32(r)); may be x or r
 *                               (in-place residual update); must not be y
 *   rstd          [M]    float32 optional output (NULL: not written)
 */
int add_rmsnorm_fwd(const void *x, const void *r, const void *w, void *y, void *residual_out,
                    float *rstd, int64_t M, int64_t N, float eps, int dtype, int w_dtype,
                    void *stream);

/*
 * Workspace, in bytes, that rmsnorm_bwd needs for these sizes: the float32
 * per-workgroup partial sums of dw, min(M, 1024) rows of N.  Pure arithmetic,
 * no HIP call.  Returns 0 for M <= 0 or N <= 0 (and for sizes whose byte count
 * does not fit in size_t).
 */
size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N);

/*
 * RMSNorm backward from the saved rstd.
 *   dy    [M, N] dtype     upstream gradient
 *   x     [M, N] dtype     forward input
 *   w     [N]    w_dtype
 *   rstd  [M]    float32   saved by the forward (required)
 *   dx    [M, N] dtype     output; may be dy or x
 *   dw    [N]    float32   output, overwritten (not accumulated)
 *   workspace              device scratch of >= rmsnorm_bwd_workspace_bytes(M, N)
 *                          bytes, any contents; clobbered; must not overlap
 *                          any other argument
 * dw's summation order is fixed by (M, N, device): repeated calls give
 * identical bits.
 */
int rmsnorm_bwd(const void *dy, const void *x, const void *w, const float *rstd, void *dx,
                float *dw, void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                int dtype, int w_dtype, void *stream);

/*
 * rmsnorm_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The dw partial sums live in a scratch array of
 * ADDRMS_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU it runs on, from the first call on that GPU until the process ends;
 * the call itself allocates nothing.  It uses as many partial rows as fit
 * (min(M, 1024, scratch / (4 N)) of them), so dx is the same as rmsnorm_bwd's
 * and dw differs from it only in summation order when N > 4096.
 *   Arguments, layout, aliasing and errors as rmsnorm_bwd, without the
 *   workspace; N above ADDRMS_NOALLOC_SCRATCH_BYTES / 4 is
 *   ADDRMS_ERR_SCRATCH.
 * Every call on one GPU shares that GPU's scratch (nothing in it needs to
 * start at zero): calls that may overlap on one GPU, from several streams or
 * threads, race on it and must be serialised by the caller.
 */
#define ADDRMS_NOALLOC_SCRATCH_BYTES (16u << 20)

int rmsnorm_bwd_noalloc(const void *dy, const void *x, const void *w, const float *rstd, void *dx,
                        float *dw, int64_t M, int64_t N, int dtype, int w_dtype, void *stream);

/*
 * Backward of the fused residual-Add + RMSNorm (KernelAgent-Oink's fused op;
 * the Machete README's autograd helpers, "Built-In Areas").  The forward
 * normalised h = residual_out and also returned it, so the gradient reaching
 * h is the RMSNorm backward of dy plus the gradient of residual_out; since
 * h = x + r, that one tensor is the gradient of both x and r:
 *     dh_ij = round(rstd_i * (g_ij - hh_ij * c_i) + dres_ij),
 *     g = dy * w,  hh = h * rstd_i,  c_i = mean_j(g_ij * hh_ij),
 *     dw_j  = sum_i dy_ij * hh_ij                       (overwritten)
 * (the rounding of the stored residual is treated as the identity).
 *   dy    [M, N] dtype     gradient of y
 *   dres  [M, N] dtype     gradient of residual_out; NULL means zero (then
 *                          this equals rmsnorm_bwd with x = h)
 *   h     [M, N] dtype     residual_out saved by the forward
 *   w     [N]    w_dtype
 *   rstd  [M]    float32   saved by the forward (required)
 *   dh    [M, N] dtype     output; may be dy, dres or h
 *   dw    [N]    float32   output, overwritten
 *   workspace              as for rmsnorm_bwd (same size function)
 */
int add_rmsnorm_bwd(const void *dy, const void *dres, const void *h, const void *w,
                    const float *rstd, void *dh, float *dw, void *workspace,
                    size_t workspace_bytes, int64_t M, int64_t N, int dtype, int w_dtype,
                    void *stream);

/*
 * RMSNorm / fused Add + RMSNorm with an FP8 output for a downstream FP8 GEMM
 * (the norm followed by the quantised epilogue; the "Machete" README's
 * "Built-In Areas" lists MXFP4 decode kernels, i.e. low-precision
 * activations after the norm).  y is computed as in rmsnorm_fwd /
 * add_rmsnorm_fwd in float32 but not stored; per row:
 *     amax_i  = max_j |y_ij|        (NaNs ignored)
 *     scale_i = amax_i / 448        (float32; 1 when amax_i = 0)
 *     q_ij    = E4M3(clamp(y_ij / scale_i, -448, 448))
 * (computed as y_ij * (448 / amax_i) in float32, which agrees with the
 * quotient to about 1e-6 relative)
 * E4M3 is the OCP 8-bit float with 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, largest value 448 (torch.float8_e4m3fn), rounded to nearest
 * even; y_ij ~= decode(q_ij) * scale_i.
 *   y_fp8    [M, N]  uint8    output E4M3 codes; must not overlap anything
 *   y_scale  [M]     float32  output per-row scale
 * Other arguments as rmsnorm_fwd / add_rmsnorm_fwd (residual_out is still
 * written in the input dtype).
 */
int rmsnorm_fwd_fp8(const void *x, const void *w, void *y_fp8, float *y_scale, float *rstd,
                    int64_t M, int64_t N, float eps, int dtype, int w_dtype, void *stream);

int add_rmsnorm_fwd_fp8(const void *x, const void *r, const void *w, void *y_fp8, float *y_scale,
                        void *residual_out, float *rstd, int64_t M, int64_t N, float eps,
                        int dtype, int w_dtype, void *stream);

/*
 * The same with one scale per group of `group` consecutive columns of a row
 * (per-block scales for an FP8 GEMM that scales activations per token and
 * per channel block, e.g. group = 128); the last group of a row may be
 * shorter.  For row i and group g (columns g*group .. min(N, (g+1)*group)-1):
 *     amax_ig = max |y_ij| over the group (NaNs ignored)
 *     scale_ig = amax_ig / 448  (1 when amax_ig = 0)
 *     q_ij = E4M3(clamp(y_ij / scale_ig, -448, 448))
 *   y_scale  [M][ceil(N / group)]  float32  output, row-major
 * group >= 1 (ADDRMS_ERR_SHAPE otherwise); group >= N gives one scale per
 * row, as rmsnorm_fwd_fp8.  The vector path takes groups of a power of two
 * of 16-byte vectors up to 64 (bf16: 8 .. 512 columns; float32: 4 .. 256);
 * other group sizes take the element-wise path with the same results.
 */
int rmsnorm_fwd_fp8_grouped(const void *x, const void *w, void *y_fp8, float *y_scale,
                            int64_t group, float *rstd, int64_t M, int64_t N, float eps, int dtype,
                            int w_dtype, void *stream);

int add_rmsnorm_fwd_fp8_grouped(const void *x, const void *r, const void *w, void *y_fp8,
                                float *y_scale, int64_t group, void *residual_out, float *rstd,
                                int64_t M, int64_t N, float eps, int dtype, int w_dtype,
                                void *stream);

/*
 * RMSNorm / fused Add + RMSNorm with an MXFP4 output (the "Machete" README's
 * "Built-In Areas" lists MXFP4 decode kernels; the format is OCP Microscaling
 * Formats v1.0 MXFP4).  y is computed as in rmsnorm_fwd / add_rmsnorm_fwd in
 * float32 but not stored.  For each block of 32 consecutive values of a row
 * (the last block may be shorter):
 *     a NaN in the block:  scale byte 0xFF (NaN), codes 0
 *     otherwise:           E = floor(log2(max |y|)) - 2, clamped below at -127
 *                          (an all-zero block has E = -127)
 *                          scale byte = E + 127 (E8M0: the scale is 2^E)
 *                          q_j = E2M1(y_j / 2^E)
 * E2M1 is the 4-bit float (sign, 2 exponent bits, 1 mantissa bit) with the
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, rounded to nearest with ties to the
 * even code and saturating at 6; y_j ~= decode(q_j) * 2^E.
 *   y_fp4    [M, N/2]         uint8  output, two codes per byte, element 2i
 *                                    in the low nibble; N must be even
 *   y_scale  [M, ceil(N/32)]  uint8  output E8M0 scale bytes
 * Other arguments as rmsnorm_fwd / add_rmsnorm_fwd (residual_out is still
 * written in the input dtype).
 */
int rmsnorm_fwd_mxfp4(const void *x, const void *w, void *y_fp4, void *y_scale, float *rstd,
                      int64_t M, int64_t N, float eps, int dtype, int w_dtype, void *stream);

int add_rmsnorm_fwd_mxfp4(const void *x, const void *r, const void *w, void *y_fp4,
                          void *y_scale, void *residual_out, float *rstd, int64_t M, int64_t N,
                          float eps, int dtype, int w_dtype, void *stream);

/*
 * LayerNorm variants.  The "CuTe DSL" skill page lists a CTA-level LayerNorm
 * example (Workflow 0, example index) and names LayerNorm beside RMSNorm in
 * its float32 reduction pattern (Workflow 0); the formula is the textbook one
 * (Ba, Kiros & Hinton 2016), biased variance, eps inside the square root:
 *     mean_i = mean_j(h_ij),  rstd_i = 1 / sqrt(mean_j((h_ij - mean_i)^2) + eps)
 *     y_ij   = round((h_ij - mean_i) * rstd_i * w_j + b_j)
 * with h = x (layernorm_fwd) or h = residual_out = round(fp32(x) + fp32(r))
 * (add_layernorm_fwd, as add_rmsnorm_fwd).  The variance is taken about the
 * mean (two passes over the row held in registers), not as E[h^2] - mean^2.
 *   b           [N]  w_dtype  bias; NULL for none
 *   mean, rstd  [M]  float32  optional outputs (NULL: not written)
 * Other arguments, aliasing and errors as for the RMSNorm calls.
 */
int layernorm_fwd(const void *x, const void *w, const void *b, void *y, float *mean, float *rstd,
                  int64_t M, int64_t N, float eps, int dtype, int w_dtype, void *stream);

int add_layernorm_fwd(const void *x, const void *r, const void *w, const void *b, void *y,
                      void *residual_out, float *mean, float *rstd, int64_t M, int64_t N,
                      float eps, int dtype, int w_dtype, void *stream);

/* Workspace for layernorm_bwd: dw and db partial sums, twice
 * rmsnorm_bwd_workspace_bytes(M, N).  Pure arithmetic, no HIP call. */
size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N);

/*
 * LayerNorm backward from the saved mean and rstd (both required):
 *     xh = (x - mean_i) * rstd_i,  g = dy * w
 *     dx = round(rstd_i * (g - mean_j(g) - xh * mean_j(g * xh)))
 *     dw_j = sum_i dy_ij * xh_ij,  db_j = sum_i dy_ij    (overwritten)
 *   db    [N] float32  output; NULL when there is no bias
 *   workspace          >= layernorm_bwd_workspace_bytes(M, N) bytes
 * Other arguments, aliasing (dx may be dy or x) and errors as rmsnorm_bwd.
 */
int layernorm_bwd(const void *dy, const void *x, const void *w, const float *mean,
                  const float *rstd, void *dx, float *dw, float *db, void *workspace,
                  size_t workspace_bytes, int64_t M, int64_t N, int dtype, int w_dtype,
                  void *stream);

/*
 * Backward of add_layernorm_fwd, as add_rmsnorm_bwd is for add_rmsnorm_fwd:
 *     dh = round(rstd_i * (g - mean_j(g) - hh * mean_j(g * hh)) + dres)
 * with hh = (h - mean_i) * rstd_i; dh is the gradient of both x and r.
 *   dres  [M, N] dtype  gradient of residual_out; NULL means zero
 *   h     [M, N] dtype  residual_out saved by the forward
 *   dh    [M, N] dtype  output; may be dy, dres or h
 * Other arguments as layernorm_bwd.
 */
int add_layernorm_bwd(const void *dy, const void *dres, const void *h, const void *w,
                      const float *mean, const float *rstd, void *dh, float *dw, float *db,
                      void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype,
                      int w_dtype, void *stream);

/*
 * Per-head RMSNorm followed by the rotary position embedding, for the query
 * and key heads of an attention layer, in one pass.  The "Machete" README
 * lists RMSNorm and RoPE side by side among the ops its persistent kernels
 * compose ("Built-In Areas"); RoPE is the rotation of RoFormer (Su et al.
 * 2021).  For every token t and every head (Hq query heads, then Hk key
 * heads) of D values x:
 *     rstd  = 1 / sqrt(mean_j(x_j^2) + eps)
 *     n_j   = x_j * rstd * w_j              (w = wq for query heads, wk for key heads)
 *     p     = pos[t];  c_i = cos[p][i],  s_i = sin[p][i],  i < D/2
 *     pair i = (n_i, n_{i+D/2})   interleaved == 0 (rotate-half layout)
 *            = (n_{2i}, n_{2i+1}) interleaved != 0
 *     (a, b) -> (round(a*c_i - b*s_i), round(b*c_i + a*s_i))
 * in float32, one rounding per output.  A position outside [0, P) has no
 * table row: that token's heads are written as NaN (nothing outside the
 * tables is read).
 *   q      [T][Hq][D]  dtype    head h of token t at q + t*q_stride + h*D
 *   k      [T][Hk][D]  dtype    likewise with k_stride (Hk may be 0, k NULL)
 *   wq, wk [D]         w_dtype  per-dimension norm weights
 *   cos, sin [P][D/2]  float32  rotary tables, row p for position p
 *   pos    [T]         int64    token positions
 *   q_out, k_out                outputs laid out as q, k with their own strides
 * Strides are in elements (at least Hq*D, resp. Hk*D), so q and k may be
 * views into one packed projection output.  D must be even.  q_out may be q
 * (same stride) and k_out may be k, which updates a packed buffer in place;
 * no other overlap of an output with any argument is allowed (query and key
 * heads interleaved in one buffer do not overlap).  T == 0 or Hq + Hk == 0
 * launches nothing and the pointers may be NULL.  The 16-byte vector path
 * needs D = 2*E*G for G in {1, 2, 4, ..., 64} (E = 8 bf16, 4 float32 values
 * per vector: D = 128 bf16 uses G = 8 lanes per head), 16-byte aligned
 * pointers and token strides that are a multiple of 16 bytes; any other even
 * D or alignment takes an element-wise path with the same results.
 */
int rmsnorm_rope_qk(const void *q, const void *k, const void *wq, const void *wk,
                    const float *cos, const float *sin, const int64_t *pos, int64_t P, void *q_out,
                    void *k_out, int64_t T, int64_t Hq, int64_t Hk, int64_t D, int64_t q_stride,
                    int64_t k_stride, int64_t q_out_stride, int64_t k_out_stride, float eps,
                    int interleaved, int dtype, int w_dtype, void *stream);

/* Static, human-readable name of a status code. */
const char *addrms_status_str(int status);

/*
 * Tuning knobs of the dispatcher: which kernel variant and grid a call uses.
 * 0 means the measured default.  Every knob starts from the environment
 * variable named beside it, read once when the library is loaded, and
 * addrms_tune changes it for the whole process (all threads and devices)
 * from then on.  The knobs change only the summation order of row and
 * column sums (see Arithmetic above), and so at most the last bit of a
 * result; a forced variant that is not built for a shape falls back to the
 * default choice.
 *   FWD_WPR            forward waves per row (1, 2, 4, 8, 16)      ADDRMS_FWD_WPR
 *   FWD_VPL            forward target 16-byte vectors a lane       ADDRMS_FWD_VPL
 *   BWD_WPR            backward waves per row (1, 2, 4, 8)         ADDRMS_BWD_WPR
 *   BWD_WIDE           1: 1024-thread backward where built; 2: never   ADDRMS_BWD_WIDE
 *   BWD_PREFETCH       1: next-row prefetch backward where built; 2: never
 *                                                                  ADDRMS_BWD_PREFETCH
 *   FORCE_ELEM         1: the element-wise kernels                 ADDRMS_FORCE_ELEM
 *   MAX_PARTIALS       cap on dw partial rows (a larger workspace must be
 *                      passed than the size functions give)        ADDRMS_MAX_PARTIALS
 *   BLOCKS_PER_CU      persistent grid of this many blocks per CU (the
 *                      forward: instead of one block per row group) ADDRMS_BLOCKS_PER_CU
 *   ROPE_BLOCKS_PER_CU RMSNorm + RoPE grid cap, blocks per CU      ADDRMS_ROPE_BLOCKS_PER_CU
 *   ROPE_HPL           RMSNorm + RoPE heads per lane group and step (1, 2, 4)
 *                                                                  ADDRMS_ROPE_HPL
 */
#define ADDRMS_KNOB_FWD_WPR 0
#define ADDRMS_KNOB_FWD_VPL 1
#define ADDRMS_KNOB_BWD_WPR 2
#define ADDRMS_KNOB_BWD_WIDE 3
#define ADDRMS_KNOB_BWD_PREFETCH 4
#define ADDRMS_KNOB_FORCE_ELEM 5
#define ADDRMS_KNOB_MAX_PARTIALS 6
#define ADDRMS_KNOB_BLOCKS_PER_CU 7
#define ADDRMS_KNOB_ROPE_BLOCKS_PER_CU 8
#define ADDRMS_KNOB_ROPE_HPL 9
#define ADDRMS_NUM_KNOBS 10

/* Set knob `knob` to `value` (>= 0) and return its previous value; with
 * value < 0 only return the current value.  ADDRMS_ERR_KNOB for an unknown
 * knob.  No HIP call.  Calls already enqueued are not affected. */
int addrms_tune(int knob, int value);

/* The hipError_t of the last ADDRMS_ERR_HIP returned on this thread (0 if none). */
int addrms_last_hip_error(void);

/*
 * Launch plan: the kernel variant a call would take, for tools and tests.
 * Assumes contiguous tensors whose pointers are 16-byte aligned, a device of
 * `cus` compute units, and the tuning knobs as they stand.  No HIP call.
 * It does not repeat the calls' own argument checks: for a call they would
 * reject (MXFP4 output of an odd N, null, misaligned or overlapping
 * buffers) the plan describes nothing that runs.
 *   op       ADDRMS_PLAN_FWD (the forwards: rmsnorm_fwd, add_rmsnorm_fwd, the
 *            LayerNorm and quantised forms) or ADDRMS_PLAN_BWD (the backwards)
 *   norm     ADDRMS_PLAN_RMS or ADDRMS_PLAN_LAYER
 *   fused    1 for the residual-Add forms
 *   qmode    forward output: 0 plain, 1 E4M3 with one scale per row, 2 E4M3
 *            with one scale per `qgroup` columns, 3 MXFP4; 0 for the backward
 *   out      written on success:
 *     vector            1: a vector kernel, 0: the element-wise kernels
 *     waves_per_row     waves a row is spread over (vector kernels)
 *     vectors_per_lane  16-byte vectors each lane holds per tensor
 *     prefetch          backward: the next-row prefetch kernel
 *     wide              backward: 1024-thread blocks
 *     blocks_per_cu     backward: 2 when the persistent grid is held to 2
 *                       blocks per CU, 0 when it takes the blocks that fit
 * Returns ADDRMS_OK, or ADDRMS_ERR_NULL (out), ADDRMS_ERR_DTYPE,
 * ADDRMS_ERR_SHAPE (M < 1, N < 1, cus < 1, qgroup < 0, an unknown op, norm or
 * qmode, or a quantised output asked of a backward or a LayerNorm).
 */
#define ADDRMS_PLAN_FWD 0
#define ADDRMS_PLAN_BWD 1
#define ADDRMS_PLAN_RMS 0
#define ADDRMS_PLAN_LAYER 1
typedef struct {
    int vector;
    int waves_per_row;
    int vectors_per_lane;
    int prefetch;
    int wide;
    int blocks_per_cu;
} addrms_plan_t;
int addrms_plan(int op, int norm, int fused, int qmode, int64_t qgroup, int64_t M, int64_t N,
                int dtype, int w_dtype, int cus, addrms_plan_t *out);

#ifdef __cplusplus
}
#endif

#endif /* ADDRMS_H */
