/*
 * CPU oracle for row-wise RMSNorm and fused residual-Add + RMSNorm,
 * forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it; the GPU
 * library never includes, links or calls it, and it shares no code with it.
 *
 * What it computes.  The pages name the operations but print no formula:
 *   - "Machete" README, section "Built-In Areas": an RMSNorm op, plus
 *     autograd helpers (so a backward exists);
 *   - KernelAgent repository digest, opening summary: KernelAgent-Oink's
 *     RMSNorm and fused Add + RMSNorm custom operators;
 *   - "CuTe DSL" skill page, Workflow 0: RMSNorm is a float32 row reduction.
 * The formula is the textbook one (Zhang & Sennrich 2019, "Root Mean Square
 * Layer Normalization"), eps inside the square root:
 *
 *   h      = x                       (plain)
 *   h      = stored(fp32(x) + fp32(r))  (fused; the residual as stored)
 *   rstd_i = 1 / sqrt( (1/N) * sum_j h_ij^2 + eps )
 *   y_ij   = h_ij * rstd_i * w_j
 *
 * and its exact derivative for the backward, given the saved rstd:
 *
 *   g_ij  = dy_ij * w_j,   xh_ij = x_ij * rstd_i
 *   c_i   = (1/N) * sum_j g_ij * xh_ij
 *   dx_ij = rstd_i * (g_ij - xh_ij * c_i)
 *   dw_j  = sum_i dy_ij * xh_ij
 *
 * Every sum and product is in IEEE binary64, left to right.  Each output is
 * rounded once, from binary64, to its storage type with round-to-nearest,
 * ties-to-even.  The one deliberate exception is the residual add of the
 * fused op for float32/bfloat16 inputs: it is a binary32 add (both operands
 * widened exactly to float32, one RNE rounding), and the residual is then
 * rounded to its storage type; the normalised value h is that stored
 * residual.  For binary64 inputs the add is a binary64 add.
 *
 * LayerNorm (the "CuTe DSL" skill page lists a CTA-level LayerNorm example
 * in Workflow 0's example index and names LayerNorm beside RMSNorm in its
 * reduction pattern) is the textbook one (Ba, Kiros & Hinton 2016), with the
 * biased variance and eps inside the square root:
 *
 *   mean_i = (1/N) * sum_j h_ij
 *   var_i  = (1/N) * sum_j (h_ij - mean_i)^2
 *   rstd_i = 1 / sqrt(var_i + eps)
 *   y_ij   = (h_ij - mean_i) * rstd_i * w_j + b_j       (b optional)
 *
 * with the same choice of h for the fused residual variant, and backward
 *
 *   xh = (x - mean) * rstd,  g = dy * w
 *   dx = rstd * (g - mean_j(g) - xh * mean_j(g * xh))
 *   dw = sum_i dy * xh,      db = sum_i dy
 *
 * Element types (codes): 0 = float32, 1 = bfloat16 (raw uint16 bits),
 * 2 = float64, 3 = float16 (IEEE binary16, raw uint16 bits).  All arrays
 * are row-major and contiguous, row stride N.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2
#define OR_F16 3

#define OR_OK 0
#define OR_ERR_ARG -1
#define OR_ERR_NOMEM -2

/* ---- bfloat16 <-> binary64 ---------------------------------------------- */

/* A bfloat16 pattern is the upper half of a binary32 pattern; the value is
 * exact in binary64. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary64 value to bfloat16 (8 significant bits, binary32's
 * exponent range, subnormals kept), round-to-nearest ties-to-even, written
 * out from the definition: find the two neighbouring bfloat16 values lo <= |v|
 * < hi on the grid of spacing ulp, and pick by comparing with their midpoint.
 * NaN gives a quiet NaN with the sign kept; overflow gives +-Inf. */
uint16_t oracle_bf16_round(double v)
{
    const double bf16_max = 0x1.FEp127; /* largest finite bfloat16 */
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a, ulp, lo, hi, mid, q;
    float f;
    uint32_t u;

    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    a = fabs(v);
    if (isinf(v) || a >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);

    if (a < 0x1p-126) {
        ulp = 0x1p-133; /* subnormal spacing: 2^-126 / 2^7 */
    } else {
        int e;
        frexp(a, &e); /* a in [2^(e-1), 2^e) */
        ulp = ldexp(1.0, e - 8);
    }
    lo = floor(a / ulp) * ulp; /* exact: scaling by a power of two */
    hi = lo + ulp;
    mid = lo + 0.5 * ulp; /* exact: at most 10 significant bits */
    if (a < mid)
        q = lo;
    else if (a > mid)
        q = hi;
    else
        q = (fmod(lo / ulp, 2.0) == 0.0) ? lo : hi; /* tie: even significand */

    if (q > bf16_max)
        return (uint16_t)(sign | 0x7F80u);
    f = (float)q; /* exact: q is a bfloat16 value */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* binary32 pattern -> bfloat16 pattern, through the same single rounding. */
uint16_t oracle_bf16_from_f32_bits(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, sizeof f);
    return oracle_bf16_round((double)f);
}

/* Bulk form of oracle_bf16_round, for the converter's own checks. */
void oracle_bf16_round_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_round(v[i]);
}

/* ---- binary16 <-> binary64 (IEEE 754 binary16: 1 sign bit, 5 exponent
 * bits with bias 15, 10 fraction bits) ------------------------------------ */

/* The value of a binary16 pattern, exact in binary64: exponent field 0 is
 * the subnormal range fraction * 2^-24, field 31 is infinity (fraction 0) or
 * NaN, otherwise (1 + fraction / 2^10) * 2^(field - 15). */
double oracle_f16_bits_to_double(uint16_t b)
{
    const int sign = (b >> 15) & 1, field = (b >> 10) & 0x1F, frac = b & 0x3FF;
    double m;
    if (field == 31)
        m = frac ? NAN : INFINITY;
    else if (field == 0)
        m = ldexp((double)frac, -24);
    else
        m = ldexp(1.0 + (double)frac / 1024.0, field - 15);
    return sign ? -m : m;
}

/* Round a binary64 value to binary16, round-to-nearest ties-to-even, written
 * out from the definition as the bfloat16 rounding above: the neighbouring
 * binary16 values lo <= |v| < hi on the grid of spacing ulp (11 significant
 * bits; 2^-24 in the subnormal range below 2^-14), the midpoint decides, a
 * tie takes the even significand.  Beyond the largest finite value 65504 the
 * result is infinity (|v| >= 65520 rounds up past it).  NaN gives a quiet
 * NaN with the sign kept. */
uint16_t oracle_f16_round(double v)
{
    const double f16_max = 65504.0;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a, ulp, lo, hi, mid, q;

    if (isnan(v))
        return (uint16_t)(sign | 0x7E00u);
    a = fabs(v);
    if (isinf(v) || a >= 0x1p17)
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14) {
        ulp = 0x1p-24;
    } else {
        int e;
        frexp(a, &e); /* a in [2^(e-1), 2^e) */
        ulp = ldexp(1.0, e - 11);
    }
    lo = floor(a / ulp) * ulp;
    hi = lo + ulp;
    mid = lo + 0.5 * ulp;
    if (a < mid)
        q = lo;
    else if (a > mid)
        q = hi;
    else
        q = (fmod(lo / ulp, 2.0) == 0.0) ? lo : hi;

    if (q > f16_max)
        return (uint16_t)(sign | 0x7C00u);
    if (q < 0x1p-14) /* subnormal or zero: fraction = q / 2^-24 */
        return (uint16_t)(sign | (uint16_t)(q * 0x1p24));
    int e;
    const double m = frexp(q, &e); /* q = m * 2^e, m in [0.5, 1) */
    const int field = e - 1 + 15;
    const int frac = (int)((2.0 * m - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)(field << 10) | (uint16_t)frac);
}

/* Bulk forms, for the converter's own checks. */
void oracle_f16_round_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f16_round(v[i]);
}

void oracle_f16_decode_array(const uint16_t *b, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f16_bits_to_double(b[i]);
}

static int dtype_ok(int dt) { return dt == OR_F32 || dt == OR_BF16 || dt == OR_F64 || dt == OR_F16; }

static double load_elem(const void *p, int dt, int64_t i)
{
    switch (dt) {
    case OR_F32:
        return (double)((const float *)p)[i];
    case OR_BF16:
        return bf16_bits_to_double(((const uint16_t *)p)[i]);
    case OR_F16:
        return oracle_f16_bits_to_double(((const uint16_t *)p)[i]);
    default:
        return ((const double *)p)[i];
    }
}

/* One rounding from binary64 to the storage type (C's double->float
 * conversion is round-to-nearest-even in the default rounding mode). */
static void store_elem(void *p, int dt, int64_t i, double v)
{
    switch (dt) {
    case OR_F32:
        ((float *)p)[i] = (float)v;
        break;
    case OR_BF16:
        ((uint16_t *)p)[i] = oracle_bf16_round(v);
        break;
    case OR_F16:
        ((uint16_t *)p)[i] = oracle_f16_round(v);
        break;
    default:
        ((double *)p)[i] = v;
        break;
    }
}

/* ---- forward ------------------------------------------------------------ */

/* RMSNorm forward.  y = x * rstd * w row by row; rstd (nullable) receives
 * 1/sqrt(mean(x^2) + eps) per row, rounded to rstd_dt. */
int oracle_rmsnorm_fwd(const void *x, int x_dt, const void *w, int w_dt, void *y, int y_dt,
                       void *rstd, int rstd_dt, int64_t M, int64_t N, double eps)
{
    if (!x || !w || !y || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(x_dt) || !dtype_ok(w_dt) || !dtype_ok(y_dt) || (rstd && !dtype_ok(rstd_dt)))
        return OR_ERR_ARG;

    for (int64_t i = 0; i < M; i++) {
        double ss = 0.0;
        for (int64_t j = 0; j < N; j++) {
            double h = load_elem(x, x_dt, i * N + j);
            ss += h * h;
        }
        double ms = ss / (double)N;
        double rs = 1.0 / sqrt(ms + eps);
        if (rstd)
            store_elem(rstd, rstd_dt, i, rs);
        for (int64_t j = 0; j < N; j++) {
            double h = load_elem(x, x_dt, i * N + j);
            store_elem(y, y_dt, i * N + j, h * rs * load_elem(w, w_dt, j));
        }
    }
    return OR_OK;
}

/* The residual of every fused op: res = stored(x + r), n elements.  For
 * float32/bfloat16 inputs the add is binary32 (both operands widened exactly,
 * one RNE rounding), then one rounding to res_dt; binary64 inputs add in
 * binary64. */
static void residual_sum(const void *x, const void *r, int in_dt, void *res, int res_dt,
                         int64_t n)
{
    for (int64_t k = 0; k < n; k++) {
        double s;
        if (in_dt == OR_F64) {
            s = load_elem(x, in_dt, k) + load_elem(r, in_dt, k);
        } else {
            float xs = (float)load_elem(x, in_dt, k); /* exact widening */
            float rs = (float)load_elem(r, in_dt, k);
            float s32 = xs + rs; /* one binary32 RNE rounding */
            s = (double)s32;
        }
        store_elem(res, res_dt, k, s);
    }
}

/* Fused residual-Add + RMSNorm forward.  residual_out = stored(x + r), with
 * the add in binary32 for float32/bfloat16 inputs; then y is RMSNorm of the
 * stored residual (the residual as written is what gets normalised). */
int oracle_add_rmsnorm_fwd(const void *x, const void *r, int in_dt, const void *w, int w_dt,
                           void *y, int y_dt, void *res, int res_dt, void *rstd, int rstd_dt,
                           int64_t M, int64_t N, double eps)
{
    if (!x || !r || !w || !y || !res || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(in_dt) || !dtype_ok(res_dt))
        return OR_ERR_ARG;
    residual_sum(x, r, in_dt, res, res_dt, M * N);
    return oracle_rmsnorm_fwd(res, res_dt, w, w_dt, y, y_dt, rstd, rstd_dt, M, N, eps);
}

/* ---- backward ----------------------------------------------------------- */

/* Backward of the fused op.  The forward's normalised input is the stored
 * residual h = x + r, and the residual itself is also an output, so the
 * gradient reaching h is the RMSNorm backward of dy plus the gradient of the
 * residual output, dres (NULL: zero).  Because h = x + r, that one tensor
 * dh is the gradient of both x and r:
 *   dh_ij = rstd_i * (g_ij - xh_ij * c_i) + dres_ij,   one rounding,
 * with g, xh, c as for RMSNorm (x replaced by h); dw as for RMSNorm.
 * (The rounding of the stored residual is treated as the identity, as
 * autograd through a bf16 add does.) */
int oracle_add_rmsnorm_bwd(const void *dy, const void *dres, const void *h, int in_dt,
                           const void *w, int w_dt, const void *rstd, int rstd_dt, void *dh,
                           int dh_dt, void *dw, int dw_dt, double *dw_abs, int64_t M, int64_t N)
{
    double *acc, *acc_abs;

    if (!dy || !h || !w || !rstd || !dh || !dw || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(in_dt) || !dtype_ok(w_dt) || !dtype_ok(rstd_dt) || !dtype_ok(dh_dt) ||
        !dtype_ok(dw_dt))
        return OR_ERR_ARG;

    acc = (double *)calloc((size_t)N, sizeof(double));
    acc_abs = (double *)calloc((size_t)N, sizeof(double));
    if (!acc || !acc_abs) {
        free(acc);
        free(acc_abs);
        return OR_ERR_NOMEM;
    }

    for (int64_t i = 0; i < M; i++) {
        double rs = load_elem(rstd, rstd_dt, i);
        double c = 0.0;
        for (int64_t j = 0; j < N; j++) {
            double g = load_elem(dy, in_dt, i * N + j) * load_elem(w, w_dt, j);
            double xh = load_elem(h, in_dt, i * N + j) * rs;
            c += g * xh;
        }
        c /= (double)N;
        for (int64_t j = 0; j < N; j++) {
            double d = load_elem(dy, in_dt, i * N + j);
            double g = d * load_elem(w, w_dt, j);
            double xh = load_elem(h, in_dt, i * N + j) * rs;
            double extra = dres ? load_elem(dres, in_dt, i * N + j) : 0.0;
            store_elem(dh, dh_dt, i * N + j, rs * (g - xh * c) + extra);
            acc[j] += d * xh;
            acc_abs[j] += fabs(d * xh);
        }
    }
    for (int64_t j = 0; j < N; j++) {
        store_elem(dw, dw_dt, j, acc[j]);
        if (dw_abs)
            dw_abs[j] = acc_abs[j];
    }
    free(acc);
    free(acc_abs);
    return OR_OK;
}

/* RMSNorm backward from the saved rstd.  dx per row; dw = sum over rows of
 * dy * x * rstd, overwritten (not accumulated).  dw_abs (nullable, binary64)
 * receives sum over rows of |dy * x * rstd| per column, the magnitude that
 * bounds the rounding error of any summation order of dw.  It is the fused
 * op's backward with no residual gradient. */
int oracle_rmsnorm_bwd(const void *dy, const void *x, int in_dt, const void *w, int w_dt,
                       const void *rstd, int rstd_dt, void *dx, int dx_dt, void *dw, int dw_dt,
                       double *dw_abs, int64_t M, int64_t N)
{
    return oracle_add_rmsnorm_bwd(dy, NULL, x, in_dt, w, w_dt, rstd, rstd_dt, dx, dx_dt, dw, dw_dt,
                                  dw_abs, M, N);
}

/* ---- LayerNorm ---------------------------------------------------------- */

/* LayerNorm forward.  b, mean, rstd may be NULL; mean and rstd are rounded to
 * stat_dt. */
int oracle_layernorm_fwd(const void *x, int x_dt, const void *w, const void *b, int w_dt,
                         void *y, int y_dt, void *mean, void *rstd, int stat_dt, int64_t M,
                         int64_t N, double eps)
{
    if (!x || !w || !y || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(x_dt) || !dtype_ok(w_dt) || !dtype_ok(y_dt) || !dtype_ok(stat_dt))
        return OR_ERR_ARG;

    for (int64_t i = 0; i < M; i++) {
        double sum = 0.0, sq = 0.0;
        for (int64_t j = 0; j < N; j++)
            sum += load_elem(x, x_dt, i * N + j);
        double mu = sum / (double)N;
        for (int64_t j = 0; j < N; j++) {
            double d = load_elem(x, x_dt, i * N + j) - mu;
            sq += d * d;
        }
        double var = sq / (double)N;
        double rs = 1.0 / sqrt(var + eps);
        if (mean)
            store_elem(mean, stat_dt, i, mu);
        if (rstd)
            store_elem(rstd, stat_dt, i, rs);
        for (int64_t j = 0; j < N; j++) {
            double v = (load_elem(x, x_dt, i * N + j) - mu) * rs * load_elem(w, w_dt, j);
            if (b)
                v += load_elem(b, w_dt, j);
            store_elem(y, y_dt, i * N + j, v);
        }
    }
    return OR_OK;
}

/* Fused residual-Add + LayerNorm forward: residual_out = stored(x + r) (the
 * binary32 add of the RMSNorm variant), then LayerNorm of the stored residual. */
int oracle_add_layernorm_fwd(const void *x, const void *r, int in_dt, const void *w,
                             const void *b, int w_dt, void *y, int y_dt, void *res, int res_dt,
                             void *mean, void *rstd, int stat_dt, int64_t M, int64_t N,
                             double eps)
{
    if (!x || !r || !w || !y || !res || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(in_dt) || !dtype_ok(res_dt))
        return OR_ERR_ARG;
    residual_sum(x, r, in_dt, res, res_dt, M * N);
    return oracle_layernorm_fwd(res, res_dt, w, b, w_dt, y, y_dt, mean, rstd, stat_dt, M, N, eps);
}

/* Backward of the fused Add + LayerNorm from the saved mean and rstd: as for
 * RMSNorm, the gradient reaching the stored residual x (= h) is the
 * LayerNorm backward of dy plus dres (NULL: zero), and it is the gradient of
 * both inputs of the add.  db may be NULL.  dw_abs and db_abs (nullable,
 * binary64) receive the per-column sums of |dy * xh| and |dy|. */
int oracle_add_layernorm_bwd(const void *dy, const void *dres, const void *x, int in_dt,
                             const void *w, int w_dt, const void *mean, const void *rstd,
                             int stat_dt, void *dx, int dx_dt, void *dw, void *db, int dwb_dt,
                             double *dw_abs, double *db_abs, int64_t M, int64_t N)
{
    double *aw, *ab, *awa, *aba;

    if (!dy || !x || !w || !mean || !rstd || !dx || !dw || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(in_dt) || !dtype_ok(w_dt) || !dtype_ok(stat_dt) || !dtype_ok(dx_dt) ||
        !dtype_ok(dwb_dt))
        return OR_ERR_ARG;
    aw = (double *)calloc((size_t)N, sizeof(double));
    ab = (double *)calloc((size_t)N, sizeof(double));
    awa = (double *)calloc((size_t)N, sizeof(double));
    aba = (double *)calloc((size_t)N, sizeof(double));
    if (!aw || !ab || !awa || !aba) {
        free(aw);
        free(ab);
        free(awa);
        free(aba);
        return OR_ERR_NOMEM;
    }
    for (int64_t i = 0; i < M; i++) {
        double mu = load_elem(mean, stat_dt, i);
        double rs = load_elem(rstd, stat_dt, i);
        double mg = 0.0, mgx = 0.0;
        for (int64_t j = 0; j < N; j++) {
            double g = load_elem(dy, in_dt, i * N + j) * load_elem(w, w_dt, j);
            double xh = (load_elem(x, in_dt, i * N + j) - mu) * rs;
            mg += g;
            mgx += g * xh;
        }
        mg /= (double)N;
        mgx /= (double)N;
        for (int64_t j = 0; j < N; j++) {
            double d = load_elem(dy, in_dt, i * N + j);
            double g = d * load_elem(w, w_dt, j);
            double xh = (load_elem(x, in_dt, i * N + j) - mu) * rs;
            double extra = dres ? load_elem(dres, in_dt, i * N + j) : 0.0;
            store_elem(dx, dx_dt, i * N + j, rs * (g - mg - xh * mgx) + extra);
            aw[j] += d * xh;
            ab[j] += d;
            awa[j] += fabs(d * xh);
            aba[j] += fabs(d);
        }
    }
    for (int64_t j = 0; j < N; j++) {
        store_elem(dw, dwb_dt, j, aw[j]);
        if (db)
            store_elem(db, dwb_dt, j, ab[j]);
        if (dw_abs)
            dw_abs[j] = awa[j];
        if (db_abs)
            db_abs[j] = aba[j];
    }
    free(aw);
    free(ab);
    free(awa);
    free(aba);
    return OR_OK;
}

/* LayerNorm backward: the fused op's backward with no residual gradient. */
int oracle_layernorm_bwd(const void *dy, const void *x, int in_dt, const void *w, int w_dt,
                         const void *mean, const void *rstd, int stat_dt, void *dx, int dx_dt,
                         void *dw, void *db, int dwb_dt, double *dw_abs, double *db_abs,
                         int64_t M, int64_t N)
{
    return oracle_add_layernorm_bwd(dy, NULL, x, in_dt, w, w_dt, mean, rstd, stat_dt, dx, dx_dt,
                                    dw, db, dwb_dt, dw_abs, db_abs, M, N);
}

/* ---- FP8 (E4M3) output with a dynamic per-row scale ----------------------- */

/* OCP 8-bit float E4M3 (the "FN" variant: sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN; largest
 * finite value 1.75 * 2^8 = 448).  Encoding from binary64: round to nearest,
 * ties to even significand, on the E4M3 grid; saturating: finite values of
 * magnitude >= 448 and infinities give +-448; NaN gives S.1111.111. */
uint8_t oracle_fp8e4m3_encode(double v)
{
    const uint8_t sign = signbit(v) ? 0x80u : 0u;
    double a, ulp, lo, hi, mid, q;
    int e;

    if (isnan(v))
        return (uint8_t)(sign | 0x7Fu);
    a = fabs(v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7Eu); /* 448 = 1.110b * 2^8 */
    if (a < 0x1p-6) {
        ulp = 0x1p-9; /* subnormal spacing: 2^-6 / 2^3 */
    } else {
        frexp(a, &e); /* a in [2^(e-1), 2^e) */
        ulp = ldexp(1.0, e - 4);
    }
    lo = floor(a / ulp) * ulp;
    hi = lo + ulp;
    mid = lo + 0.5 * ulp;
    if (a < mid)
        q = lo;
    else if (a > mid)
        q = hi;
    else
        q = (fmod(lo / ulp, 2.0) == 0.0) ? lo : hi;

    if (q == 0.0)
        return sign;
    if (q < 0x1p-6) /* subnormal: exponent field 0, mantissa q / 2^-9 */
        return (uint8_t)(sign | (uint8_t)(q / 0x1p-9));
    frexp(q, &e); /* q = 1.mmm * 2^(e-1) */
    {
        int exp_field = (e - 1) + 7;
        int mant = (int)((ldexp(q, -(e - 1)) - 1.0) * 8.0);
        return (uint8_t)(sign | (uint8_t)(exp_field << 3) | (uint8_t)mant);
    }
}

/* E4M3 code -> exact binary64 value (NaN for S.1111.111). */
double oracle_fp8e4m3_decode(uint8_t c)
{
    const double sgn = (c & 0x80u) ? -1.0 : 1.0;
    const int ef = (c >> 3) & 0xF, m = c & 7;
    if (ef == 0xF && m == 7)
        return NAN;
    if (ef == 0)
        return sgn * ldexp((double)m, -9);
    return sgn * ldexp(1.0 + m / 8.0, ef - 7);
}

void oracle_fp8e4m3_encode_array(const double *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_fp8e4m3_encode(v[i]);
}

/* RMSNorm with an E4M3 output and dynamic scales, for a downstream FP8 GEMM.
 * The scales are per group of `group` consecutive columns of a row (the last
 * group of a row may be shorter); group <= 0 means one group per row.  Per
 * row: y_j = h_j * rstd * w_j in binary64; per group, by the definition of a
 * dynamic scale (the group's largest magnitude maps to E4M3's largest value,
 * 448) and of the codes relative to the scale the caller receives:
 *     amax  = max |y_j| over the group's columns      (binary64; NaNs ignored)
 *     scale = binary32(amax / 448)                     (the stored scale)
 *     q_j   = E4M3(y_j / scale)                        (binary64 quotient, one rounding)
 * with scale = 1 for a group with no non-zero finite |y| (a NaN encodes as
 * NaN).  y_j ~= decode(q_j) * scale of its group.  scale is
 * [M][ceil(N / group)], row-major. */
static size_t elem_size(int dt) { return dt == OR_F32 ? 4 : dt == OR_F64 ? 8 : 2; }

int oracle_rmsnorm_fwd_fp8_grouped(const void *x, int x_dt, const void *w, int w_dt, uint8_t *q,
                                   float *scale, int64_t group, void *rstd, int rstd_dt,
                                   int64_t M, int64_t N, double eps)
{
    double *y;

    if (!x || !w || !q || !scale || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(x_dt) || !dtype_ok(w_dt) || (rstd && !dtype_ok(rstd_dt)))
        return OR_ERR_ARG;
    if (group <= 0 || group > N)
        group = N;
    const int64_t ngroups = (N + group - 1) / group;
    y = (double *)malloc((size_t)N * sizeof(double));
    if (!y)
        return OR_ERR_NOMEM;
    for (int64_t i = 0; i < M; i++) {
        /* the row's RMSNorm in binary64, by the forward above */
        const void *xi = (const char *)x + (size_t)(i * N) * elem_size(x_dt);
        void *ri = rstd ? (void *)((char *)rstd + (size_t)i * elem_size(rstd_dt)) : NULL;
        oracle_rmsnorm_fwd(xi, x_dt, w, w_dt, y, OR_F64, ri, rstd_dt, 1, N, eps);
        for (int64_t g = 0; g < ngroups; g++) {
            const int64_t j0 = g * group, j1 = j0 + group < N ? j0 + group : N;
            double amax = 0.0;
            for (int64_t j = j0; j < j1; j++) {
                double m = fabs(y[j]);
                if (m > amax) /* NaN never compares greater: NaNs do not set the scale */
                    amax = m;
            }
            float sc = 1.0f;
            if (amax != 0.0)
                sc = (float)(amax / 448.0);
            scale[i * ngroups + g] = sc;
            for (int64_t j = j0; j < j1; j++)
                q[i * N + j] = oracle_fp8e4m3_encode(y[j] / (double)sc);
        }
    }
    free(y);
    return OR_OK;
}

/* One scale per row: the grouped form with a single group per row. */
int oracle_rmsnorm_fwd_fp8(const void *x, int x_dt, const void *w, int w_dt, uint8_t *q,
                           float *scale, void *rstd, int rstd_dt, int64_t M, int64_t N, double eps)
{
    return oracle_rmsnorm_fwd_fp8_grouped(x, x_dt, w, w_dt, q, scale, 0, rstd, rstd_dt, M, N, eps);
}

/* Fused residual-Add + RMSNorm with the E4M3 output: the residual as in
 * oracle_add_rmsnorm_fwd, then oracle_rmsnorm_fwd_fp8_grouped of the stored
 * residual (group <= 0: one scale per row). */
int oracle_add_rmsnorm_fwd_fp8_grouped(const void *x, const void *r, int in_dt, const void *w,
                                       int w_dt, uint8_t *q, float *scale, int64_t group,
                                       void *res, int res_dt, void *rstd, int rstd_dt, int64_t M,
                                       int64_t N, double eps)
{
    if (!x || !r || !res || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(in_dt) || !dtype_ok(res_dt))
        return OR_ERR_ARG;
    residual_sum(x, r, in_dt, res, res_dt, M * N);
    return oracle_rmsnorm_fwd_fp8_grouped(res, res_dt, w, w_dt, q, scale, group, rstd, rstd_dt, M,
                                          N, eps);
}

int oracle_add_rmsnorm_fwd_fp8(const void *x, const void *r, int in_dt, const void *w, int w_dt,
                               uint8_t *q, float *scale, void *res, int res_dt, void *rstd,
                               int rstd_dt, int64_t M, int64_t N, double eps)
{
    return oracle_add_rmsnorm_fwd_fp8_grouped(x, r, in_dt, w, w_dt, q, scale, 0, res, res_dt,
                                              rstd, rstd_dt, M, N, eps);
}

/* ---- per-head RMSNorm followed by RoPE ------------------------------------ */

/*
 * The composition of two ops the "Machete" README lists side by side in
 * "Built-In Areas" (RMSNorm, RoPE), as they meet in an attention layer: each
 * query or key head of each token is RMS-normalised over its D values with a
 * per-dimension weight w[D], then rotated by the token's position (rotary
 * position embedding, Su et al. 2021, "RoFormer"). The rotation acts on pairs
 * of normalised values:
 *
 *   rotate-half layout (interleaved = 0):  pair i = (n_i, n_{i+D/2})
 *   interleaved layout (interleaved = 1):  pair i = (n_{2i}, n_{2i+1})
 *   c = cos_t[p][i], s = sin_t[p][i], p = pos[t], i in [0, D/2)
 *   (a, b) -> (a*c - b*s, b*c + a*s)
 *
 * The tables are float32 [P][D/2], widened exactly to binary64. The norm is
 * oracle_rmsnorm_fwd of the head's row into binary64. The rotation is
 * binary64, and each output is rounded once. A position outside [0, P) has
 * no table row: that token's heads are all NaN.
 *
 * x: head h of token t starts at element t*x_stride + h*D (heads contiguous);
 * y: the same with y_stride.  T tokens, H heads, D even.
 */
int oracle_rmsnorm_rope(const void *x, int x_dt, int64_t x_stride, const void *w, int w_dt,
                        const float *cos_t, const float *sin_t, const int64_t *pos, int64_t P,
                        void *y, int y_dt, int64_t y_stride, int64_t T, int64_t H, int64_t D,
                        int interleaved, double eps)
{
    double *n;
    const int64_t half = D / 2;

    if (!x || !w || !cos_t || !sin_t || !pos || !y || T < 0 || H < 0 || D <= 0 || D % 2 != 0 ||
        P < 0 || x_stride < H * D || y_stride < H * D)
        return OR_ERR_ARG;
    if (!dtype_ok(x_dt) || !dtype_ok(w_dt) || !dtype_ok(y_dt))
        return OR_ERR_ARG;
    n = (double *)malloc((size_t)D * sizeof(double));
    if (!n)
        return OR_ERR_NOMEM;
    for (int64_t t = 0; t < T; t++) {
        const int64_t p = pos[t];
        for (int64_t h = 0; h < H; h++) {
            const int64_t xo = t * x_stride + h * D, yo = t * y_stride + h * D;
            if (p < 0 || p >= P) {
                for (int64_t j = 0; j < D; j++)
                    store_elem(y, y_dt, yo + j, NAN);
                continue;
            }
            const void *xh = (const char *)x + (size_t)xo * elem_size(x_dt);
            oracle_rmsnorm_fwd(xh, x_dt, w, w_dt, n, OR_F64, NULL, OR_F32, 1, D, eps);
            for (int64_t i = 0; i < half; i++) {
                const int64_t ja = interleaved ? 2 * i : i;
                const int64_t jb = interleaved ? 2 * i + 1 : i + half;
                const double c = (double)cos_t[p * half + i];
                const double s = (double)sin_t[p * half + i];
                const double a = n[ja], b = n[jb];
                store_elem(y, y_dt, yo + ja, a * c - b * s);
                store_elem(y, y_dt, yo + jb, b * c + a * s);
            }
        }
    }
    free(n);
    return OR_OK;
}

/* ---- MXFP4 output: E2M1 elements with a shared E8M0 scale per 32 ---------- */

/* FP4 E2M1 (OCP Microscaling Formats v1.0: sign, 2 exponent bits with bias 1,
 * 1 mantissa bit; no infinities or NaN).  Magnitudes of codes 0..7:
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Round to nearest on that grid, ties to the
 * even code; magnitudes above 6 saturate to 6 (the MX conversion clamps
 * normal values); the sign is kept, also for a zero result. */
static const double e2m1_grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

uint8_t oracle_fp4e2m1_encode(double v)
{
    const uint8_t sign = signbit(v) ? 0x8u : 0x0u;
    const double a = fabs(v);
    if (a >= 6.0)
        return (uint8_t)(sign | 0x7u);
    int k = 0;
    while (k < 7 && e2m1_grid[k + 1] <= a)
        k++; /* e2m1_grid[k] <= a < e2m1_grid[k + 1] */
    const double lo = e2m1_grid[k], hi = e2m1_grid[k + 1];
    const double mid = 0.5 * (lo + hi);
    int code;
    if (a < mid)
        code = k;
    else if (a > mid)
        code = k + 1;
    else
        code = (k % 2 == 0) ? k : k + 1; /* the even code */
    return (uint8_t)(sign | (uint8_t)code);
}

double oracle_fp4e2m1_decode(uint8_t c)
{
    const double m = e2m1_grid[c & 0x7u];
    return (c & 0x8u) ? -m : m;
}

/* RMSNorm with an MXFP4 output (OCP MX v1.0): per row, y_j = h_j * rstd * w_j
 * in binary64, rounded once to binary32 (yf_j); per block of 32 consecutive
 * columns (the last block of a row may be shorter):
 *     a block with a NaN:   scale code 0xFF (NaN), element codes 0
 *     otherwise:            amax = max |yf_j|
 *                           E = floor(log2(amax)) - 2, clamped to [-127, 127]
 *                           (E = -127 when amax is 0: the smallest scale)
 *                           scale code = E + 127 (E8M0), X = 2^E
 *                           q_j = E2M1(yf_j / X)       (exact division)
 * 2 is the exponent of E2M1's largest value (6 = 1.5 * 2^2), so the block's
 * largest magnitude lands in [4, 8) and values above 6 saturate.  Codes are
 * packed two per byte, element 2i in the low nibble: q [M][N/2] (N even);
 * scale [M][ceil(N/32)].  y_j ~= decode(q_j) * 2^(scale - 127). */
int oracle_rmsnorm_fwd_mxfp4(const void *x, int x_dt, const void *w, int w_dt, uint8_t *q,
                             uint8_t *scale, void *rstd, int rstd_dt, int64_t M, int64_t N,
                             double eps)
{
    double *y;
    float *yf;

    if (!x || !w || !q || !scale || M < 0 || N <= 0 || N % 2 != 0)
        return OR_ERR_ARG;
    if (!dtype_ok(x_dt) || !dtype_ok(w_dt) || (rstd && !dtype_ok(rstd_dt)))
        return OR_ERR_ARG;
    const int64_t nb = (N + 31) / 32;
    y = (double *)malloc((size_t)N * sizeof(double));
    yf = (float *)malloc((size_t)N * sizeof(float));
    if (!y || !yf) {
        free(y);
        free(yf);
        return OR_ERR_NOMEM;
    }
    for (int64_t i = 0; i < M; i++) {
        const void *xi = (const char *)x + (size_t)(i * N) * elem_size(x_dt);
        void *ri = rstd ? (void *)((char *)rstd + (size_t)i * elem_size(rstd_dt)) : NULL;
        oracle_rmsnorm_fwd(xi, x_dt, w, w_dt, y, OR_F64, ri, rstd_dt, 1, N, eps);
        for (int64_t j = 0; j < N; j++)
            yf[j] = (float)y[j];
        for (int64_t b = 0; b < nb; b++) {
            const int64_t j0 = b * 32, j1 = j0 + 32 < N ? j0 + 32 : N;
            int has_nan = 0;
            double amax = 0.0;
            for (int64_t j = j0; j < j1; j++) {
                if (isnan(yf[j]))
                    has_nan = 1;
                else if (fabs((double)yf[j]) > amax)
                    amax = fabs((double)yf[j]);
            }
            uint8_t codes[32];
            int E = -127;
            if (has_nan) {
                scale[i * nb + b] = 0xFF;
                for (int64_t j = j0; j < j1; j++)
                    codes[j - j0] = 0;
            } else {
                if (amax > 0.0) {
                    int e2;
                    frexp(amax, &e2); /* amax = f * 2^e2, f in [0.5, 1): floor(log2) = e2 - 1 */
                    E = (e2 - 1) - 2;
                    if (E < -127)
                        E = -127;
                    if (E > 127)
                        E = 127;
                }
                scale[i * nb + b] = (uint8_t)(E + 127);
                for (int64_t j = j0; j < j1; j++)
                    codes[j - j0] = oracle_fp4e2m1_encode(ldexp((double)yf[j], -E));
            }
            for (int64_t j = j0; j < j1; j += 2)
                q[(i * N + j) / 2] = (uint8_t)(codes[j - j0] | (codes[j + 1 - j0] << 4));
        }
    }
    free(y);
    free(yf);
    return OR_OK;
}

/* Fused residual-Add + RMSNorm with the MXFP4 output: the residual as in
 * oracle_add_rmsnorm_fwd, then oracle_rmsnorm_fwd_mxfp4 of the stored residual. */
int oracle_add_rmsnorm_fwd_mxfp4(const void *x, const void *r, int in_dt, const void *w, int w_dt,
                                 uint8_t *q, uint8_t *scale, void *res, int res_dt, void *rstd,
                                 int rstd_dt, int64_t M, int64_t N, double eps)
{
    if (!x || !r || !res || M < 0 || N <= 0)
        return OR_ERR_ARG;
    if (!dtype_ok(in_dt) || !dtype_ok(res_dt))
        return OR_ERR_ARG;
    residual_sum(x, r, in_dt, res, res_dt, M * N);
    return oracle_rmsnorm_fwd_mxfp4(res, res_dt, w, w_dt, q, scale, rstd, rstd_dt, M, N, eps);
}

void oracle_fp4e2m1_encode_array(const double *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_fp4e2m1_encode(v[i]);
}
