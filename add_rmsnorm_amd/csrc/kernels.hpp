// HIP kernels for gfx950 (CDNA4): RMSNorm, fused residual-Add + RMSNorm, and
// the LayerNorm variants, forward and backward.
//
// The operations are the RMSNorm and fused Add + RMSNorm ops named by the
// "Machete" README ("Built-In Areas") and the KernelAgent digest (the
// KernelAgent-Oink summary), and the LayerNorm that the "CuTe DSL" skill page
// lists beside RMSNorm (Workflow 0: the CTA-norm example and the reduction
// pattern).  The row reduction follows that page's float32 pattern (Workflow
// 0: per-thread loops, a butterfly within the warp, then a cross-warp step
// through shared memory), which here becomes per-lane FMAs, a DPP wave64 sum,
// and an LDS step only when several waves share a row.
//
// Memory traffic is the whole cost (a few VALU ops per 2-4 bytes moved), so
// the design is about HBM streaming, not arithmetic:
//   * each row is read once into registers with 128-bit loads (one wave64
//     covers 1 KiB per load instruction, fully coalesced), normalised from
//     registers, and written once: x, r read once; y, residual_out written
//     once;
//   * rows are spread over enough waves that each lane holds about two
//     16-byte vectors per tensor: many short, independent row-blocks keep the
//     most rows in flight (one LDS exchange per row sum when a row has several
//     waves; none when it has one);
//   * every kernel walks rows with a grid stride, so the same code serves a
//     one-block-per-row grid (the forward's default) and a persistent grid
//     sized to the device (the backward, whose blocks keep dw partial sums
//     in registers across the rows they visit).
#pragma once

#include <utility>

#include "device.hpp"
#include "internal.hpp"

namespace addrms {

// Cache policy of the streamed row data (see ld_stream / st_stream): rows are
// touched once, so loads and stores are non-temporal by default (measured on
// MI355X: a 2-read/2-write stream moves ~6.3 TB/s with both non-temporal
// versus ~5.5 TB/s with the default policy).
#ifndef ADDRMS_STREAM_POLICY
#define ADDRMS_STREAM_POLICY 3
#endif

constexpr int kPol = ADDRMS_STREAM_POLICY;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Arithmetic type of the backward's row reductions and dx.  float32 tensors
// use binary64: dx = rstd * (g - xh * c) cancels when xh * c is close to g
// (always so for very short rows), and the float32 products and sum would then
// leave too few correct bits for a float32 result.  bfloat16 tensors use
// float32.
template <typename T> struct BwdCompute { using type = float; };
template <> struct BwdCompute<float> { using type = double; };

// 1/N in the compute type.
template <typename CT> __device__ __forceinline__ CT inv_n_ct(int N) { return (CT)1 / (CT)N; }

__device__ __forceinline__ float fma_ct(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_ct(double a, double b, double c) { return __builtin_fma(a, b, c); }

// ---------------------------------------------------------------------------
// Forward, vector path.  WPR waves per row, VPL 16-byte vectors per lane:
// lane `l` of wave `q` (of the row's WPR waves) owns vectors
// v = q*64 + l + k*64*WPR, k < VPL.  Requires 16-byte aligned rows.
// NORM = kRms: y = h * rstd * w, rstd = 1/sqrt(mean(h^2) + eps).
// NORM = kLayer: y = (h - mean) * rstd * w (+ b), rstd = 1/sqrt(var + eps),
// the variance taken about the mean from the registers (two passes over the
// row, one over memory).
// QM != kQNone (RMSNorm only): y is not stored but quantised for a
// downstream low-precision GEMM.  kQRow / kQGroup: its absmax sets a scale
// (scale = amax/448, inv = 448/amax, binary32), per row or per group of
// a.qlanes consecutive vectors (a group maximum over that many lanes), and
// y * inv is written as OCP E4M3 codes, one byte per element.  kQMx: MXFP4,
// one E8M0 scale per 32 values and E2M1 codes, two per byte.
// ---------------------------------------------------------------------------
// Whether a forward vector kernel holds the weights of a lane's columns in
// registers, in their stored form, loaded once before the row loop so that
// their fetch overlaps the row's loads.  The quantised modes do (measured on
// MI355X, bf16, 2048 to 8192 columns: MXFP4 3-7 % and grouped E4M3 2.5-5 %
// faster): their output pass is longer and its per-vector weight loads sat
// on the critical path.  The other modes keep the registers for occupancy
// and load the weights at each use (holding them measured 6-11 % slower for
// the plain LayerNorm and up to 10 % slower at 512 rows of 8192), except the
// variant with 16 waves per row and one vector a lane, which serves batches
// too small to give every SIMD a wave: there the early fetch takes the weight
// load off the path after the row reduction (2.62 -> 2.45 us for one row of
// 8192 with float32 weights).  Held only
// within 32 dwords a lane and a lane state (row vectors, quantiser values,
// weights) within 3/8 of the registers the block size allows (512- and
// 1024-thread blocks: 256 and 128), which keeps every variant free of spills.
template <typename T, typename WT, int NORM, bool FUSED, int QM, int WPR, int VPL>
constexpr bool fwd_hold_w()
{
    constexpr int dw = WRaw<T, WT>::dw;
    constexpr int state = VPL * (4 * (FUSED ? 2 : 1) + (QM != kQNone ? Vec<T>::n : 0) + dw);
    constexpr int cap = 512 * 256 / (kBlockFwd(WPR) > 256 ? kBlockFwd(WPR) : 256);
    return (QM != kQNone || (WPR == 16 && VPL == 1)) && VPL * dw <= 32 && 8 * state <= 3 * cap;
}

template <typename T, typename WT, int NORM, bool FUSED, int QM, int WPR, int VPL>
__global__ void __launch_bounds__(kBlockFwd(WPR)) fwd_vec_kernel(FwdArgs a)
{
    constexpr int NV = Vec<T>::n;
    constexpr int VSTRIDE = 64 * WPR;
    constexpr int RPB = kBlockFwd(WPR) / (64 * WPR); // rows per block step
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int rib = (WPR == 1) ? wave : 0;
    const int wir = (WPR == 1) ? 0 : wave;
    const int vbase = wir * 64 + lane;
    const int nvec = a.nvec;
    const float inv_n = 1.0f / (float)a.N;

    // Row sums.  With up to 2 vectors a lane (NS = VPL), in one order
    // whatever the launch shape: each vector's values are summed in order,
    // each block of 64 consecutive vectors (a wave's lanes at one k) by the
    // fixed DPP tree of wave_sum, and the blocks, b = v / 64 = wir + k * WPR,
    // one after another from the first; blocks past the row hold exactly
    // zero.  So those shapes all give the same float32 sum, bit for bit, and
    // the plain and the fused forward agree on the same residual even where
    // the dispatcher gives them different shapes (16 waves of one vector
    // against 8 of two).  Longer per-lane chains (NS = 1) sum a lane's
    // vectors together first, then the waves in order: a tree per vector
    // would hold more registers than those shapes have.  Each reduction of a
    // row has its own LDS slot; a slot is reused two rows later, after at
    // least two barriers, so one barrier per reduction suffices.
    constexpr int NS = VPL <= 2 ? VPL : 1;
    __shared__ float part[4][WPR * NS > 16 ? WPR * NS : 16];
    auto row_sum = [&](const float (&v)[NS], int slot) -> float {
        float t = 0.0f;
        if constexpr (WPR > 1) {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const float tj = wave_sum(v[j]);
                if (lane == 0)
                    part[slot][j * WPR + wir] = tj;
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < WPR * NS; ++b)
                t += part[slot][b];
        } else {
#pragma unroll
            for (int j = 0; j < NS; ++j)
                t += wave_sum(v[j]);
        }
        return t;
    };
    auto row_max = [&](float v, int slot) -> float {
        float t = wave_max(v);
        if constexpr (WPR > 1) {
            if (lane == 0)
                part[slot][wir] = t;
            __syncthreads();
            t = 0.0f;
#pragma unroll
            for (int i = 0; i < WPR; ++i)
                t = __builtin_fmaxf(t, part[slot][i]);
        }
        return t;
    };

    // The weights of the lane's columns (fwd_hold_w).  A vector past the row
    // reads the row's last vector (in bounds) and is masked at use, so the
    // loads need no branch and issue together.
    constexpr bool HOLD_W = fwd_hold_w<T, WT, NORM, FUSED, QM, WPR, VPL>();
    WRaw<T, WT> wr[HOLD_W ? VPL : 1];
    if constexpr (HOLD_W) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            wr[k] = ld_w_raw<T, WT>(a.w, v < nvec ? v : nvec - 1);
        }
    }
    auto weights = [&](int k, int v, float (&wf)[NV]) {
        if constexpr (HOLD_W)
            unpack_w<T, WT>(wr[k], wf);
        else
            load_w<T, WT>(a.w, v < nvec ? v : nvec - 1, wf);
    };

    // Blocks are dealt to the 8 XCDs round-robin, so the rows in flight form
    // one compact window of memory; giving each XCD a contiguous range of rows
    // instead measured 8 % slower.
    const int64_t step = (int64_t)gridDim.x * RPB;
    int it = 0;
    for (int64_t row = (int64_t)blockIdx.x * RPB + rib; row < a.M; row += step, ++it) {
        const size_t base = (size_t)row * (size_t)a.N;
        const u32x4 *xp = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.x) + base);
        const u32x4 *rp = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.r) + base);
        u32x4 *yp = reinterpret_cast<u32x4 *>(static_cast<T *>(a.y) + base);
        u32x4 *resp = reinterpret_cast<u32x4 *>(static_cast<T *>(a.res) + base);

        // 1. issue every load of the row before any use
        u32x4 hv[VPL];
        u32x4 rv[FUSED ? VPL : 1];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            if (v < nvec) {
                hv[k] = ld_stream<kPol>(xp + v);
                if constexpr (FUSED)
                    rv[k] = ld_stream<kPol>(rp + v);
            } else {
                hv[k] = u32x4{0u, 0u, 0u, 0u};
                if constexpr (FUSED)
                    rv[k] = u32x4{0u, 0u, 0u, 0u};
            }
        }

        // 2. residual add (float32), store the residual as T, and accumulate
        //    the first row sum of the stored residual: h^2 (RMS) or h (Layer).
        //    E4M3 with a per-row scale and held weights: also max |h * w|,
        //    so that the row's absmax, rstd * max |h * w| (rstd > 0), comes
        //    from the same exchange as the sum instead of a second one after
        //    y (it differs from max |y| only in float32 rounding).
        constexpr bool EARLY_MAX = QM == kQRow && HOLD_W;
        float s1[NS], hwmax = 0.0f;
#pragma unroll
        for (int j = 0; j < NS; ++j)
            s1[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float h[NV];
            unpack<T>(hv[k], h);
            if constexpr (FUSED) {
                float rr[NV];
                unpack<T>(rv[k], rr);
#pragma unroll
                for (int e = 0; e < NV; ++e)
                    h[e] = h[e] + rr[e];
                hv[k] = pack<T>(h); // rounds to T (bf16: RNE)
                unpack<T>(hv[k], h);
                const int v = vbase + k * VSTRIDE;
                if (v < nvec)
                    st_stream<kPol>(resp + v, hv[k]);
            }
            float &acc = s1[NS == VPL ? k : 0];
#pragma unroll
            for (int e = 0; e < NV; ++e)
                acc = (NORM == kRms) ? __builtin_fmaf(h[e], h[e], acc) : acc + h[e];
            if constexpr (EARLY_MAX) {
                float wf[NV];
                unpack_w<T, WT>(wr[k], wf);
#pragma unroll
                for (int e = 0; e < NV; ++e)
                    hwmax = __builtin_fmaxf(hwmax, __builtin_fabsf(h[e] * wf[e]));
            }
        }

        // 3. row statistics
        const int slot = (it & 1) * 2;
        float mu = 0.0f, rs;
        if constexpr (EARLY_MAX) {
            // the sum (in the order of row_sum) and the maximum through one
            // LDS exchange and barrier
            float t = 0.0f, m = wave_max(hwmax);
            if constexpr (WPR > 1) {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const float tj = wave_sum(s1[j]);
                    if (lane == 0)
                        part[slot][j * WPR + wir] = tj;
                }
                if (lane == 0)
                    part[slot + 1][wir] = m;
                __syncthreads();
                m = 0.0f;
#pragma unroll
                for (int b = 0; b < WPR * NS; ++b)
                    t += part[slot][b];
#pragma unroll
                for (int i = 0; i < WPR; ++i)
                    m = __builtin_fmaxf(m, part[slot + 1][i]);
            } else {
#pragma unroll
                for (int j = 0; j < NS; ++j)
                    t += wave_sum(s1[j]);
            }
            rs = 1.0f / __builtin_sqrtf(t * inv_n + a.eps);
            hwmax = m;
        } else if constexpr (NORM == kRms) {
            rs = 1.0f / __builtin_sqrtf(row_sum(s1, slot) * inv_n + a.eps);
        } else {
            mu = row_sum(s1, slot) * inv_n;
            float s2[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j)
                s2[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (vbase + k * VSTRIDE < nvec) {
                    float h[NV];
                    unpack<T>(hv[k], h);
                    float &acc = s2[NS == VPL ? k : 0];
#pragma unroll
                    for (int e = 0; e < NV; ++e) {
                        const float d = h[e] - mu;
                        acc = __builtin_fmaf(d, d, acc);
                    }
                }
            }
            rs = 1.0f / __builtin_sqrtf(row_sum(s2, slot + 1) * inv_n + a.eps);
            if (a.mean != nullptr && wir == 0 && lane == 0)
                a.mean[row] = mu;
        }
        if (a.rstd != nullptr && wir == 0 && lane == 0)
            a.rstd[row] = rs;

        if constexpr (QM != kQNone) {
            // 4'. y in registers, then its quantised form instead of y
            float o[VPL][NV];
            float am = 0.0f;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int v = vbase + k * VSTRIDE;
                float h[NV], wf[NV];
                unpack<T>(hv[k], h);
                weights(k, v, wf);
#pragma unroll
                for (int e = 0; e < NV; ++e) {
                    o[k][e] = v < nvec ? (h[e] * rs) * wf[e] : 0.0f;
                    if constexpr (QM == kQRow && !EARLY_MAX)
                        am = __builtin_fmaxf(am, __builtin_fabsf(o[k][e]));
                }
            }
            if constexpr (QM == kQMx) {
                // MXFP4: blocks of 32 values (32 / NV lanes); a NaN makes the
                // block's maximum +Inf (y is never infinite), which marks the
                // block NaN: scale 0xFF, codes 0
                uint8_t *qrow4 = a.q + base / 2;
                uint8_t *srow = static_cast<uint8_t *>(a.qscale) + (size_t)row * (size_t)a.qgroups;
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    const int v = vbase + k * VSTRIDE;
                    float g = 0.0f;
#pragma unroll
                    for (int e = 0; e < NV; ++e) {
                        const float m = __builtin_fabsf(o[k][e]);
                        g = __builtin_fmaxf(g, m != m ? __builtin_inff() : m);
                    }
                    g = group_max_n<32 / NV>(g);
                    const bool nanb = g == __builtin_inff();
                    const int E = mx_exponent(g);
                    const float inv = __uint_as_float((uint32_t)(127 - E) << 23); // 2^-E
                    if (v < nvec && (lane & (32 / NV - 1)) == 0)
                        srow[v / (32 / NV)] = nanb ? (uint8_t)0xFF : (uint8_t)(E + 127);
                    if (v < nvec) {
                        uint32_t word = pack_e2m1x2<0>(0u, o[k][0] * inv, o[k][1] * inv);
                        word = pack_e2m1x2<1>(word, o[k][2] * inv, o[k][3] * inv);
                        if constexpr (NV == 8) {
                            word = pack_e2m1x2<2>(word, o[k][4] * inv, o[k][5] * inv);
                            word = pack_e2m1x2<3>(word, o[k][6] * inv, o[k][7] * inv);
                        }
                        if (nanb)
                            word = 0u;
                        if constexpr (NV == 8)
                            __builtin_nontemporal_store(
                                word, reinterpret_cast<uint32_t *>(qrow4 + (size_t)v * 4));
                        else
                            __builtin_nontemporal_store(
                                (uint16_t)word, reinterpret_cast<uint16_t *>(qrow4 + (size_t)v * 2));
                    }
                }
            } else {
                // E4M3: one scale per row (kQRow), or one per group of
                // a.qlanes consecutive vectors, which sit in as many
                // consecutive lanes (kQGroup)
                float inv_k[VPL];
                if constexpr (QM == kQRow) {
                    if constexpr (EARLY_MAX) {
                        am = rs * hwmax;
                        if (!(am == am)) // NaN row (rstd NaN) or 0 * inf: as max |y| over no finite y
                            am = 0.0f;
                    } else {
                        am = row_max(am, slot + 1);
                    }
                    float inv = 1.0f, sc = 1.0f;
                    if (am != 0.0f) {
                        inv = 448.0f / am;
                        sc = am / 448.0f;
                    }
                    if (wir == 0 && lane == 0)
                        static_cast<float *>(a.qscale)[row] = sc;
#pragma unroll
                    for (int k = 0; k < VPL; ++k)
                        inv_k[k] = inv;
                } else {
                    float *srow = static_cast<float *>(a.qscale) + (size_t)row * (size_t)a.qgroups;
#pragma unroll
                    for (int k = 0; k < VPL; ++k) {
                        const int v = vbase + k * VSTRIDE;
                        float g = 0.0f;
#pragma unroll
                        for (int e = 0; e < NV; ++e)
                            g = __builtin_fmaxf(g, __builtin_fabsf(o[k][e]));
                        g = group_max(g, a.qlanes);
                        float inv = 1.0f, sc = 1.0f;
                        if (g != 0.0f) {
                            inv = 448.0f / g;
                            sc = g / 448.0f;
                        }
                        if (v < nvec && (lane & (a.qlanes - 1)) == 0)
                            srow[v / a.qlanes] = sc;
                        inv_k[k] = inv;
                    }
                }
                uint8_t *qrow = a.q + base;
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    const int v = vbase + k * VSTRIDE;
                    const float inv = inv_k[k];
                    if (v < nvec) {
                        uint32_t wd[NV / 4];
#pragma unroll
                        for (int i = 0; i < NV / 4; ++i)
                            wd[i] = pack_e4m3x2(e4m3_clamp(o[k][4 * i] * inv),
                                                e4m3_clamp(o[k][4 * i + 1] * inv)) |
                                    (pack_e4m3x2(e4m3_clamp(o[k][4 * i + 2] * inv),
                                                 e4m3_clamp(o[k][4 * i + 3] * inv))
                                     << 16);
                        if constexpr (NV == 8)
                            __builtin_nontemporal_store(
                                u32x2{wd[0], wd[1]}, reinterpret_cast<u32x2 *>(qrow + (size_t)v * 8));
                        else
                            __builtin_nontemporal_store(
                                wd[0], reinterpret_cast<uint32_t *>(qrow + (size_t)v * 4));
                    }
                }
            }
            continue;
        }

        // 4. y = (h - mean) * rstd * w (+ b), rounded once to T
        const bool bias = NORM == kLayer && a.b != nullptr;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            if (v < nvec) {
                float h[NV], wf[NV], o[NV];
                unpack<T>(hv[k], h);
                weights(k, v, wf);
#pragma unroll
                for (int e = 0; e < NV; ++e)
                    o[e] = ((NORM == kLayer ? h[e] - mu : h[e]) * rs) * wf[e];
                if (bias) {
                    float bf[NV];
                    load_w<T, WT>(a.b, v, bf);
#pragma unroll
                    for (int e = 0; e < NV; ++e)
                        o[e] += bf[e];
                }
                st_stream<kPol>(yp + v, pack<T>(o));
            }
        }
    }
}

// Block-wide sum for 256-thread blocks.  Each call site uses its own slot of
// `part`, alternating between rows, so one barrier per call suffices.
template <typename S, int NS>
__device__ __forceinline__ S block256_sum(S v, S (&part)[NS][4], int slot)
{
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    S t = wave_sum(v);
    if (lane == 0)
        part[slot][wave] = t;
    __syncthreads();
    return (part[slot][0] + part[slot][1]) + (part[slot][2] + part[slot][3]);
}

// ---------------------------------------------------------------------------
// Forward, element-wise path: any N, any alignment.  One 256-thread block per
// row; the row is re-read from memory (mostly cache) for each pass: the sum,
// the LayerNorm variance, and the output.  The fused op re-reads the stored
// residual.
// ---------------------------------------------------------------------------
// Block-wide maximum, as block256_sum (IEEE maxNum: NaNs ignored).
template <int NS>
__device__ __forceinline__ float block256_max(float v, float (&part)[NS][4], int slot)
{
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    float t = wave_max(v);
    if (lane == 0)
        part[slot][wave] = t;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(part[slot][0], part[slot][1]),
                           __builtin_fmaxf(part[slot][2], part[slot][3]));
}

template <typename T, typename WT, int NORM, bool FUSED, int QM>
__global__ void __launch_bounds__(256) fwd_elem_kernel(FwdArgs a)
{
    __shared__ float part[4][4];
    const int tid = threadIdx.x;
    const int N = a.N;
    const float inv_n = 1.0f / (float)N;
    const void *src = FUSED ? a.res : a.x; // where h is read back from
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x, ++it) {
        const int64_t base = row * (int64_t)N;
        const int slot = (it & 1) * 2;
        float s1 = 0.0f;
        for (int j = tid; j < N; j += 256) {
            float h;
            if constexpr (FUSED) {
                const float s = ld_elem<T>(a.x, base + j) + ld_elem<T>(a.r, base + j);
                st_elem<T>(a.res, base + j, s);
                h = as_stored<T>(s);
            } else {
                h = ld_elem<T>(a.x, base + j);
            }
            s1 = (NORM == kRms) ? __builtin_fmaf(h, h, s1) : s1 + h;
        }
        float mu = 0.0f, rs;
        if constexpr (NORM == kRms) {
            rs = 1.0f / __builtin_sqrtf(block256_sum(s1, part, slot) * inv_n + a.eps);
        } else {
            mu = block256_sum(s1, part, slot) * inv_n;
            float s2 = 0.0f;
            for (int j = tid; j < N; j += 256) {
                const float d = ld_elem<T>(src, base + j) - mu;
                s2 = __builtin_fmaf(d, d, s2);
            }
            rs = 1.0f / __builtin_sqrtf(block256_sum(s2, part, slot + 1) * inv_n + a.eps);
            if (a.mean != nullptr && tid == 0)
                a.mean[row] = mu;
        }
        if (a.rstd != nullptr && tid == 0)
            a.rstd[row] = rs;
        if constexpr (QM == kQMx) {
            // MXFP4: each thread takes whole blocks of 32 columns
            for (int g = tid; g < a.qgroups; g += 256) {
                const int j0 = g * 32, j1 = j0 + 32 < N ? j0 + 32 : N;
                float am = 0.0f;
                bool nanb = false;
                for (int j = j0; j < j1; ++j) {
                    const float o = (ld_elem<T>(src, base + j) * rs) * ld_elem<WT>(a.w, j);
                    nanb = nanb || o != o;
                    am = __builtin_fmaxf(am, __builtin_fabsf(o));
                }
                const int E = mx_exponent(am);
                const float inv = __uint_as_float((uint32_t)(127 - E) << 23);
                static_cast<uint8_t *>(a.qscale)[row * (int64_t)a.qgroups + g] =
                    nanb ? (uint8_t)0xFF : (uint8_t)(E + 127);
                for (int j = j0; j < j1; j += 2) {
                    const float o0 = (ld_elem<T>(src, base + j) * rs) * ld_elem<WT>(a.w, j);
                    const float o1 = (ld_elem<T>(src, base + j + 1) * rs) * ld_elem<WT>(a.w, j + 1);
                    a.q[(base + j) / 2] = nanb ? (uint8_t)0 : (uint8_t)pack_e2m1x2<0>(0u, o0 * inv, o1 * inv);
                }
            }
            continue;
        }
        if constexpr (QM == kQGroup) {
            // one scale per group of qgroup columns: each thread takes whole
            // groups
            const int G = a.qgroup;
            for (int g = tid; g < a.qgroups; g += 256) {
                const int j0 = g * G, j1 = j0 + G < N ? j0 + G : N;
                float am = 0.0f;
                for (int j = j0; j < j1; ++j)
                    am = __builtin_fmaxf(am, __builtin_fabsf((ld_elem<T>(src, base + j) * rs) *
                                                             ld_elem<WT>(a.w, j)));
                float inv = 1.0f, sc = 1.0f;
                if (am != 0.0f) {
                    inv = 448.0f / am;
                    sc = am / 448.0f;
                }
                static_cast<float *>(a.qscale)[row * (int64_t)a.qgroups + g] = sc;
                for (int j = j0; j < j1; ++j) {
                    const float o = (ld_elem<T>(src, base + j) * rs) * ld_elem<WT>(a.w, j);
                    a.q[base + j] = (uint8_t)pack_e4m3x2(e4m3_clamp(o * inv), 0.0f);
                }
            }
            continue;
        }
        if constexpr (QM == kQRow) {
            float am = 0.0f;
            for (int j = tid; j < N; j += 256)
                am = __builtin_fmaxf(am, __builtin_fabsf((ld_elem<T>(src, base + j) * rs) *
                                                         ld_elem<WT>(a.w, j)));
            am = block256_max(am, part, slot + 1);
            float inv = 1.0f, sc = 1.0f;
            if (am != 0.0f) {
                inv = 448.0f / am;
                sc = am / 448.0f;
            }
            if (tid == 0)
                static_cast<float *>(a.qscale)[row] = sc;
            for (int j = tid; j < N; j += 256) {
                const float o = (ld_elem<T>(src, base + j) * rs) * ld_elem<WT>(a.w, j);
                a.q[base + j] = (uint8_t)pack_e4m3x2(e4m3_clamp(o * inv), 0.0f);
            }
            continue;
        }
        const bool bias = NORM == kLayer && a.b != nullptr;
        for (int j = tid; j < N; j += 256) {
            const float h = ld_elem<T>(src, base + j);
            float o = ((NORM == kLayer ? h - mu : h) * rs) * ld_elem<WT>(a.w, j);
            if (bias)
                o += ld_elem<WT>(a.b, j);
            st_elem<T>(a.y, base + j, o);
        }
    }
}

// Backward register budget.  A lane holds across a row its vectors of dy, x
// and (RES) dres, 4 dwords each; one float sum per element for dw (and db);
// the weights when it keeps them (HOLD_W below); and, for float32 rows, whose
// arithmetic is binary64, about one more dword per element of temporaries.
// The kernel asks the register allocator (amdgpu_waves_per_eu) for the most
// waves per SIMD, of 4, 3 and 2 (at most 128, 168 and 256 VGPRs a lane),
// whose budget holds that state plus 28 + 5 * VPL for addresses and
// temporaries.  Without a request the allocator spends registers on
// instruction-level parallelism and lands below these levels; the margin was
// fitted to the variants' compiled register counts so that none spills.
template <typename T, typename WT> constexpr bool bwd_hold_w(int vpl)
{
    return vpl * WRaw<T, WT>::dw <= 32;
}
template <typename T, typename WT, int NORM, bool RES, int VPL, bool PF = false> constexpr int bwd_waves()
{
    constexpr int nv = Vec<T>::n;
    constexpr int state = VPL * (4 * (2 + (RES ? 1 : 0)) * (PF ? 2 : 1) + nv * (NORM == kLayer ? 2 : 1) +
                                 (bwd_hold_w<T, WT>(VPL) ? WRaw<T, WT>::dw : 0) +
                                 (sizeof(T) == 4 ? nv : 0));
    constexpr int need = state + 28 + 5 * VPL + (PF ? 8 : 0);
    return need <= 128 ? 4 : need <= 168 ? 3 : need <= 256 ? 2 : 1;
}

// ---------------------------------------------------------------------------
// Backward, vector path, 256-thread blocks with WPR in {1, 2, 4} (RPB = 4 / WPR
// rows per block step), or 512-thread blocks with WPR = 8 (one row per step),
// or (WIDE) 1024-thread blocks with WPR = 2 (8 rows per step).  Each lane keeps its columns' dw (and, for LayerNorm,
// db) partial sums in registers across all rows it visits; at the end the
// block's row groups are summed through LDS (pairwise, fixed order) and
// written as one row of the workspace: ws[blockIdx.x, :] (and ws2 for db).
// Dynamic LDS: (RPB / 2) * N floats.
// NORM = kRms: g = dy*w, xh = x*rstd, dx = rstd*(g - xh*mean(g*xh)).
// NORM = kLayer: xh = (x - mean)*rstd, dx = rstd*(g - mean(g) - xh*mean(g*xh)),
// db = sum dy.
// RES: the fused op's backward, which adds the residual gradient dres to dx
// before its one rounding (dx then holds dh, the gradient of x and of r).
// ---------------------------------------------------------------------------
template <typename T, typename WT, int NORM, bool RES, int WPR, int VPL, bool WIDE = false, bool PF = false>
__global__ void __launch_bounds__(kBwdBlockOf(WPR, WIDE))
    __attribute__((amdgpu_waves_per_eu(bwd_waves<T, WT, NORM, RES, VPL, PF>()))) bwd_vec_kernel(BwdArgs a)
{
    constexpr int NV = Vec<T>::n;
    constexpr int VSTRIDE = 64 * WPR;
    constexpr int RPB = bwd_rpb(WPR, WIDE);
    constexpr bool LN = NORM == kLayer;
    using CT = typename BwdCompute<T>::type;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ CT part[2][2][kBwdBlockOf(WPR, WIDE) / 64]; // [row parity][sum][wave]

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int rib = wave / WPR;
    const int wir = wave % WPR;
    const int vbase = wir * 64 + lane;
    const int nvec = a.nvec;
    const int N = a.N;
    const CT inv_n = inv_n_ct<CT>(N);

    float accw[VPL][NV];
    float accb[LN ? VPL : 1][LN ? NV : 1];
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            accw[k][e] = 0.0f;
            if constexpr (LN)
                accb[k][e] = 0.0f;
        }

    // w is the same for every row: each lane loads its columns' weights once,
    // in their stored form, and widens them at each use.  The row passes below
    // then issue no loads, so no wait inside them stalls on a weight fetch or
    // on the acknowledgement of an earlier store.  Long rows (more than 32
    // dwords of weights per lane) load them at each use instead, which keeps
    // those variants free of spills.
    constexpr bool HOLD_W = bwd_hold_w<T, WT>(VPL);
    WRaw<T, WT> wr[HOLD_W ? VPL : 1];
    if constexpr (HOLD_W) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            wr[k] = ld_w_raw<T, WT>(a.w, v < nvec ? v : nvec - 1);
        }
    }
    auto weights = [&](int k, int v, float (&wf)[NV]) {
        if constexpr (HOLD_W)
            unpack_w<T, WT>(wr[k], wf);
        else
            load_w<T, WT>(a.w, v, wf);
    };

    const int64_t step = (int64_t)gridDim.x * RPB;
    // Loads of one row group into registers.  Vector indices past the row are
    // clamped to its last vector (in bounds) and masked out at use, so the
    // loads need no branches; a row past M reads row 0 and is not used.
    auto load_row = [&](int64_t row, u32x4 (&dyv)[VPL], u32x4 (&xv)[VPL],
                        u32x4 (&drv)[RES ? VPL : 1], float &rs, float &mu) {
        const bool act = row < a.M;
        const size_t base = (size_t)(act ? row : 0) * (size_t)N;
        const u32x4 *dyp = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.dy) + base);
        const u32x4 *xp = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.x) + base);
        const u32x4 *drp = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.dres) + base);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            const int vc = v < nvec ? v : nvec - 1;
            dyv[k] = ld_stream<kPol>(dyp + vc);
            xv[k] = ld_stream<kPol>(xp + vc);
            if constexpr (RES)
                drv[k] = ld_stream<kPol>(drp + vc);
        }
        rs = act ? a.rstd[row] : 0.0f;
        mu = (LN && act) ? a.mean[row] : 0.0f;
    };
    u32x4 dyv[VPL], xv[VPL];
    u32x4 drv[RES ? VPL : 1];
    float rs = 0.0f, mu = 0.0f;
    // PF: the next row's loads go out after this row's sums, so they are in
    // flight across the row exchange and the output pass.  The lane then holds
    // two rows, so fewer waves fit per SIMD (RMS at 4 vectors a lane: 3
    // instead of 4), and the kernel still streams faster at 4 vectors a lane
    // and 2 waves per row (measured on MI355X: RMS 1.5-3.6 %, LayerNorm
    // 3.5-5.8 %, fused LayerNorm 2-5 %).  dx is bit-identical; dw differs
    // only in how rows group into partial sums (the grid follows residency).
    u32x4 ndy[PF ? VPL : 1], nx[PF ? VPL : 1];
    u32x4 ndr[(PF && RES) ? VPL : 1];
    float nrs = 0.0f, nmu = 0.0f;
    if constexpr (PF) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) { // defined values past the last row
            ndy[k] = nx[k] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (RES)
                ndr[k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (PF)
        load_row((int64_t)blockIdx.x * RPB + rib, dyv, xv, drv, rs, mu);
    int it = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * RPB; row0 < a.M; row0 += step, ++it) {
        const int64_t row = row0 + rib;
        const bool active = row < a.M; // uniform per wave
        const size_t base = (size_t)(active ? row : 0) * (size_t)N;
        u32x4 *dxp = reinterpret_cast<u32x4 *>(static_cast<T *>(a.dx) + base);
        if constexpr (!PF)
            load_row(row, dyv, xv, drv, rs, mu);

        // row sums: p = sum dy*w*x (RMS) or sum g (Layer); q = sum g*xh (Layer)
        CT p = 0, q = 0;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            if (v < nvec) {
                float d[NV], xx[NV], wf[NV];
                unpack<T>(dyv[k], d);
                unpack<T>(xv[k], xx);
                weights(k, v, wf);
#pragma unroll
                for (int e = 0; e < NV; ++e) {
                    const CT g = (CT)d[e] * (CT)wf[e];
                    if constexpr (LN) {
                        p += g;
                        q = fma_ct(g, ((CT)xx[e] - (CT)mu) * (CT)rs, q);
                    } else {
                        p = fma_ct(g, (CT)xx[e], p);
                    }
                }
            }
        }
        if constexpr (PF) {
            if (row + step < a.M) // uniform per wave
                load_row(row + step, ndy, nx, ndr, nrs, nmu);
        }
        p = wave_sum(p);
        if constexpr (LN)
            q = wave_sum(q);
        if constexpr (WPR > 1) {
            if (lane == 0) {
                part[it & 1][0][wave] = p;
                part[it & 1][1][wave] = q;
            }
            __syncthreads();
            p = 0;
            q = 0;
#pragma unroll
            for (int i = 0; i < WPR; ++i) {
                p += part[it & 1][0][rib * WPR + i];
                q += part[it & 1][1][rib * WPR + i];
            }
        }
        // RMS: c1 = 0, c2 = mean(g*xh) = rstd*mean(dy*w*x)
        // Layer: c1 = mean(g), c2 = mean(g*xh)
        const CT c1 = LN ? p * inv_n : (CT)0;
        const CT c2 = LN ? q * inv_n : (p * (CT)rs) * inv_n;

        if (active) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int v = vbase + k * VSTRIDE;
                if (v < nvec) {
                    float d[NV], xx[NV], wf[NV], o[NV], dr[NV];
                    unpack<T>(dyv[k], d);
                    unpack<T>(xv[k], xx);
                    weights(k, v, wf);
                    if constexpr (RES)
                        unpack<T>(drv[k], dr);
#pragma unroll
                    for (int e = 0; e < NV; ++e) {
                        const CT xh = ((CT)xx[e] - (CT)mu) * (CT)rs;
                        const CT g = (CT)d[e] * (CT)wf[e];
                        CT dxe = (CT)rs * (g - c1 - xh * c2);
                        if constexpr (RES)
                            dxe += (CT)dr[e];
                        o[e] = (float)dxe;
                        accw[k][e] = __builtin_fmaf(d[e], (float)xh, accw[k][e]);
                        if constexpr (LN)
                            accb[k][e] += d[e];
                    }
                    st_stream<kPol>(dxp + v, pack<T>(o));
                }
            }
        }
        if constexpr (PF) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                dyv[k] = ndy[k];
                xv[k] = nx[k];
                if constexpr (RES)
                    drv[k] = ndr[k];
            }
            rs = nrs;
            mu = nmu;
        }
    }

    // dw (db): sum the block's RPB row groups (same columns) and write one row.
    auto put = [&](auto &acc, float *dst) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            if (v < nvec) {
                u32x4 *qq = reinterpret_cast<u32x4 *>(dst + (size_t)v * NV);
#pragma unroll
                for (int h = 0; h < NV / 4; ++h)
                    qq[h] = u32x4{__float_as_uint(acc[k][4 * h]), __float_as_uint(acc[k][4 * h + 1]),
                                  __float_as_uint(acc[k][4 * h + 2]), __float_as_uint(acc[k][4 * h + 3])};
            }
        }
    };
    auto add = [&](auto &acc, const float *src) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vbase + k * VSTRIDE;
            if (v < nvec) {
                const u32x4 *qq = reinterpret_cast<const u32x4 *>(src + (size_t)v * NV);
#pragma unroll
                for (int h = 0; h < NV / 4; ++h) {
                    const u32x4 t = qq[h];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[k][4 * h + i] += __uint_as_float(t[i]);
                }
            }
        }
    };
    // Pairwise tree over the RPB row groups (a power of two), fixed order:
    // at each level the upper half of the remaining groups parks its sums in
    // LDS ((RPB / 2) * N floats) and the lower half adds them.
    auto merge = [&](auto &acc, float *out) {
#pragma unroll
        for (int half = RPB / 2; half >= 1; half /= 2) {
            if (rib >= half && rib < 2 * half)
                put(acc, lds + (size_t)(rib - half) * N);
            __syncthreads();
            if (rib < half)
                add(acc, lds + (size_t)rib * N);
            if (half > 1)
                __syncthreads(); // the next level's parking overwrites these slots
        }
        if (rib == 0)
            put(acc, out);
    };
    merge(accw, a.ws + (size_t)blockIdx.x * (size_t)N);
    if constexpr (LN) {
        __syncthreads(); // the LDS is reused for db
        merge(accb, a.ws2 + (size_t)blockIdx.x * (size_t)N);
    }
}

// ---------------------------------------------------------------------------
// Backward, element-wise path (any N, any alignment): dx one block per row in
// two passes; dw (db) partials per (column block, row chunk).  dw runs first,
// so dx may overwrite dy or x.
// ---------------------------------------------------------------------------
template <typename T, typename WT, int NORM, bool RES>
__global__ void __launch_bounds__(256) bwd_elem_dx_kernel(BwdArgs a)
{
    using CT = typename BwdCompute<T>::type;
    constexpr bool LN = NORM == kLayer;
    __shared__ CT part[4][4];
    const int tid = threadIdx.x;
    const int N = a.N;
    const CT inv_n = inv_n_ct<CT>(N);
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x, ++it) {
        const int64_t base = row * (int64_t)N;
        const CT rs = (CT)a.rstd[row];
        const CT mu = LN ? (CT)a.mean[row] : (CT)0;
        CT p = 0, q = 0;
        for (int j = tid; j < N; j += 256) {
            const CT g = (CT)ld_elem<T>(a.dy, base + j) * (CT)ld_elem<WT>(a.w, j);
            const CT xv = (CT)ld_elem<T>(a.x, base + j);
            if constexpr (LN) {
                p += g;
                q = fma_ct(g, (xv - mu) * rs, q);
            } else {
                p = fma_ct(g, xv, p);
            }
        }
        const int slot = (it & 1) * 2;
        p = block256_sum(p, part, slot);
        if constexpr (LN)
            q = block256_sum(q, part, slot + 1);
        const CT c1 = LN ? p * inv_n : (CT)0;
        const CT c2 = LN ? q * inv_n : (p * rs) * inv_n;
        for (int j = tid; j < N; j += 256) {
            const CT xh = ((CT)ld_elem<T>(a.x, base + j) - mu) * rs;
            const CT g = (CT)ld_elem<T>(a.dy, base + j) * (CT)ld_elem<WT>(a.w, j);
            CT dxe = rs * (g - c1 - xh * c2);
            if constexpr (RES)
                dxe += (CT)ld_elem<T>(a.dres, base + j);
            st_elem<T>(a.dx, base + j, (float)dxe);
        }
    }
}

template <typename T, int NORM>
__global__ void __launch_bounds__(256) bwd_elem_dw_kernel(BwdArgs a)
{
    constexpr bool LN = NORM == kLayer;
    __shared__ float red[2][4][64];
    const int lane = threadIdx.x & 63;
    const int s = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const int64_t r0 = (int64_t)blockIdx.y * a.chunk;
    const int64_t r1 = r0 + a.chunk < a.M ? r0 + a.chunk : a.M;
    float aw = 0.0f, ab = 0.0f;
    if (c < a.N)
        for (int64_t i = r0 + s; i < r1; i += 4) {
            const int64_t idx = i * (int64_t)a.N + c;
            const float d = ld_elem<T>(a.dy, idx);
            const float mu = LN ? a.mean[i] : 0.0f;
            aw = __builtin_fmaf(d, (ld_elem<T>(a.x, idx) - mu) * a.rstd[i], aw);
            ab += d;
        }
    red[0][s][lane] = aw;
    red[1][s][lane] = ab;
    __syncthreads();
    if (s == 0 && c < a.N) {
        a.ws[(size_t)blockIdx.y * a.N + c] =
            (red[0][0][lane] + red[0][1][lane]) + (red[0][2][lane] + red[0][3][lane]);
        if constexpr (LN)
            a.ws2[(size_t)blockIdx.y * a.N + c] =
                (red[1][0][lane] + red[1][1][lane]) + (red[1][2][lane] + red[1][3][lane]);
    }
}

// dw[c] = sum_p ws[p, c], the second stage of the dw reduction (and, for
// LayerNorm, db[c] = sum_p ws2[p, c] in the same launch: blockIdx.y = 1).  The
// partial rows are few (P <= 1024) and the columns many, so a block takes a
// narrow column strip and splits the rows over slices of threads; the slices
// are then merged in LDS by a fixed-order tree, so the result is
// deterministic.  Vector form: 32-column strips, so that each block reads
// whole 128-byte lines of every partial row (with 16-column strips two blocks
// fetched each line, and 1024 partial rows of 7168 columns took 11 us instead
// of 3.6); 8 x 16-byte lanes by 128 row slices, and up to 8 rows per thread
// loaded at once (the kernel is short and latency-bound: every load of a
// thread is in flight together).  Requires N % 4 == 0 and 16-byte aligned
// partials and outputs.  (Templates only so that each translation unit's copy
// is a weak symbol.)
template <int Unused = 0>
__global__ void __launch_bounds__(kColReduceVecBlock)
    dw_colreduce_vec_kernel(const float *ws, const float *ws2, int P, int N, float *dw, float *db)
{
    constexpr int Q = kColReduceVecCols / 4;   // 16-byte lanes per strip row
    constexpr int S = kColReduceVecBlock / Q;  // row slices
    constexpr int U = 8;                       // rows per thread per load batch
    __shared__ u32x4 red[S][Q];
    const float *src = blockIdx.y ? ws2 : ws;
    float *dst = blockIdx.y ? db : dw;
    const int q = threadIdx.x % Q;
    const int sl = threadIdx.x / Q;
    const int n4 = N / 4;
    const int c4 = blockIdx.x * Q + q;
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c4 < n4) {
        const u32x4 *base = reinterpret_cast<const u32x4 *>(src) + c4;
        for (int p0 = sl; p0 < P; p0 += U * S) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + u * S;
                v[u] = p < P ? base[(size_t)p * n4] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] += __uint_as_float(v[u][i]);
        }
    }
    red[sl][q] = u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                       __float_as_uint(a[3])};
    __syncthreads();
#pragma unroll
    for (int h = S / 2; h >= 1; h >>= 1) {
        if (sl < h) {
            const u32x4 o = red[sl + h][q];
            u32x4 m = red[sl][q];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m[i] = __float_as_uint(__uint_as_float(m[i]) + __uint_as_float(o[i]));
            red[sl][q] = m;
        }
        __syncthreads();
    }
    if (sl == 0 && c4 < n4)
        reinterpret_cast<u32x4 *>(dst)[c4] = red[0][q];
}

// Element form for any N / alignment: 16-column strips, 16 row slices.
template <int Unused = 0>
__global__ void __launch_bounds__(256)
    dw_colreduce_kernel(const float *ws, const float *ws2, int P, int N, float *dw, float *db)
{
    constexpr int W = 16, S = 256 / W;
    __shared__ float red[S][W];
    const float *src = blockIdx.y ? ws2 : ws;
    float *dst = blockIdx.y ? db : dw;
    const int q = threadIdx.x % W;
    const int sl = threadIdx.x / W;
    const int c = blockIdx.x * W + q;
    float acc = 0.0f;
    if (c < N)
        for (int p = sl; p < P; p += S)
            acc += src[(size_t)p * N + c];
    red[sl][q] = acc;
    __syncthreads();
#pragma unroll
    for (int h = S / 2; h >= 1; h >>= 1) {
        if (sl < h)
            red[sl][q] += red[sl + h][q];
        __syncthreads();
    }
    if (sl == 0 && c < N)
        dst[c] = red[0][q];
}

// ---------------------------------------------------------------------------
// Kernel tables for one (row dtype, weight dtype) combination.
// ---------------------------------------------------------------------------
template <typename T, typename WT> struct TableBuilder {
    template <int NM, bool F, int QM, int WPR, int VPL> static KernelRef fwd_ref()
    {
        if constexpr (QM == kQNone ? fwd_built(WPR, VPL) : q_built(QM, WPR, VPL))
            return KernelRef{
                reinterpret_cast<const void *>(&fwd_vec_kernel<T, WT, NM, F, QM, WPR, VPL>),
                kBlockFwd(WPR)};
        else
            return KernelRef{nullptr, 0};
    }
    template <int NM, bool F, int QM, int WI, int... VI>
    static void fwd_row(KernelRef (&row)[kNumVpl], std::integer_sequence<int, VI...>)
    {
        ((row[VI] = fwd_ref<NM, F, QM, kWprList[WI], kVplList[VI]>()), ...);
    }
    template <int NM, bool F, int QM, int... WI>
    static void fwd_all(KernelRef (&tab)[kNumWpr][kNumVpl], std::integer_sequence<int, WI...>)
    {
        (fwd_row<NM, F, QM, WI>(tab[WI], std::make_integer_sequence<int, kNumVpl>{}), ...);
    }
    template <bool F, int QM> static KernelRef elem_ref()
    {
        return KernelRef{reinterpret_cast<const void *>(&fwd_elem_kernel<T, WT, kRms, F, QM>), 256};
    }
    template <int NM> static void fwd_norm(FwdTable &t)
    {
        fwd_all<NM, false, kQNone>(t.vec[NM][0], std::make_integer_sequence<int, kNumWpr>{});
        fwd_all<NM, true, kQNone>(t.vec[NM][1], std::make_integer_sequence<int, kNumWpr>{});
        t.elem[NM][0] = KernelRef{
            reinterpret_cast<const void *>(&fwd_elem_kernel<T, WT, NM, false, kQNone>), 256};
        t.elem[NM][1] = KernelRef{
            reinterpret_cast<const void *>(&fwd_elem_kernel<T, WT, NM, true, kQNone>), 256};
    }
    template <int QM> static void fwd_quant(FwdTable &t)
    {
        fwd_all<kRms, false, QM>(t.vec_q8[0][QM - 1], std::make_integer_sequence<int, kNumWpr>{});
        fwd_all<kRms, true, QM>(t.vec_q8[1][QM - 1], std::make_integer_sequence<int, kNumWpr>{});
        t.elem_q8[0][QM - 1] = elem_ref<false, QM>();
        t.elem_q8[1][QM - 1] = elem_ref<true, QM>();
    }
    static FwdTable fwd()
    {
        FwdTable t{};
        fwd_norm<kRms>(t);
        fwd_norm<kLayer>(t);
        fwd_quant<kQRow>(t);
        fwd_quant<kQGroup>(t);
        fwd_quant<kQMx>(t);
        return t;
    }

    template <int NM, bool R, int WPR, int VPL> static KernelRef bwd_ref()
    {
        if constexpr (bwd_built(NM, R, WPR, VPL))
            return KernelRef{
                reinterpret_cast<const void *>(&bwd_vec_kernel<T, WT, NM, R, WPR, VPL>),
                kBwdBlockOf(WPR)};
        else
            return KernelRef{nullptr, 0};
    }
    template <int NM, bool R, int WI, int... VI>
    static void bwd_row(KernelRef (&row)[kNumVpl], std::integer_sequence<int, VI...>)
    {
        ((row[VI] = bwd_ref<NM, R, kWprList[WI], kVplList[VI]>()), ...);
    }
    // The wide variant: built where a lane's state fits the 128 VGPRs that 16
    // waves per CU leave (4 waves per SIMD) and the row takes at most 8
    // vectors a lane.
    template <int NM, bool R, int VPL> static KernelRef bwd_wide_ref()
    {
        if constexpr (bwd_built(NM, R, kBwdWideWpr, VPL) && VPL <= 8 &&
                      bwd_waves<T, WT, NM, R, VPL>() == 4)
            return KernelRef{
                reinterpret_cast<const void *>(&bwd_vec_kernel<T, WT, NM, R, kBwdWideWpr, VPL, true>),
                kBwdBlockOf(kBwdWideWpr, true)};
        else
            return KernelRef{nullptr, 0};
    }
    template <int NM, bool R, int... VI>
    static void bwd_wide_row(KernelRef (&row)[kNumVpl], std::integer_sequence<int, VI...>)
    {
        ((row[VI] = bwd_wide_ref<NM, R, kVplList[VI]>()), ...);
    }
    // Next-row prefetch variants: 2 waves per row, up to 4 vectors a lane.
    template <int NM, bool R, int WPR, int VPL> static KernelRef bwd_pf_ref()
    {
        if constexpr (WPR == 2 && VPL <= 4 && bwd_built(NM, R, WPR, VPL))
            return KernelRef{
                reinterpret_cast<const void *>(&bwd_vec_kernel<T, WT, NM, R, WPR, VPL, false, true>),
                kBwdBlockOf(WPR)};
        else
            return KernelRef{nullptr, 0};
    }
    template <int NM, bool R, int WI, int... VI>
    static void bwd_pf_row(KernelRef (&row)[kNumVpl], std::integer_sequence<int, VI...>)
    {
        ((row[VI] = bwd_pf_ref<NM, R, kWprList[WI], kVplList[VI]>()), ...);
    }
    template <int NM, bool R, int... WI>
    static void bwd_pf_all(BwdTable &t, std::integer_sequence<int, WI...>)
    {
        (bwd_pf_row<NM, R, WI>(t.pf[NM][R ? 1 : 0][WI], std::make_integer_sequence<int, kNumVpl>{}), ...);
    }
    template <int NM, bool R, int... WI>
    static void bwd_all(BwdTable &t, std::integer_sequence<int, WI...>)
    {
        (bwd_row<NM, R, WI>(t.vec[NM][R ? 1 : 0][WI], std::make_integer_sequence<int, kNumVpl>{}),
         ...);
    }
    static BwdTable bwd()
    {
        BwdTable t{};
        bwd_all<kRms, false>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_all<kRms, true>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_all<kLayer, false>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_all<kLayer, true>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_pf_all<kRms, false>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_pf_all<kLayer, false>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_pf_all<kRms, true>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_pf_all<kLayer, true>(t, std::make_integer_sequence<int, kBwdNumWpr>{});
        bwd_wide_row<kRms, false>(t.wide[kRms][0], std::make_integer_sequence<int, kNumVpl>{});
        bwd_wide_row<kRms, true>(t.wide[kRms][1], std::make_integer_sequence<int, kNumVpl>{});
        bwd_wide_row<kLayer, false>(t.wide[kLayer][0], std::make_integer_sequence<int, kNumVpl>{});
        bwd_wide_row<kLayer, true>(t.wide[kLayer][1], std::make_integer_sequence<int, kNumVpl>{});
        t.elem_dx[kRms][0] =
            KernelRef{reinterpret_cast<const void *>(&bwd_elem_dx_kernel<T, WT, kRms, false>), 256};
        t.elem_dx[kRms][1] =
            KernelRef{reinterpret_cast<const void *>(&bwd_elem_dx_kernel<T, WT, kRms, true>), 256};
        t.elem_dx[kLayer][0] =
            KernelRef{reinterpret_cast<const void *>(&bwd_elem_dx_kernel<T, WT, kLayer, false>), 256};
        t.elem_dx[kLayer][1] =
            KernelRef{reinterpret_cast<const void *>(&bwd_elem_dx_kernel<T, WT, kLayer, true>), 256};
        t.elem_dw[kRms] = KernelRef{reinterpret_cast<const void *>(&bwd_elem_dw_kernel<T, kRms>), 256};
        t.elem_dw[kLayer] =
            KernelRef{reinterpret_cast<const void *>(&bwd_elem_dw_kernel<T, kLayer>), 256};
        return t;
    }
};

} // namespace addrms
