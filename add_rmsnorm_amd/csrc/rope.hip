// Per-head RMSNorm followed by the rotary position embedding, in one pass, for
// the query and key heads of an attention layer: HIP kernels for gfx950 and
// their table for one (row dtype, weight dtype) combination, selected at
// compile time by ADDRMS_COMBO (combo_types.hpp).
//
// The "Machete" README lists RMSNorm and RoPE side by side among the ops its
// persistent kernels compose ("Built-In Areas").  They meet where each query
// and key head is RMS-normalised over its D values and then rotated by the
// token's position (RoFormer, Su et al. 2021): every pair (a, b) of
// normalised values becomes (a*c - b*s, b*c + a*s), with c and s read from
// the caller's float32 tables at the token's position.  Two pair layouts:
// rotate-half, pair i = (i, i + D/2); interleaved, pair i = (2i, 2i + 1).
//
// The work streams heads through registers exactly once, so it is bound by
// HBM like the other norms.  A head is handled by G lanes (a power of two).
// Lane g holds the two 16-byte vectors at columns g*E and D/2 + g*E, where E
// is the number of values per vector.  Both members of every rotate-half pair
// are therefore in the same lane, and interleaved pairs lie inside each
// vector, so the rotation needs no data from other lanes.  Only the head's sum
// of squares crosses lanes: DPP steps within the group (and a lane shuffle
// for groups of 32 or 64).  The tables and weights are read with the default
// cache policy (every head of a token reuses the token's table row).  The head
// data is streamed non-temporally.
#include <utility>

#include "device.hpp"
#include "internal.hpp"

#include "combo_types.hpp"

#ifndef ADDRMS_STREAM_POLICY
#define ADDRMS_STREAM_POLICY 3
#endif

namespace addrms {

constexpr int kRopePol = ADDRMS_STREAM_POLICY;

// Sum over each aligned group of G lanes (G a power of two up to 64); every
// lane of a group gets the same value.  Within 16-lane rows: DPP quad_perm
// [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror (the pattern of
// wave_sum); across rows, lane shuffles by 16 and 32.
template <int G> __device__ __forceinline__ float group_sum(float v)
{
    if constexpr (G >= 2)
        v += dpp_f32<0xB1>(v);
    if constexpr (G >= 4)
        v += dpp_f32<0x4E>(v);
    if constexpr (G >= 8)
        v += dpp_f32<0x141>(v);
    if constexpr (G >= 16)
        v += dpp_f32<0x140>(v);
    if constexpr (G >= 32)
        v += __shfl_xor(v, 16);
    if constexpr (G >= 64)
        v += __shfl_xor(v, 32);
    return v;
}

// Streaming 16-byte store through an explicitly global pointer: the output
// pointers pass through per-head arrays, where the compiler no longer proves
// them global and would otherwise emit flat stores.
typedef __attribute__((address_space(1))) u32x4 global_u32x4;
__device__ __forceinline__ void st_global(void *p, const u32x4 &v)
{
    global_u32x4 *g = (global_u32x4 *)p;
    if constexpr (kRopePol & 2)
        __builtin_nontemporal_store(v, g);
    else
        *g = v;
}

// K consecutive float32 values (K = 2, 4 or 8) from p, which is 8-byte
// aligned for K = 2 and 16-byte aligned otherwise.
template <int K> __device__ __forceinline__ void ld_f32(const float *p, float (&f)[K])
{
    if constexpr (K == 2) {
        const u32x2 a = *reinterpret_cast<const u32x2 *>(p);
        f[0] = __uint_as_float(a[0]);
        f[1] = __uint_as_float(a[1]);
    } else {
#pragma unroll
        for (int j = 0; j < K / 4; ++j) {
            const u32x4 a = reinterpret_cast<const u32x4 *>(p)[j];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[4 * j + e] = __uint_as_float(a[e]);
        }
    }
}

// Token and head of flat head index i (heads of a token are consecutive).
__device__ __forceinline__ void split_head(int64_t i, int H, bool narrow, int64_t &t, int &h)
{
    if (narrow) { // every index fits 32 bits: the cheaper division
        const uint32_t u = (uint32_t)i, q = u / (uint32_t)H;
        t = q;
        h = (int)(u - q * (uint32_t)H);
    } else {
        t = i / H;
        h = (int)(i - t * H);
    }
}

// Where head i of the flat (token, head) order lives: input, output, weights
// and token.
template <typename T> struct HeadRef {
    const T *src;
    T *dst;
    const void *w;
    int64_t t;
    bool isq; // a query head (weights wq), else a key head (wk)
};

template <typename T>
__device__ __forceinline__ HeadRef<T> locate(const RopeArgs &a, int64_t i, int H, bool narrow)
{
    int64_t t;
    int h;
    split_head(i, H, narrow, t, h);
    HeadRef<T> r;
    r.t = t;
    r.isq = h < a.Hq;
    if (r.isq) {
        r.src = static_cast<const T *>(a.q) + t * a.q_stride + (int64_t)h * a.D;
        r.dst = static_cast<T *>(a.qo) + t * a.qo_stride + (int64_t)h * a.D;
        r.w = a.wq;
    } else {
        r.src = static_cast<const T *>(a.k) + t * a.k_stride + (int64_t)(h - a.Hq) * a.D;
        r.dst = static_cast<T *>(a.ko) + t * a.ko_stride + (int64_t)(h - a.Hq) * a.D;
        r.w = a.wk;
    }
    return r;
}

// The lane's table values for one position: rotate-half pairs use columns
// c0 .. c0+E-1; interleaved pairs use c0/2 .. c0/2+E/2-1 (first vector) and
// c1/2 .. c1/2+E/2-1 (second vector).
template <int E, bool IL> struct TableCols {
    float c[E], s[E];
};

template <int E, bool IL>
__device__ __forceinline__ void load_cols(const RopeArgs &a, int64_t p, int c0, int c1, int half,
                                          TableCols<E, IL> &tc)
{
    const float *cr = a.cos + p * half, *sr = a.sin + p * half;
    if constexpr (!IL) {
        ld_f32<E>(cr + c0, tc.c);
        ld_f32<E>(sr + c0, tc.s);
    } else {
        float h0[E / 2], h1[E / 2];
        ld_f32<E / 2>(cr + c0 / 2, h0);
        ld_f32<E / 2>(cr + c1 / 2, h1);
#pragma unroll
        for (int j = 0; j < E / 2; ++j) {
            tc.c[j] = h0[j];
            tc.c[E / 2 + j] = h1[j];
        }
        ld_f32<E / 2>(sr + c0 / 2, h0);
        ld_f32<E / 2>(sr + c1 / 2, h1);
#pragma unroll
        for (int j = 0; j < E / 2; ++j) {
            tc.s[j] = h0[j];
            tc.s[E / 2 + j] = h1[j];
        }
    }
}

// One head on its G lanes, from the lane's two loaded vectors (columns c0 and
// c1 = D/2 + c0): the head's sum of squares over the group, rstd, the
// normalised values, the rotation by the table columns tc (ok = the position
// has a table row; otherwise the head is NaN), and the two stores.  Every
// lane of the group must call it.
template <typename T, int G, bool IL>
__device__ __forceinline__ void rope_head(const RopeArgs &a, const u32x4 &va, const u32x4 &vb,
                                          bool ok, const TableCols<Vec<T>::n, IL> &tc,
                                          const float (&wa)[Vec<T>::n],
                                          const float (&wb)[Vec<T>::n], T *dst, int c0, int c1,
                                          float inv_d)
{
    constexpr int E = Vec<T>::n;
    float xa[E], xb[E];
    unpack<T>(va, xa);
    unpack<T>(vb, xb);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        ss = __builtin_fmaf(xa[e], xa[e], ss);
        ss = __builtin_fmaf(xb[e], xb[e], ss);
    }
    ss = group_sum<G>(ss);
    const float rs = 1.0f / __builtin_sqrtf(ss * inv_d + a.eps);

    float ya[E], yb[E];
    if (!ok) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            ya[e] = yb[e] = __builtin_nanf("");
    } else {
        float na[E], nb[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            na[e] = (xa[e] * rs) * wa[e];
            nb[e] = (xb[e] * rs) * wb[e];
        }
        if constexpr (!IL) {
            // pair (c0 + e, c1 + e) uses table column c0 + e
#pragma unroll
            for (int e = 0; e < E; ++e) {
                ya[e] = na[e] * tc.c[e] - nb[e] * tc.s[e];
                yb[e] = nb[e] * tc.c[e] + na[e] * tc.s[e];
            }
        } else {
            // pairs (2j, 2j + 1) inside each vector
#pragma unroll
            for (int j = 0; j < E / 2; ++j) {
                const float ca = tc.c[j], sa = tc.s[j], cb = tc.c[E / 2 + j], sb = tc.s[E / 2 + j];
                ya[2 * j] = na[2 * j] * ca - na[2 * j + 1] * sa;
                ya[2 * j + 1] = na[2 * j + 1] * ca + na[2 * j] * sa;
                yb[2 * j] = nb[2 * j] * cb - nb[2 * j + 1] * sb;
                yb[2 * j + 1] = nb[2 * j + 1] * cb + nb[2 * j] * sb;
            }
        }
    }
    st_global(dst + c0, pack<T>(ya));
    st_global(dst + c1, pack<T>(yb));
}

// 16-byte vector path: D = 2 * E * G, every pointer 16-byte aligned and every
// token stride a multiple of 16 bytes.  A block of 256 lanes holds 256 / G
// groups; in each step of its grid-stride loop a group takes HPL consecutive
// heads (mostly of one token) and issues all of their loads before any
// arithmetic.  The lane's query and key weights are loaded once, and a table
// row is loaded once per run of equal positions.  Whether a head exists
// depends only on the group, so the group reductions always see their own
// lanes active.
template <typename T, typename WT, int G, bool IL, int HPL>
__global__ __launch_bounds__(kRopeBlock) void rope_vec_kernel(RopeArgs a)
{
    constexpr int E = Vec<T>::n;
    constexpr int GPB = kRopeBlock / G;
    constexpr int STEP = GPB * HPL;
    const int g = (int)threadIdx.x % G, gi = (int)threadIdx.x / G;
    const int H = a.Hq + a.Hk;
    const int64_t total = a.T * H;
    const bool narrow = total <= (int64_t)UINT32_MAX;
    const int half = a.D / 2;
    const float inv_d = 1.0f / (float)a.D;
    const int c0 = g * E, c1 = half + g * E;

    float wqa[E], wqb[E], wka[E], wkb[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        wqa[e] = wqb[e] = wka[e] = wkb[e] = 0.0f;
    if (a.Hq > 0) {
        load_w<T, WT>(a.wq, c0 / E, wqa);
        load_w<T, WT>(a.wq, c1 / E, wqb);
    }
    if (a.Hk > 0) {
        load_w<T, WT>(a.wk, c0 / E, wka);
        load_w<T, WT>(a.wk, c1 / E, wkb);
    }

    for (int64_t base = (int64_t)blockIdx.x * STEP + (int64_t)gi * HPL; base < total;
         base += (int64_t)gridDim.x * STEP) {
        u32x4 va[HPL], vb[HPL];
        int64_t p[HPL];
        T *dst[HPL];
        bool isq[HPL];
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
            va[j] = vb[j] = u32x4{0u, 0u, 0u, 0u};
            p[j] = -1;
            dst[j] = nullptr;
            isq[j] = true;
            if (base + j < total) {
                const HeadRef<T> r = locate<T>(a, base + j, H, narrow);
                va[j] = ld_stream<kRopePol>(reinterpret_cast<const u32x4 *>(r.src + c0));
                vb[j] = ld_stream<kRopePol>(reinterpret_cast<const u32x4 *>(r.src + c1));
                p[j] = a.pos[r.t];
                dst[j] = r.dst;
                isq[j] = r.isq;
            }
        }
        TableCols<E, IL> tc;
        int64_t loaded = -1;
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
            if (base + j >= total)
                break;
            const bool ok = p[j] >= 0 && p[j] < a.P;
            if (ok && p[j] != loaded) {
                load_cols<E, IL>(a, p[j], c0, c1, half, tc);
                loaded = p[j];
            }
            rope_head<T, G, IL>(a, va[j], vb[j], ok, tc, isq[j] ? wqa : wka, isq[j] ? wqb : wkb,
                                dst[j], c0, c1, inv_d);
        }
    }
}

// Element-wise path: any even D, any alignment and stride.  One wave per head
// (grid-stride over heads): pass 1 sums the squares, pass 2 re-reads each pair
// (from cache), normalises, rotates and stores it.  Each lane writes only the
// pairs it read, so the output may be the input.
template <typename T, typename WT, bool IL>
__global__ __launch_bounds__(64) void rope_elem_kernel(RopeArgs a)
{
    const int lane = (int)threadIdx.x;
    const int H = a.Hq + a.Hk;
    const int64_t total = a.T * H;
    const bool narrow = total <= (int64_t)UINT32_MAX;
    const int half = a.D / 2;
    const float inv_d = 1.0f / (float)a.D;

    for (int64_t head = blockIdx.x; head < total; head += gridDim.x) {
        const HeadRef<T> r = locate<T>(a, head, H, narrow);
        const T *src = r.src;
        T *dst = r.dst;
        const void *w = r.w;
        const int64_t t = r.t;

        float ss = 0.0f;
        for (int i = lane; i < half; i += 64) {
            const int ja = IL ? 2 * i : i, jb = IL ? 2 * i + 1 : i + half;
            const float xa = ld_elem<T>(src, ja), xb = ld_elem<T>(src, jb);
            ss = __builtin_fmaf(xa, xa, ss);
            ss = __builtin_fmaf(xb, xb, ss);
        }
        ss = wave_sum(ss);
        const float rs = 1.0f / __builtin_sqrtf(ss * inv_d + a.eps);
        const int64_t p = a.pos[t];
        const bool bad = p < 0 || p >= a.P;

        for (int i = lane; i < half; i += 64) {
            const int ja = IL ? 2 * i : i, jb = IL ? 2 * i + 1 : i + half;
            float ya = __builtin_nanf(""), yb = __builtin_nanf("");
            if (!bad) {
                const float na = (ld_elem<T>(src, ja) * rs) * ld_elem<WT>(w, ja);
                const float nb = (ld_elem<T>(src, jb) * rs) * ld_elem<WT>(w, jb);
                const float c = a.cos[p * half + i], s = a.sin[p * half + i];
                ya = na * c - nb * s;
                yb = nb * c + na * s;
            }
            st_elem<T>(dst, ja, ya);
            st_elem<T>(dst, jb, yb);
        }
    }
}

template <typename T, typename WT> struct RopeBuilder {
    template <bool IL, int G, int HPL> static KernelRef vec_ref()
    {
        if constexpr (rope_built(G, HPL))
            return KernelRef{reinterpret_cast<const void *>(&rope_vec_kernel<T, WT, G, IL, HPL>),
                             kRopeBlock};
        else
            return KernelRef{nullptr, 0};
    }
    template <bool IL, int LG, int... LH>
    static void vec_cell(KernelRef (&cell)[kRopeNumHpl], std::integer_sequence<int, LH...>)
    {
        ((cell[LH] = vec_ref<IL, (1 << LG), (1 << LH)>()), ...);
    }
    template <bool IL, int... LG>
    static void vec_row(KernelRef (&row)[kRopeNumGroups][kRopeNumHpl],
                        std::integer_sequence<int, LG...>)
    {
        (vec_cell<IL, LG>(row[LG], std::make_integer_sequence<int, kRopeNumHpl>{}), ...);
    }
    static RopeTable build()
    {
        RopeTable t{};
        vec_row<false>(t.vec[0], std::make_integer_sequence<int, kRopeNumGroups>{});
        vec_row<true>(t.vec[1], std::make_integer_sequence<int, kRopeNumGroups>{});
        t.elem[0] = KernelRef{reinterpret_cast<const void *>(&rope_elem_kernel<T, WT, false>), 64};
        t.elem[1] = KernelRef{reinterpret_cast<const void *>(&rope_elem_kernel<T, WT, true>), 64};
        return t;
    }
};

const RopeTable &ADDRMS_CAT(rope_table_, ADDRMS_COMBO)()
{
    static const RopeTable t = RopeBuilder<ADDRMS_ROW_T, ADDRMS_W_T>::build();
    return t;
}

} // namespace addrms
