// Device-side building blocks for the gfx950 RMSNorm kernels: 128-bit vector
// element access, bfloat16 and float16 packing, and the wave64 / workgroup
// float sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace addrms {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Storage tags for bfloat16 (the upper half of a binary32) and IEEE binary16;
// never computed on.
struct bf16_t {
    uint16_t bits;
};
struct f16_t {
    uint16_t bits;
};

// Elements of T in one 16-byte vector.
template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int n = 4; };
template <> struct Vec<bf16_t> { static constexpr int n = 8; };
template <> struct Vec<f16_t> { static constexpr int n = 8; };

// ---- bfloat16 <-> float ------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bfloat16 in one dword (a in the low half), each rounded to
// nearest-even by the hardware converter v_cvt_pk_bf16_f32 (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float a) { return (uint16_t)pack_bf16x2(a, 0.0f); }

// ---- binary16 <-> float ----------------------------------------------------

// The two binary16 values of a dword (low half first), widened exactly.
__device__ __forceinline__ f32x2 f16x2_to_f32(uint32_t u)
{
    return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
}

// Two floats -> two binary16 in one dword (a in the low half), each rounded
// to nearest-even by the hardware conversion (overflow to infinity, subnormal
// results kept, NaN stays NaN).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ uint16_t to_f16(float a) { return (uint16_t)pack_f16x2(a, 0.0f); }

// The two 16-bit values of a dword of type T (bf16_t or f16_t), as floats.
template <typename T> __device__ __forceinline__ void widen2(uint32_t u, float &lo, float &hi)
{
    if constexpr (__is_same(T, f16_t)) {
        const f32x2 f = f16x2_to_f32(u);
        lo = f[0];
        hi = f[1];
    } else {
        lo = bf16_lo(u);
        hi = bf16_hi(u);
    }
}

// ---- one 16-byte vector <-> floats -------------------------------------------

template <typename T>
__device__ __forceinline__ void unpack(const u32x4 &v, float (&f)[Vec<T>::n]);

template <>
__device__ __forceinline__ void unpack<float>(const u32x4 &v, float (&f)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f[i] = __uint_as_float(v[i]);
}

template <>
__device__ __forceinline__ void unpack<bf16_t>(const u32x4 &v, float (&f)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
}

template <>
__device__ __forceinline__ void unpack<f16_t>(const u32x4 &v, float (&f)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        widen2<f16_t>(v[i], f[2 * i], f[2 * i + 1]);
}

template <typename T>
__device__ __forceinline__ u32x4 pack(const float (&f)[Vec<T>::n]);

template <>
__device__ __forceinline__ u32x4 pack<float>(const float (&f)[4])
{
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = __float_as_uint(f[i]);
    return v;
}

template <>
__device__ __forceinline__ u32x4 pack<bf16_t>(const float (&f)[8])
{
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
}

template <>
__device__ __forceinline__ u32x4 pack<f16_t>(const float (&f)[8])
{
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = pack_f16x2(f[2 * i], f[2 * i + 1]);
    return v;
}

// ---- global memory -----------------------------------------------------------

// Streaming loads/stores of row data.  Policy bits: 1 = non-temporal loads,
// 2 = non-temporal stores (the data is touched once; keep it out of the way
// of the weight vector in the caches).
template <int POL>
__device__ __forceinline__ u32x4 ld_stream(const u32x4 *p)
{
    if constexpr (POL & 1)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int POL>
__device__ __forceinline__ void st_stream(u32x4 *p, const u32x4 &v)
{
    if constexpr (POL & 2)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// The weights matching vector index v of a row of T: Vec<T>::n consecutive
// elements of w (stored as WT), kept in their stored form (2, 4 or 8 dwords)
// so that a kernel can hold them in registers across rows and widen them at
// each use.  w is 16-byte aligned.
template <typename T, typename WT> struct WRaw {
    static constexpr int dw = Vec<T>::n * (int)sizeof(WT) / 4;
    uint32_t d[dw];
};

template <typename T, typename WT>
__device__ __forceinline__ WRaw<T, WT> ld_w_raw(const void *w, int v)
{
    constexpr int dw = WRaw<T, WT>::dw;
    WRaw<T, WT> r;
    if constexpr (dw == 2) { // bf16 weights, float rows
        const u32x2 a = reinterpret_cast<const u32x2 *>(w)[v];
        r.d[0] = a[0];
        r.d[1] = a[1];
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(w) + (dw / 4) * v;
#pragma unroll
        for (int h = 0; h < dw / 4; ++h) {
            const u32x4 a = p[h];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r.d[4 * h + i] = a[i];
        }
    }
    return r;
}

template <typename T, typename WT>
__device__ __forceinline__ void unpack_w(const WRaw<T, WT> &r, float (&f)[Vec<T>::n])
{
    constexpr int n = Vec<T>::n;
    if constexpr (sizeof(WT) == 4) {
#pragma unroll
        for (int i = 0; i < n; ++i)
            f[i] = __uint_as_float(r.d[i]);
    } else {
#pragma unroll
        for (int i = 0; i < n / 2; ++i)
            widen2<WT>(r.d[i], f[2 * i], f[2 * i + 1]);
    }
}

// The same weights loaded and widened to floats in one step.
template <typename T, typename WT>
__device__ __forceinline__ void load_w(const void *w, int v, float (&f)[Vec<T>::n])
{
    unpack_w<T, WT>(ld_w_raw<T, WT>(w, v), f);
}

// Scalar element access for the unaligned/element-wise path.
template <typename T> __device__ __forceinline__ float ld_elem(const void *p, int64_t i);
template <> __device__ __forceinline__ float ld_elem<float>(const void *p, int64_t i)
{
    return reinterpret_cast<const float *>(p)[i];
}
template <> __device__ __forceinline__ float ld_elem<bf16_t>(const void *p, int64_t i)
{
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
}
template <> __device__ __forceinline__ float ld_elem<f16_t>(const void *p, int64_t i)
{
    return (float)reinterpret_cast<const _Float16 *>(p)[i];
}
template <typename T> __device__ __forceinline__ void st_elem(void *p, int64_t i, float v);
template <> __device__ __forceinline__ void st_elem<float>(void *p, int64_t i, float v)
{
    reinterpret_cast<float *>(p)[i] = v;
}
template <> __device__ __forceinline__ void st_elem<bf16_t>(void *p, int64_t i, float v)
{
    reinterpret_cast<uint16_t *>(p)[i] = to_bf16(v);
}
template <> __device__ __forceinline__ void st_elem<f16_t>(void *p, int64_t i, float v)
{
    reinterpret_cast<uint16_t *>(p)[i] = to_f16(v);
}
// The value an element has once stored as T (the rounding a store applies).
template <typename T> __device__ __forceinline__ float as_stored(float v);
template <> __device__ __forceinline__ float as_stored<float>(float v) { return v; }
template <> __device__ __forceinline__ float as_stored<bf16_t>(float v)
{
    return __uint_as_float((uint32_t)to_bf16(v) << 16);
}
template <> __device__ __forceinline__ float as_stored<f16_t>(float v)
{
    return (float)__builtin_bit_cast(_Float16, to_f16(v));
}

// ---- reductions --------------------------------------------------------------

#define ADDRMS_DPP(v, ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))

// Sum over the 64 lanes of a wave, result in every lane (a wave-uniform value).
// Within each 16-lane row: DPP quad_perm [1,0,3,2] and [2,3,0,1] give quad
// sums, row_half_mirror pairs quads into 8-lane sums, row_mirror pairs halves
// into 16-lane sums.  The four row sums are then read with v_readlane.  Every
// lane must be active.  The order is fixed, so results are deterministic.
__device__ __forceinline__ float wave_sum(float v)
{
    v += ADDRMS_DPP(v, 0xB1);  // quad_perm [1,0,3,2]
    v += ADDRMS_DPP(v, 0x4E);  // quad_perm [2,3,0,1]
    v += ADDRMS_DPP(v, 0x141); // row_half_mirror
    v += ADDRMS_DPP(v, 0x140); // row_mirror
    const int b = __builtin_bit_cast(int, v);
    float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Maximum over the 64 lanes of a wave (same DPP pattern as wave_sum), result
// in every lane.  v_max_f32 follows IEEE maxNum: a NaN operand is ignored.
__device__ __forceinline__ float wave_max(float v)
{
    v = __builtin_fmaxf(v, ADDRMS_DPP(v, 0xB1));
    v = __builtin_fmaxf(v, ADDRMS_DPP(v, 0x4E));
    v = __builtin_fmaxf(v, ADDRMS_DPP(v, 0x141));
    v = __builtin_fmaxf(v, ADDRMS_DPP(v, 0x140));
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

// ---- FP8 (OCP E4M3) -----------------------------------------------------------

// Clamp to the E4M3 range [-448, 448], keeping NaN (comparisons with NaN are
// false, so NaN passes through unchanged).
__device__ __forceinline__ float e4m3_clamp(float v)
{
    return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);
}

#ifndef ADDRMS_FP8_SOFTWARE
#define ADDRMS_FP8_SOFTWARE 0
#endif

// Two floats already in [-448, 448] (or NaN) -> two E4M3 codes in the low 16
// bits (a in the low byte).  Hardware: v_cvt_pk_fp8_f32, gfx950's converter to
// the OCP E4M3 format, round-to-nearest-even.  Software (the alternative,
// written from the format): RNE on the binary32 bit pattern for normals,
// rint(v * 2^9) on the subnormal grid.
__device__ __forceinline__ uint32_t e4m3_sw(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7Fu;
    const float av = __uint_as_float(a);
    if (av < 0x1p-6f)
        return sign | (uint32_t)__builtin_rintf(av * 512.0f); // m * 2^-9, m <= 8
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) & 0xFFF00000u; // keep 3 mantissa bits
    return sign | ((((r >> 23) - 127u + 7u) & 0xFu) << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ uint32_t pack_e4m3x2(float a, float b)
{
#if ADDRMS_FP8_SOFTWARE
    return e4m3_sw(a) | (e4m3_sw(b) << 8);
#else
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
#endif
}

// OCP FP4 E2M1 code (4 bits) of v: nearest of the magnitudes 0, 0.5, 1, 1.5,
// 2, 3, 4, 6, ties to the even code, larger magnitudes saturating to 6, sign
// kept.  The code is the number of rounding thresholds |v| has passed; each
// threshold is a midpoint of the grid, taken with > where the lower code is
// even (a tie stays) and >= where it is odd (a tie moves up).  NaN gives 0
// or 8 (callers handle NaN blocks themselves).
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    const float a = __builtin_fabsf(v);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 0x8u);
}

#ifndef ADDRMS_FP4_SOFTWARE
#define ADDRMS_FP4_SOFTWARE 0
#endif

// Two floats, already divided by their block's scale, -> two E2M1 codes in
// byte SEL of `old` (a in the low nibble), the other bytes of `old` kept.
// Hardware: gfx950's v_cvt_scalef32_pk_fp4_f32 with a scale of 1.  Checked
// on MI355X against the oracle's encoder over every grid point, midpoint and
// neighbouring float of the E2M1 range, a dense sweep of [-10, 10], zeros and
// subnormals, with power-of-two scales: round to nearest even, saturating at
// 6, the sign kept for zero and subnormal inputs; the instruction divides by
// its scale.  Software (the alternative): e2m1_code above.
template <int SEL> __device__ __forceinline__ uint32_t pack_e2m1x2(uint32_t old, float a, float b)
{
#if ADDRMS_FP4_SOFTWARE
    return (old & ~(0xFFu << (8 * SEL))) | ((e2m1_code(a) | (e2m1_code(b) << 4)) << (8 * SEL));
#else
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
#endif
}

// E8M0 exponent of an MX block from its largest magnitude g (finite, >= 0):
// floor(log2(g)) - 2, clamped below at -127 (zero and tiny blocks).
__device__ __forceinline__ int mx_exponent(float g)
{
    const int ef = (int)((__float_as_uint(g) >> 23) & 0xFFu);
    const int e = ef == 0 ? -127 : ef - 129;
    return e < -127 ? -127 : e;
}

// One DPP move of a float within 16-lane rows (source lanes must be active).
template <int CTRL> __device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum over each aligned group of L lanes (L a power of two up to 64, the
// same for the whole wave); every lane of a group gets the group's maximum.
// The DPP steps of wave_max within 16-lane rows, then lane shuffles by 16 and
// 32.  Every lane of a group must be active.
__device__ __forceinline__ float group_max(float v, int L)
{
    // every step runs and its result is selected (no branches, so no exec
    // masks to keep across a caller's unrolled loop)
    v = __builtin_fmaxf(v, L >= 2 ? dpp_f32<0xB1>(v) : v);
    v = __builtin_fmaxf(v, L >= 4 ? dpp_f32<0x4E>(v) : v);
    v = __builtin_fmaxf(v, L >= 8 ? dpp_f32<0x141>(v) : v);
    v = __builtin_fmaxf(v, L >= 16 ? dpp_f32<0x140>(v) : v);
    const float t16 = __shfl_xor(v, 16);
    v = __builtin_fmaxf(v, L >= 32 ? t16 : v);
    const float t32 = __shfl_xor(v, 32);
    return __builtin_fmaxf(v, L >= 64 ? t32 : v);
}

// Maximum over each aligned group of L lanes, L a compile-time power of two
// up to 16 (the DPP steps of group_max only).
template <int L> __device__ __forceinline__ float group_max_n(float v)
{
    static_assert(L >= 1 && L <= 16 && (L & (L - 1)) == 0, "L: power of two up to 16");
    if constexpr (L >= 2)
        v = __builtin_fmaxf(v, dpp_f32<0xB1>(v));
    if constexpr (L >= 4)
        v = __builtin_fmaxf(v, dpp_f32<0x4E>(v));
    if constexpr (L >= 8)
        v = __builtin_fmaxf(v, dpp_f32<0x141>(v));
    if constexpr (L >= 16)
        v = __builtin_fmaxf(v, dpp_f32<0x140>(v));
    return v;
}

// The same sum for doubles (each DPP step moves both 32-bit halves).
template <int CTRL> __device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

#undef ADDRMS_DPP

} // namespace addrms
