// C ABI of the library (declared in include/addrms.h): argument validation,
// variant choice, grid sizing and launch on the caller's stream.
//
// Validation happens before any HIP call.  The library allocates nothing; the
// only state is a per-device cache of CU counts and kernel occupancies.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "addrms.h"
#include "internal.hpp"

namespace addrms {

// One table of each kind per (row dtype, weight dtype) combination, from
// tables.hip and rope.hip compiled once per ADDRMS_COMBO (0..8).
#define ADDRMS_DECLARE_COMBO(c)                                                                   \
    const FwdTable &fwd_table_##c();                                                              \
    const BwdTable &bwd_table_##c();                                                              \
    const RopeTable &rope_table_##c();
ADDRMS_DECLARE_COMBO(0)
ADDRMS_DECLARE_COMBO(1)
ADDRMS_DECLARE_COMBO(2)
ADDRMS_DECLARE_COMBO(3)
ADDRMS_DECLARE_COMBO(4)
ADDRMS_DECLARE_COMBO(5)
ADDRMS_DECLARE_COMBO(6)
ADDRMS_DECLARE_COMBO(7)
ADDRMS_DECLARE_COMBO(8)
#undef ADDRMS_DECLARE_COMBO

#define ADDRMS_TABLE_SWITCH(kind, c)                                                              \
    switch (c) {                                                                                  \
    case 0: return kind##_0();                                                                    \
    case 1: return kind##_1();                                                                    \
    case 2: return kind##_2();                                                                    \
    case 3: return kind##_3();                                                                    \
    case 4: return kind##_4();                                                                    \
    case 5: return kind##_5();                                                                    \
    case 6: return kind##_6();                                                                    \
    case 7: return kind##_7();                                                                    \
    default: return kind##_8();                                                                   \
    }

const FwdTable &fwd_table(int c) { ADDRMS_TABLE_SWITCH(fwd_table, c) }
const BwdTable &bwd_table(int c) { ADDRMS_TABLE_SWITCH(bwd_table, c) }
const RopeTable &rope_table(int c) { ADDRMS_TABLE_SWITCH(rope_table, c) }
#undef ADDRMS_TABLE_SWITCH

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxPartials = 1024; // dw partial rows (workspace rows)
constexpr int kRopeHpl = 4;            // RMSNorm + RoPE: heads per lane group and step
constexpr size_t kMaxDynLds = 65536;

int fail_hip(hipError_t e)
{
    g_last_hip_error = (int)e;
    return ADDRMS_ERR_HIP;
}

bool dtype_ok(int d) { return d == ADDRMS_F32 || d == ADDRMS_BF16 || d == ADDRMS_F16; }
size_t esize(int d) { return d == ADDRMS_F32 ? 4 : 2; }
int vec_elems(int d) { return d == ADDRMS_F32 ? 4 : 8; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tuning knobs (ADDRMS_KNOB_* in addrms.h): 0 means the measured default.
// Each starts from its environment variable, read once when the library is
// loaded; addrms_tune changes it afterwards (tests use it to force every
// variant through parity inside one process).
const char *const kKnobEnv[ADDRMS_NUM_KNOBS] = {
    "ADDRMS_FWD_WPR",      "ADDRMS_FWD_VPL",        "ADDRMS_BWD_WPR",
    "ADDRMS_BWD_WIDE",     "ADDRMS_BWD_PREFETCH",   "ADDRMS_FORCE_ELEM",
    "ADDRMS_MAX_PARTIALS", "ADDRMS_BLOCKS_PER_CU",  "ADDRMS_ROPE_BLOCKS_PER_CU",
    "ADDRMS_ROPE_HPL",
};

struct Knobs {
    std::atomic<int> v[ADDRMS_NUM_KNOBS];
    Knobs()
    {
        for (int k = 0; k < ADDRMS_NUM_KNOBS; ++k) {
            const char *s = std::getenv(kKnobEnv[k]);
            const int x = s ? std::atoi(s) : 0;
            v[k].store(x > 0 ? x : 0, std::memory_order_relaxed);
        }
    }
};
Knobs g_knobs; // constructed when the library is loaded

int knob(int k) { return g_knobs.v[k].load(std::memory_order_relaxed); }

// Byte range of a buffer.
struct Span {
    uintptr_t lo = 0, hi = 0;
};
Span span(const void *p, size_t bytes)
{
    Span s;
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + bytes;
    return s;
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
// An output may be the very same buffer as an input of its shape, or disjoint.
bool bad_alias(Span out, Span in, bool same_ok)
{
    if (!overlaps(out, in))
        return false;
    return !(same_ok && out.lo == in.lo && out.hi == in.hi);
}

// Shape check shared by every entry point: M >= 0, N >= 1, N and the element
// count in range.
int check_shape(int64_t M, int64_t N, int dtype)
{
    if (M < 0 || N <= 0 || N > INT_MAX)
        return ADDRMS_ERR_SHAPE;
    if (M > 0 && (uint64_t)M > ((uint64_t)1 << 62) / ((uint64_t)N * esize(dtype)))
        return ADDRMS_ERR_SHAPE;
    return ADDRMS_OK;
}

// ---- device facts (cached) --------------------------------------------------

std::mutex g_mu;
std::map<int, int> g_cus;
std::map<std::tuple<int, const void *, size_t>, int> g_occ;

int device_cus(int dev, int *cus)
{
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_cus.find(dev);
        if (it != g_cus.end()) {
            *cus = it->second;
            return ADDRMS_OK;
        }
    }
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return fail_hip(e);
    std::lock_guard<std::mutex> lk(g_mu);
    g_cus[dev] = n;
    *cus = n;
    return ADDRMS_OK;
}

// Resident blocks per CU of a kernel (the BLOCKS_PER_CU knob overrides).
int blocks_per_cu(int dev, const KernelRef &k, size_t smem, int *out)
{
    const int forced = knob(ADDRMS_KNOB_BLOCKS_PER_CU);
    if (forced > 0) {
        *out = forced;
        return ADDRMS_OK;
    }
    auto key = std::make_tuple(dev, k.fn, smem);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_occ.find(key);
        if (it != g_occ.end()) {
            *out = it->second;
            return ADDRMS_OK;
        }
    }
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k.fn, k.block, smem);
    if (e != hipSuccess)
        return fail_hip(e);
    if (n < 1)
        n = 1;
    std::lock_guard<std::mutex> lk(g_mu);
    g_occ[key] = n;
    *out = n;
    return ADDRMS_OK;
}

// Persistent grid: no more blocks than the device holds at once, and no more
// than there is work for.
int persistent_grid(const KernelRef &k, size_t smem, int64_t blocks_needed, int64_t cap,
                    int *grid)
{
    int dev = 0, cus = 0, per_cu = 0, rc;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail_hip(e);
    if ((rc = device_cus(dev, &cus)) != ADDRMS_OK)
        return rc;
    if ((rc = blocks_per_cu(dev, k, smem, &per_cu)) != ADDRMS_OK)
        return rc;
    int64_t g = (int64_t)cus * per_cu;
    if (g > blocks_needed)
        g = blocks_needed;
    if (g > cap)
        g = cap;
    if (g < 1)
        g = 1;
    *grid = (int)g;
    return ADDRMS_OK;
}

int launch(const KernelRef &k, dim3 grid, size_t smem, void *args, hipStream_t s)
{
    void *argv[] = {args};
    hipError_t e = hipLaunchKernel(k.fn, grid, dim3(k.block), argv, smem, s);
    if (e != hipSuccess)
        return fail_hip(e);
    return ADDRMS_OK;
}

int device_cus_current(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail_hip(e);
    // the last device this thread asked about, without the lock and map
    thread_local int tl_dev = -1, tl_cus = 0;
    if (dev == tl_dev) {
        *cus = tl_cus;
        return ADDRMS_OK;
    }
    const int rc = device_cus(dev, cus);
    if (rc == ADDRMS_OK) {
        tl_dev = dev;
        tl_cus = *cus;
    }
    return rc;
}

// Index of the smallest supported VPL >= need, or -1.
int vpl_index(int need)
{
    for (int i = 0; i < kNumVpl; ++i)
        if (kVplList[i] >= need)
            return i;
    return -1;
}

// Forward variant.  A row is spread over enough waves that each lane holds
// about ADDRMS_FWD_VPL (default 2) 16-byte vectors per tensor, or up to 4 with
// 8 waves per row: measured on MI355X, short per-lane chains in many small
// row-blocks keep more rows in flight and stream fastest (fused bf16 16384 x
// 7168: 8 waves per row reach 6.2 TB/s, one wave per row 5.5 TB/s), but
// 1024-thread blocks (16 waves per row) hold at most two rows per CU: at
// 12288 and 16384 columns 8 waves with 3 or 4 vectors a lane beat 16 with 2
// (fused 6.0-6.1 against 5.8-5.9 TB/s; the E4M3 and MXFP4 outputs, with a
// second row reduction or more registers, 5.7-6.2 against 4.5-5.1).  When
// there are too few rows to give every SIMD a wave, rows get more waves
// still.
//
// Measured exceptions for plain (unquantised) outputs, from per-call medians
// on MI355X over bf16 rows of 2048 to 8192 columns and 2048 to 32768 rows,
// every waves-per-row choice timed side by side:
// - fused Add+RMSNorm, at least 8 rows per CU: one vector a lane, in 16
//   waves for 601 to 1024 vectors a row (5120 to 8192 columns 0.3-1.9 %
//   faster than 8 waves of two, 4608 columns level; 512 rows 17 % slower),
//   in 8 waves for 257 to 448 from 16 rows per CU (2560 to 3584 columns
//   2.2-4.7 % faster than 4 waves of two; 2-3 % slower at 8 rows per CU),
//   and in 8 waves for 449 to 512 from 64 rows per CU (4096
//   columns: 1-2.5 % faster at 16384 and 32768 rows, level at 8192, 1.6 %
//   slower at 4096).  With one or two vectors a lane the row sums do not
//   depend on the launch shape, so the fused y stays the plain forward of
//   residual_out bit for bit; the plain RMSNorm keeps two vectors a lane
//   (one is 3-29 % slower there);
// - fused Add+LayerNorm: one vector a lane in 8 waves for 257 to 512 vectors
//   from 16 rows per CU (2.5-5.6 % faster than 4 waves of two), in 4 waves
//   for 193 to 256 from 32 rows per CU (3.0-4.1 %; 7-11 % slower at 4096
//   rows), 4 waves of up to 4 vectors for 769 to 960 from 16 rows per CU
//   (6656 to 7680 columns 0.8-2.4 % faster than 8 waves of two), and 16
//   waves of one for 961 to 1024 (bf16 8192 columns 1.8-2.7 %, level with 4
//   waves; float32 4096 columns 2.6-3.6 %, where 4 waves gain 0-1 %);
// - LayerNorm without the residual: each lane up to 4 vectors, in the fewest
//   waves that hold the row that way, and at least 2 waves for rows of more
//   than 128 vectors (at 2048 columns 2 waves of two match 1 of four at 16384
//   rows and beat it by 3 % at 4096): 2560 to 7168
//   columns 4-40 % faster than 8 waves of two or 4 of one (the statistics
//   take two exchanges per row, which more waves make dearer), 8192 columns
//   1-3 %.
// qm (a quantised mode, or kQNone) restricts the choice to built variants of
// that mode.  ADDRMS_FWD_WPR forces a WPR when it is built.
bool pick_fwd(int64_t M, int nvec, int cus, int norm, bool fused, int qm, int *wi_out,
              int *vi_out)
{
    const int forced = knob(ADDRMS_KNOB_FWD_WPR);
    const int env_vpl = knob(ADDRMS_KNOB_FWD_VPL);
    const bool plain_ln = norm == kLayer && !fused && qm == kQNone && env_vpl <= 0;
    const int target = env_vpl > 0 ? env_vpl : plain_ln ? 4 : 2;
    auto need_of = [&](int wi) { return (nvec + 64 * kWprList[wi] - 1) / (64 * kWprList[wi]); };
    auto ok = [&](int wi) {
        const int vi = vpl_index(need_of(wi));
        return vi >= 0 && (qm == kQNone ? fwd_built(kWprList[wi], kVplList[vi])
                                        : q_built(qm, kWprList[wi], kVplList[vi]));
    };
    auto take = [&](int wpr) {
        for (int wi = 0; wi < kNumWpr; ++wi)
            if (kWprList[wi] == wpr && ok(wi)) {
                *wi_out = wi;
                *vi_out = vpl_index(need_of(wi));
                return true;
            }
        return false;
    };
    if (forced > 0 && take(forced))
        return true;
    // Quantised outputs, 513 to 640 vectors a row (and for E4M3 with one scale
    // per group of columns up to 768): 4 waves of 3 vectors rather than 8 of
    // 2, which leave a third of the lanes idle (fused bf16, 4608 to 6144
    // columns, 4096 to 32768 rows: grouped E4M3 4-17 % faster, per-row E4M3
    // 2-8 %, MXFP4 1-4 %; level beyond 640 for the last two)
    if (qm != kQNone && env_vpl <= 0 && nvec > 512 && nvec <= (qm == kQGroup ? 768 : 640) &&
        M >= 8LL * cus && take(4))
        return true;
    if (qm == kQNone && env_vpl <= 0 && fused && M >= 8LL * cus) {
        const int64_t per_cu = M / cus;
        if (norm == kRms) {
            if (nvec > 600 && nvec <= 1024 && take(16))
                return true;
            if (nvec > 256 && ((nvec <= 448 && per_cu >= 16) || (nvec <= 512 && per_cu >= 64)) &&
                take(8))
                return true;
        } else {
            if (nvec > 256 && nvec <= 512 && per_cu >= 16 && take(8))
                return true;
            if (nvec > 192 && nvec <= 256 && per_cu >= 32 && take(4))
                return true;
            if (nvec > 960 && nvec <= 1024 && per_cu >= 16 && take(16))
                return true;
            if (nvec > 768 && nvec <= 960 && per_cu >= 16 && take(4))
                return true;
        }
    }
    int wi = plain_ln && nvec > 128 ? 1 : 0; // LayerNorm without the residual: 2 waves or more
    while (wi < kNumWpr - 1 &&
           need_of(wi) > (kWprList[wi] == 8 && env_vpl <= 0 ? 4 : target))
        ++wi;
    while (wi < kNumWpr - 1 && M * kWprList[wi] < 4LL * cus && need_of(wi) > 1)
        ++wi;
    while (wi < kNumWpr && !ok(wi)) // a built variant with at least as many waves
        ++wi;
    if (wi >= kNumWpr)
        return false;
    *wi_out = wi;
    *vi_out = vpl_index(need_of(wi));
    return true;
}

// Backward variant.  The fused and LayerNorm backwards of rows of 768 to 2048
// vectors take 8 waves per row (512-thread blocks, one row per step): they
// hold the most per lane (dres, or the db sums), and with 2 waves per row their
// 7 or 8 vectors per lane leave 1 or 2 waves per SIMD (measured on MI355X,
// bf16, 7168 and 8192 columns: fused 5.9-6.0 TB/s against 5.5-5.7, LayerNorm
// 5.1 against 3.8-3.9).  Otherwise WPR in {1, 2, 4}: first choice 2 waves per
// row with up to 8 vectors per lane, or 1 or 4 waves with up to 4 (2 waves per
// row streams best for the plain backward at 4096 to 8192 columns), except
// that the fused RMS backward also takes 1 wave per row with up to 8 (no
// barrier per row: 5.9 TB/s at 4096 columns against 5.56 with 2 waves), then
// up to 8, then up to 16 vectors per lane, among the instantiated variants;
// enough waves to fill the device; and a dw exchange that fits in 64 KiB of
// LDS.  ADDRMS_BWD_WPR forces a WPR.
bool pick_bwd(int norm, bool res, int64_t M, int N, int nvec, int cus, int *wi_out, int *vi_out)
{
    const int forced = knob(ADDRMS_KNOB_BWD_WPR);
    int best_wi = -1, best_vi = -1;
    // The fused RMS backward at 4 vectors a lane with 2 waves per row (385 to
    // 512 vectors) takes the next-row prefetch kernel rather than 1 wave per
    // row with 7 or 8 vectors: measured on MI355X, bf16, 24576 x 3584 120.8
    // against 127.9 us, 32768 x 4096 and 16384 x 4096 level or 0.8 % faster.
    if (forced == 0 && res && norm == kRms && (nvec + 127) / 128 == 4 && M * 2 >= 4LL * cus &&
        knob(ADDRMS_KNOB_BWD_PREFETCH) != 2 && bwd_built(norm, res, 2, 4)) {
        *wi_out = 1; // kWprList[1] == 2
        *vi_out = vpl_index(4);
        return true;
    }
    if (forced == 0 && (res || norm == kLayer) && nvec >= 768 && M * 8 >= 4LL * cus) {
        const int vi = vpl_index((nvec + 511) / 512);
        if (vi >= 0 && bwd_built(norm, res, 8, kVplList[vi])) {
            *wi_out = kBwdNumWpr - 1;
            *vi_out = vi;
            return true;
        }
    }
    for (int pass = 0; pass < 3 && best_wi < 0; ++pass) {
        for (int wi = 0; wi < kBwdNumWpr; ++wi) {
            const int wpr = kWprList[wi];
            const int max_vpl = pass == 0 ? ((wpr == 2 || (wpr == 1 && res && norm == kRms)) ? 8 : 4)
                                          : pass == 1 ? 8 : kMaxVpl;
            const int need = (nvec + 64 * wpr - 1) / (64 * wpr);
            const int vi = vpl_index(need);
            const int rpb = bwd_rpb(wpr);
            if (wpr == 8 && forced != 8) // 8 waves per row: only on request
                continue;
            if (vi < 0 || kVplList[vi] > max_vpl || !bwd_built(norm, res, wpr, kVplList[vi]))
                continue;
            if ((size_t)(rpb / 2) * (size_t)N * 4u > kMaxDynLds)
                continue;
            if (forced > 0 && wpr != forced)
                continue;
            if (forced > 0 || M * wpr >= 4LL * cus || wi == kBwdNumWpr - 2) {
                best_wi = wi;
                best_vi = vi;
                break;
            }
            if (best_wi < 0) { // remember the first fit in case none fills the device
                best_wi = wi;
                best_vi = vi;
            }
        }
    }
    if (best_wi < 0)
        return false;
    *wi_out = best_wi;
    *vi_out = best_vi;
    return true;
}

// Backward launch shapes measured over every choice (float32 rows: in the
// body), for 16-bit rows of 257 to 512 vectors (2056 to 4096 bf16 or float16
// columns), and for the plain
// RMS backward also 641 to 768 and 961 to 1024, with at least 32 rows per
// CU: per-call medians on MI355X of each forced shape (2, 4 or 8 waves per
// row, the next-row prefetch on or off, the wide block, 2 or 3 blocks per
// CU) at 2048 to 8192 columns and 4096 to 65536 rows, in alternating
// rounds, against the default of the rules below (2 waves with the
// prefetch at 4 vectors a lane, the wide block at 3):
//
//   vectors   RMS            fused RMS      LayerNorm      fused LayerNorm
//   257-384   2, no pf       2, pf          2, pf          2, pf
//   385-448   8              2, no pf       8              8
//   449-512   8              8              8              8
//   641-768   4              (rules)        (rules)        (rules)
//   961-1024  8              (rules)        (rules)        (rules)
//
// all on 2 blocks per CU (waves per row, prefetch).  Gains, rerun with the
// table in place against the former default: 2560 and 3072 columns 3-13 %;
// 3584 columns 3-10 %; 4096 columns 2-11 % (the RMS backward at 32768 x
// 4096: 135.4 against 139.3 us per call); 6144 columns, RMS 3-6 %; 8192
// columns, RMS 2-4 %.  Every table entry is within 0.8 % of the fastest
// forced shape at every measured size.  At 8 waves a row takes one vector
// a lane, and 2 blocks per CU (16 waves) beat the 3 or 4 that fit by 6-11 %
// for LayerNorm (fewer dw partial rows, whole row steps).  Returns false
// (the rules below decide) for other shapes or when a tuning knob is set.
bool bwd_measured_choice(int norm, bool res, bool half, int64_t M, int nvec, int cus, int *wpr,
                         int *pf)
{
    if (M < 32LL * cus || knob(ADDRMS_KNOB_BWD_WPR) != 0 || knob(ADDRMS_KNOB_BWD_PREFETCH) != 0 ||
        knob(ADDRMS_KNOB_BWD_WIDE) != 0 || knob(ADDRMS_KNOB_BLOCKS_PER_CU) != 0)
        return false;
    const bool ln = norm == kLayer;
    if (!half) {
        // float32 rows (binary64 row arithmetic), swept the same way at 1024
        // to 4096 columns: 2 waves with the prefetch at 257 to 384 vectors
        // (1536 columns: 4-8 % faster) and for the fused forms at 193 to 256
        // (1024 columns: 4-7 %; the plain forms stay on the grid that fits,
        // 2 blocks per CU being 5-8 % slower there), 8 waves at 449 to 512
        // (2048 columns: 3-11 %), and for the RMS backwards 8 waves at 961
        // to 1024 (4096 columns: 1-6 %); level elsewhere
        if ((nvec > 256 && nvec <= 384) || (nvec > 192 && nvec <= 256 && res)) {
            *wpr = 2;
            *pf = 1;
            return true;
        }
        if ((nvec > 448 && nvec <= 512) || (nvec > 960 && nvec <= 1024 && !ln)) {
            *wpr = 8;
            *pf = 0;
            return true;
        }
        return false;
    }
    if (nvec > 256 && nvec <= 384) {
        *wpr = 2;
        *pf = (ln || res) ? 1 : 0;
        return true;
    }
    if (nvec > 384 && nvec <= 448) {
        *wpr = (res && !ln) ? 2 : 8;
        *pf = 0;
        return true;
    }
    if (nvec > 448 && nvec <= 512) {
        *wpr = 8;
        *pf = 0;
        return true;
    }
    if (nvec > 640 && nvec <= 768 && !ln && !res) {
        *wpr = 4;
        *pf = 0;
        return true;
    }
    if (nvec > 960 && nvec <= 1024 && !ln && !res) {
        *wpr = 8;
        *pf = 0;
        return true;
    }
    return false;
}

// The wide backward (one 1024-thread block per CU, 8 rows of 2 waves per
// step) instead of four 256-thread blocks of 2 rows: the same waves per CU
// and the same per-row work, with a quarter of the dw partial rows for the
// column reduce to read, but a barrier per row step that spans 16 waves.
// Measured on MI355X, bf16, wide / 256-thread time: 3 vectors a lane (3072
// columns) 0.69-0.98 at 2048 to 32768 rows; 4 vectors a lane (4096
// columns) 0.67 / 0.81 / 0.95 at 2048 / 4096 / 8192 rows, 1.01-1.03 at
// 12288 rows and more.  So it is taken when the picker chose 2 waves per row,
// the variant is built, its LDS tree fits, every CU gets a block, and the row
// has at most 3 vectors a lane or the batch has at most 32 rows per CU.
// ADDRMS_BWD_WIDE=1 forces it where built, ADDRMS_BWD_WIDE=2 turns it off.
bool use_wide_bwd(const BwdTable &tab, int norm, bool res, int64_t M, int64_t N, int wi, int vi,
                  int cus)
{
    const int mode = knob(ADDRMS_KNOB_BWD_WIDE);
    if (mode == 2 || kWprList[wi] != kBwdWideWpr || tab.wide[norm][res ? 1 : 0][vi].fn == nullptr)
        return false;
    const int rpb = bwd_rpb(kBwdWideWpr, true);
    if ((size_t)(rpb / 2) * (size_t)N * 4u > kMaxDynLds)
        return false;
    if (mode == 1)
        return true;
    return M >= (int64_t)rpb * cus && (kVplList[vi] <= 3 || M <= 32LL * cus);
}

// The backwards with the next row's loads in flight across the current row's
// exchange and output pass (the PF kernels), measured on MI355X at 4 vectors
// a lane and 2 waves per row: RMS 1.5-3.6 % faster (3584 to 4096 bf16 or
// 1792 to 2048 float32 columns, 12288 to 65536 rows), LayerNorm 3.5-5.8 %
// (3584 to 4096 bf16 columns, 8192 to 32768 rows), fused LayerNorm 2-5 %
// (bf16, 3584 and 4096 columns); so it is the default there.  The fused RMS
// backward takes it too (see pick_bwd).  ADDRMS_BWD_PREFETCH=1 takes it
// wherever it is built (2 waves per row, up to 4 vectors a lane),
// ADDRMS_BWD_PREFETCH=2 never.
bool use_prefetch_bwd(const BwdTable &tab, int norm, bool res, int wi, int vi)
{
    const int mode = knob(ADDRMS_KNOB_BWD_PREFETCH);
    if (mode == 2 || tab.pf[norm][res ? 1 : 0][wi][vi].fn == nullptr)
        return false;
    return mode == 1 || kVplList[vi] == 4;
}

// dw[c] = sum over P partial rows of ws[:, c], and, when db is given,
// db[c] = sum of ws2[:, c], in one launch (P = 0 writes zeros; nothing read).
int colreduce(const void *workspace, const void *workspace2, int P, int N, float *dw, float *db,
              hipStream_t s)
{
    const float *ws = static_cast<const float *>(workspace);
    const float *ws2 = static_cast<const float *>(workspace2);
    const bool vec = (N % 4) == 0 && aligned16(dw) && (!db || aligned16(db)) &&
                     (P == 0 || (aligned16(ws) && (!db || aligned16(ws2))));
    const KernelRef k = colreduce_kernel(vec);
    const int cols = vec ? kColReduceVecCols : kColReduceCols;
    void *argv[] = {(void *)&ws, (void *)&ws2, (void *)&P, (void *)&N, (void *)&dw, (void *)&db};
    hipError_t e = hipLaunchKernel(k.fn, dim3((unsigned)((N + cols - 1) / cols), db ? 2u : 1u),
                                   dim3(k.block), argv, 0, s);
    return e == hipSuccess ? ADDRMS_OK : fail_hip(e);
}

int fwd_common(int norm, const void *x, const void *r, const void *w, const void *b, void *y,
               void *res, float *mean, float *rstd, int64_t M, int64_t N, float eps, int dtype,
               int w_dtype, void *stream, bool fused, uint8_t *q = nullptr, void *qscale = nullptr,
               int64_t qgroup = 0, int qfmt = 0)
{
    // ---- validation (no HIP call) ----
    // With M == 0 the matrices are empty and may be NULL.  The FP8 variant
    // writes q and qscale in place of y.
    const bool q8 = q != nullptr || qscale != nullptr;
    if (q8)
        y = q; // the output matrix, for the checks below (1 byte per element; MXFP4: half)
    if (!w || (M != 0 && (!x || !y || (fused && (!r || !res)) || (q8 && (!q || !qscale)))))
        return ADDRMS_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(w_dtype))
        return ADDRMS_ERR_DTYPE;
    int rc = check_shape(M, N, dtype);
    if (rc != ADDRMS_OK)
        return rc;
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return ADDRMS_ERR_EPS;
    const size_t mat = (size_t)M * (size_t)N * esize(dtype);
    const Span sx = span(x, mat), sw = span(w, (size_t)N * esize(w_dtype));
    const Span sy = span(y, q8 ? (size_t)M * (size_t)N / (qfmt == 1 ? 2 : 1) : mat);
    // FP8 scales: one per row (qgroup == 0, or a group spanning the row), else
    // one per group of qgroup columns
    // MXFP4 (qfmt 1): E2M1 codes two per byte, one E8M0 byte per 32 columns
    const bool mx = qfmt == 1;
    if (qgroup < 0 || (mx && N % 2 != 0))
        return ADDRMS_ERR_SHAPE;
    if (mx)
        qgroup = 32;
    else if (qgroup >= N)
        qgroup = 0;
    const int64_t ngroups = qgroup > 0 ? (N + qgroup - 1) / qgroup : 1;
    const Span sqs = q8 ? span(qscale, (size_t)M * (size_t)ngroups * (mx ? 1u : 4u)) : Span{};
    const Span sr = fused ? span(r, mat) : Span{}, sres = fused ? span(res, mat) : Span{};
    const Span srs = rstd ? span(rstd, (size_t)M * 4u) : Span{};
    const Span sb = b ? span(b, (size_t)N * esize(w_dtype)) : Span{};
    const Span smu = mean ? span(mean, (size_t)M * 4u) : Span{};
    if (bad_alias(sy, sx, true) || bad_alias(sy, sw, false) || bad_alias(sy, srs, false) ||
        bad_alias(sy, sb, false) || bad_alias(sy, smu, false))
        return ADDRMS_ERR_ALIAS;
    if (fused && (bad_alias(sres, sb, false) || bad_alias(sres, smu, false)))
        return ADDRMS_ERR_ALIAS;
    if (mean && (bad_alias(smu, sx, false) || bad_alias(smu, sw, false) ||
                 bad_alias(smu, sb, false) || bad_alias(smu, srs, false) ||
                 (fused && bad_alias(smu, sr, false))))
        return ADDRMS_ERR_ALIAS;
    if (rstd && bad_alias(srs, sb, false))
        return ADDRMS_ERR_ALIAS;
    if (q8 && (bad_alias(sy, sx, false) || (fused && bad_alias(sy, sr, false)) ||
               bad_alias(sqs, sx, false) || bad_alias(sqs, sw, false) || bad_alias(sqs, sy, false) ||
               bad_alias(sqs, srs, false) || (fused && (bad_alias(sqs, sr, false) ||
                                                        bad_alias(sqs, sres, false)))))
        return ADDRMS_ERR_ALIAS;
    if (fused && (bad_alias(sy, sr, true) || bad_alias(sres, sx, true) ||
                  bad_alias(sres, sr, true) || bad_alias(sres, sw, false) ||
                  bad_alias(sres, srs, false) || bad_alias(sres, sy, false)))
        return ADDRMS_ERR_ALIAS;
    if (rstd && (bad_alias(srs, sx, false) || bad_alias(srs, sw, false) ||
                 (fused && bad_alias(srs, sr, false))))
        return ADDRMS_ERR_ALIAS;
    if (M == 0)
        return ADDRMS_OK;

    // ---- variant and launch ----
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int c = combo(dtype, w_dtype);
    const FwdTable &tab = fwd_table(c);
    FwdArgs a{x, fused ? r : x, w, b, y, fused ? res : y, mean, rstd, q, qscale, M, (int)N, 0, eps};
    a.qgroup = (int)qgroup;
    a.qgroups = (int)ngroups;
    // quantised mode, as an index of the tables (mode - 1)
    const int qm = mx ? kQMx - 1 : qgroup > 0 ? kQGroup - 1 : kQRow - 1;

    const int nv = vec_elems(dtype);
    // grouped scales on the vector path: a group is a power of two of whole
    // vectors, at most one wave wide
    int qlanes = 0;
    if (qgroup > 0 && qgroup % nv == 0) {
        const int64_t L = qgroup / nv;
        if (L <= 64 && (L & (L - 1)) == 0)
            qlanes = (int)L;
    }
    a.qlanes = qlanes;
    // codes per 16-byte vector: nv bytes (E4M3) or nv / 2 (MXFP4), stored as one word
    const bool y_ok = q8 ? (reinterpret_cast<uintptr_t>(q) % (uintptr_t)(mx ? nv / 2 : nv)) == 0
                         : aligned16(y);
    const bool vec_ok = knob(ADDRMS_KNOB_FORCE_ELEM) == 0 && (N % nv) == 0 && aligned16(x) &&
                        aligned16(w) && y_ok && (!b || aligned16(b)) &&
                        (!fused || (aligned16(r) && aligned16(res))) &&
                        (qgroup == 0 || qlanes > 0);
    int cus = 0;
    if ((rc = device_cus_current(&cus)) != ADDRMS_OK)
        return rc;
    int wi = 0, vi = 0;
    if (vec_ok &&
        pick_fwd(M, (int)(N / nv), cus, norm, fused, q8 ? qm + 1 : (int)kQNone, &wi, &vi) &&
        (!q8 || tab.vec_q8[fused ? 1 : 0][qm][wi][vi].fn != nullptr)) {
        a.nvec = (int)(N / nv);
        const KernelRef &k =
            q8 ? tab.vec_q8[fused ? 1 : 0][qm][wi][vi] : tab.vec[norm][fused ? 1 : 0][wi][vi];
        const int rpb = kWprList[wi] == 1 ? 4 : 1;
        const int64_t blocks = (M + rpb - 1) / rpb;
        // One block per row group (the hardware dispatcher balances the
        // tail); ADDRMS_BLOCKS_PER_CU > 0 selects a persistent grid instead.
        int grid = (int)(blocks < INT_MAX ? blocks : INT_MAX);
        if (knob(ADDRMS_KNOB_BLOCKS_PER_CU) > 0 &&
            (rc = persistent_grid(k, 0, blocks, INT_MAX, &grid)) != ADDRMS_OK)
            return rc;
        return launch(k, dim3(grid), 0, &a, s);
    }
    const KernelRef &k = q8 ? tab.elem_q8[fused ? 1 : 0][qm] : tab.elem[norm][fused ? 1 : 0];
    int grid = 0;
    if ((rc = persistent_grid(k, 0, M, INT_MAX, &grid)) != ADDRMS_OK)
        return rc;
    return launch(k, dim3(grid), 0, &a, s);
}

// fit_ws: the workspace has a fixed capacity (the no-allocation entry point's
// scratch): the call uses as many dw partial rows as fit in it, at least one,
// instead of requiring the size rmsnorm_bwd_workspace_bytes gives.
int bwd_common(int norm, const void *dy, const void *dres, const void *x, const void *w,
               const float *mean, const float *rstd, void *dx, float *dw, float *db,
               void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype,
               int w_dtype, void *stream, bool fit_ws = false)
{
    const bool res = dres != nullptr;
    const bool ln = norm == kLayer;
    // ---- validation (no HIP call) ----
    // With M == 0 the row data is empty and may be NULL; dw is still written.
    if (!w || !dw || (M != 0 && (!dy || !x || !rstd || !dx || (ln && !mean))))
        return ADDRMS_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(w_dtype))
        return ADDRMS_ERR_DTYPE;
    int rc = check_shape(M, N, dtype);
    if (rc != ADDRMS_OK)
        return rc;
    size_t need = ln ? layernorm_bwd_workspace_bytes(M, N) : rmsnorm_bwd_workspace_bytes(M, N);
    if (fit_ws && M > 0 && need > workspace_bytes) {
        // one partial row (two for LayerNorm) is the least a call can use
        if ((uint64_t)N > (uint64_t)workspace_bytes / 4u / (ln ? 2u : 1u))
            return ADDRMS_ERR_SCRATCH;
        need = workspace_bytes;
    }
    if (M > 0 && (!workspace || workspace_bytes < need || need == 0))
        return ADDRMS_ERR_WORKSPACE;
    const size_t mat = (size_t)M * (size_t)N * esize(dtype);
    const Span sdy = span(dy, mat), sx = span(x, mat), sw = span(w, (size_t)N * esize(w_dtype));
    const Span srs = span(rstd, (size_t)M * 4u), sdx = span(dx, mat), sdw = span(dw, (size_t)N * 4u);
    const Span sws = workspace ? span(workspace, need) : Span{};
    const Span sdr = res ? span(dres, mat) : Span{};
    const Span smu = (ln && mean) ? span(mean, (size_t)M * 4u) : Span{};
    const Span sdb = db ? span(db, (size_t)N * 4u) : Span{};
    if (res && (bad_alias(sdx, sdr, true) || bad_alias(sdw, sdr, false) || bad_alias(sws, sdr, false)))
        return ADDRMS_ERR_ALIAS;
    if (bad_alias(sdx, smu, false) || bad_alias(sdw, smu, false) || bad_alias(sws, smu, false) ||
        bad_alias(sdw, sdb, false))
        return ADDRMS_ERR_ALIAS;
    if (db && (bad_alias(sdb, sdy, false) || bad_alias(sdb, sx, false) || bad_alias(sdb, sw, false) ||
               bad_alias(sdb, srs, false) || bad_alias(sdb, smu, false) ||
               bad_alias(sdb, sws, false) || bad_alias(sdb, sdx, false) ||
               (res && bad_alias(sdb, sdr, false))))
        return ADDRMS_ERR_ALIAS;
    if (bad_alias(sdx, sdy, true) || bad_alias(sdx, sx, true) || bad_alias(sdx, sw, false) ||
        bad_alias(sdx, srs, false) || bad_alias(sdx, sdw, false) || bad_alias(sdx, sws, false))
        return ADDRMS_ERR_ALIAS;
    if (bad_alias(sdw, sdy, false) || bad_alias(sdw, sx, false) || bad_alias(sdw, sw, false) ||
        bad_alias(sdw, srs, false) || bad_alias(sdw, sws, false))
        return ADDRMS_ERR_ALIAS;
    if (bad_alias(sws, sdy, false) || bad_alias(sws, sx, false) || bad_alias(sws, sw, false) ||
        bad_alias(sws, srs, false))
        return ADDRMS_ERR_ALIAS;

    // ---- variant and launch ----
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (M == 0) // dw (db) of an empty batch is zero: the column reduce over P = 0 rows writes it
        return colreduce(workspace, workspace, 0, (int)N, dw, db, s);
    const BwdTable &tab = bwd_table(combo(dtype, w_dtype));
    // LayerNorm: the workspace holds dw partials then db partials, pmax rows each
    const int64_t ws_rows = (int64_t)(workspace_bytes / ((size_t)N * 4u)) / (ln ? 2 : 1);
    // ADDRMS_MAX_PARTIALS raises the partial-row cap when the caller passes a
    // larger workspace (tuning); the size function assumes the default cap.
    const int64_t cap = knob(ADDRMS_KNOB_MAX_PARTIALS) > 0 ? knob(ADDRMS_KNOB_MAX_PARTIALS) : kMaxPartials;
    const int64_t pmax = ws_rows < cap ? ws_rows : cap;
    float *ws = static_cast<float *>(workspace);
    BwdArgs a{dy, res ? dres : dy, x, w, mean, rstd, dx, ws, ln ? ws + (size_t)pmax * N : ws,
              M, (int)N, 0, 0, 0};

    const int nv = vec_elems(dtype);
    const bool vec_ok = knob(ADDRMS_KNOB_FORCE_ELEM) == 0 && (N % nv) == 0 && aligned16(dy) &&
                        aligned16(x) && aligned16(w) && aligned16(dx) && aligned16(workspace) &&
                        (!res || aligned16(dres)) && (!ln || (pmax * N) % 4 == 0);
    int cus = 0;
    if ((rc = device_cus_current(&cus)) != ADDRMS_OK)
        return rc;
    int wi = 0, vi = 0, m_wpr = 0, m_pf = 0;
    const int nvec = (int)(N / nv);
    // the measured table first, where it covers the shape and its variant is built
    bool measured = vec_ok && bwd_measured_choice(norm, res, dtype != ADDRMS_F32, M, nvec, cus,
                                                  &m_wpr, &m_pf);
    if (measured) {
        const int need = (nvec + 64 * m_wpr - 1) / (64 * m_wpr);
        vi = vpl_index(need);
        wi = m_wpr == 2 ? 1 : m_wpr == 4 ? 2 : m_wpr == 8 ? 3 : -1; // kWprList: 1, 2, 4, 8
        measured = vi >= 0 && wi >= 0 && kWprList[wi] == m_wpr &&
                   bwd_built(norm, res, m_wpr, kVplList[vi]) &&
                   (size_t)(bwd_rpb(m_wpr) / 2) * (size_t)N * 4u <= kMaxDynLds &&
                   (m_pf == 1 ? tab.pf[norm][res ? 1 : 0][wi][vi].fn
                              : tab.vec[norm][res ? 1 : 0][wi][vi].fn) != nullptr;
    }
    if (measured || (vec_ok && pick_bwd(norm, res, M, (int)N, nvec, cus, &wi, &vi))) {
        a.nvec = nvec;
        const bool wide = !measured && use_wide_bwd(tab, norm, res, M, N, wi, vi, cus);
        const bool pf = measured ? m_pf == 1 : !wide && use_prefetch_bwd(tab, norm, res, wi, vi);
        const KernelRef &k = wide ? tab.wide[norm][res ? 1 : 0][vi]
                             : pf ? tab.pf[norm][res ? 1 : 0][wi][vi]
                                  : tab.vec[norm][res ? 1 : 0][wi][vi];
        const int rpb = bwd_rpb(kWprList[wi], wide);
        const size_t smem = (size_t)(rpb / 2) * (size_t)N * 4u;
        int grid = 0;
        if ((rc = persistent_grid(k, smem, (M + rpb - 1) / rpb, pmax, &grid)) != ADDRMS_OK)
            return rc;
        // The RMS backwards (plain and fused) over many rows: 2 blocks per CU
        // rather than the 3 or 4 that fit.  Fewer blocks write fewer dw partial
        // rows (2 P N floats of extra traffic, and the column reduce reads
        // them), and the rows divide into whole steps more often.  Measured on
        // MI355X, per-call medians against the grid that fits: bf16, 4096
        // columns 2.1-2.8 % faster at 16384 to 65536 rows, 2048 columns
        // 3.4-6.7 %, the fused form 9 % at 16384 x 2048; float32, 2048
        // columns 1-3 %, fused 2 %.  Slower, so keeping the grid that fits:
        // 1024 bf16 or float32 columns (1-2 %), fewer than 12288 rows of 4096
        // bf16 columns (6-14 %), and LayerNorm (9 % at 32768 x 2048).
        if (norm == kRms && !wide && knob(ADDRMS_KNOB_BLOCKS_PER_CU) == 0 &&
            a.nvec >= (dtype == ADDRMS_F32 ? 512 : 256) && M >= 48LL * cus && grid > 2 * cus)
            grid = 2 * cus;
        if (measured && grid > 2 * cus) // the measured table's shapes: 2 blocks per CU
            grid = 2 * cus;
        a.P = grid;
        if ((rc = launch(k, dim3(grid), smem, &a, s)) != ADDRMS_OK)
            return rc;
    } else {
        // element-wise: dw partials over row chunks first (reads dy, x intact),
        // then dx (which may overwrite dy or x)
        int64_t chunk = (M + pmax - 1) / pmax;
        const int64_t P = (M + chunk - 1) / chunk;
        a.P = (int)P;
        a.chunk = chunk;
        if ((rc = launch(tab.elem_dw[norm], dim3((unsigned)((N + 63) / 64), (unsigned)P), 0, &a, s)) !=
            ADDRMS_OK)
            return rc;
        int grid = 0;
        const KernelRef &kdx = tab.elem_dx[norm][res ? 1 : 0];
        if ((rc = persistent_grid(kdx, 0, M, INT_MAX, &grid)) != ADDRMS_OK)
            return rc;
        if ((rc = launch(kdx, dim3(grid), 0, &a, s)) != ADDRMS_OK)
            return rc;
    }
    // dw (db) = column sums of the partials, same stream (ordered after stage 1)
    return colreduce(a.ws, a.ws2, a.P, (int)N, dw, (ln && db) ? db : nullptr, s);
}

// Do two strided sets of byte ranges, {a + i*sa + [0, la)} for i < na and
// {b + j*sb + [0, lb)} for j < nb, share a byte?  Exact when the whole spans
// are disjoint, and for equal strides with la, lb <= stride: the heads of one
// packed projection buffer (query and key parts of every token) interleave
// without touching.  Otherwise the answer is yes (conservative).
bool strided_overlap(const void *pa, int64_t sa, int64_t la, int64_t na, const void *pb,
                     int64_t sb, int64_t lb, int64_t nb)
{
    if (na <= 0 || nb <= 0 || la <= 0 || lb <= 0)
        return false;
    const Span A = span(pa, (size_t)((na - 1) * sa + la));
    const Span B = span(pb, (size_t)((nb - 1) * sb + lb));
    if (!overlaps(A, B))
        return false;
    if (sa == sb && la <= sa && lb <= sb) {
        const int64_t d = (int64_t)(B.lo - A.lo);
        int64_t r = d % sa;
        if (r < 0)
            r += sa;
        return !(r >= la && r + lb <= sa);
    }
    return true;
}

// Per-head RMSNorm + RoPE (see rmsnorm_rope_qk in addrms.h).
int rope_common(const void *q, const void *k, const void *wq, const void *wk, const float *cos,
                const float *sin, const int64_t *pos, int64_t P, void *qo, void *ko, int64_t T,
                int64_t Hq, int64_t Hk, int64_t D, int64_t q_stride, int64_t k_stride,
                int64_t qo_stride, int64_t ko_stride, float eps, int interleaved, int dtype,
                int w_dtype, hipStream_t s)
{
    if (!dtype_ok(dtype) || !dtype_ok(w_dtype))
        return ADDRMS_ERR_DTYPE;
    if (T < 0 || Hq < 0 || Hk < 0 || P < 0 || D < 2 || D % 2 != 0 || D > INT_MAX ||
        Hq > INT_MAX || Hk > INT_MAX || Hq + Hk > INT_MAX / D)
        return ADDRMS_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return ADDRMS_ERR_EPS;
    if (T == 0 || Hq + Hk == 0)
        return ADDRMS_OK; // nothing to do; the pointers may be NULL
    if (!cos || !sin || !pos || (Hq > 0 && (!q || !qo || !wq)) || (Hk > 0 && (!k || !ko || !wk)))
        return ADDRMS_ERR_NULL;
    const int64_t es = (int64_t)esize(dtype);
    const int64_t lim = ((int64_t)1 << 62) / es;
    // each token's heads fit inside its stride, and the last element is addressable
    auto bad_stride = [&](int64_t H, int64_t st) {
        return H > 0 && (st < H * D || st > lim / (T > 1 ? T : 1));
    };
    if (bad_stride(Hq, q_stride) || bad_stride(Hq, qo_stride) || bad_stride(Hk, k_stride) ||
        bad_stride(Hk, ko_stride) || (int64_t)(P > 0 ? P : 1) > lim / D)
        return ADDRMS_ERR_SHAPE;

    // outputs: each may be its own input (same address and stride); nothing
    // else overlaps an output
    const Span sc = span(cos, (size_t)(P * (D / 2) * 4)), ssn = span(sin, (size_t)(P * (D / 2) * 4));
    const Span sp = span(pos, (size_t)T * 8u);
    const Span swq = Hq > 0 ? span(wq, (size_t)(D * (int64_t)esize(w_dtype))) : Span{};
    const Span swk = Hk > 0 ? span(wk, (size_t)(D * (int64_t)esize(w_dtype))) : Span{};
    struct Set {
        const void *p;
        int64_t stride, len;
    };
    const Set sq{q, q_stride * es, Hq * D * es}, sk{k, k_stride * es, Hk * D * es};
    const Set sqo{qo, qo_stride * es, Hq * D * es}, sko{ko, ko_stride * es, Hk * D * es};
    auto hit = [&](const Set &a, const Set &b) {
        return strided_overlap(a.p, a.stride, a.len, T, b.p, b.stride, b.len, T);
    };
    auto whole = [&](const Set &a) {
        return a.len > 0 ? span(a.p, (size_t)((T - 1) * a.stride + a.len)) : Span{};
    };
    const bool q_inplace = qo == q && qo_stride == q_stride;
    const bool k_inplace = ko == k && ko_stride == k_stride;
    if ((!q_inplace && hit(sqo, sq)) || (!k_inplace && hit(sko, sk)) || hit(sqo, sk) ||
        hit(sko, sq) || hit(sqo, sko))
        return ADDRMS_ERR_ALIAS;
    for (const Set *o : {&sqo, &sko}) {
        const Span so = whole(*o);
        if (overlaps(so, sc) || overlaps(so, ssn) || overlaps(so, sp) || overlaps(so, swq) ||
            overlaps(so, swk))
            return ADDRMS_ERR_ALIAS;
    }

    RopeArgs a{};
    a.q = q;
    a.k = k;
    a.wq = wq;
    a.wk = wk;
    a.cos = cos;
    a.sin = sin;
    a.pos = pos;
    a.qo = qo;
    a.ko = ko;
    a.q_stride = q_stride;
    a.k_stride = k_stride;
    a.qo_stride = qo_stride;
    a.ko_stride = ko_stride;
    a.T = T;
    a.P = P;
    a.Hq = (int)Hq;
    a.Hk = (int)Hk;
    a.D = (int)D;
    a.eps = eps;

    const RopeTable &tab = rope_table(combo(dtype, w_dtype));
    const int il = interleaved ? 1 : 0;
    const int64_t total = T * (Hq + Hk);
    // vector path: D = 2 * E * G with G = 1, 2, 4, ..., 64 lanes per head,
    // every pointer 16-byte aligned, every token stride a multiple of 16 bytes
    const int E = vec_elems(dtype);
    const int64_t G = D / (2 * E);
    int lg = -1;
    if (D % (2 * E) == 0)
        for (int i = 0; i < kRopeNumGroups; ++i)
            if (G == ((int64_t)1 << i))
                lg = i;
    auto al = [&](const void *p, int64_t H, int64_t st) {
        return H == 0 || (aligned16(p) && (st * es) % 16 == 0);
    };
    const bool vec = knob(ADDRMS_KNOB_FORCE_ELEM) == 0 && lg >= 0 && al(q, Hq, q_stride) &&
                     al(qo, Hq, qo_stride) && al(k, Hk, k_stride) && al(ko, Hk, ko_stride) &&
                     (Hq == 0 || aligned16(wq)) && (Hk == 0 || aligned16(wk)) && aligned16(cos) &&
                     aligned16(sin);
    if (vec) {
        // heads per lane group and loop step: ADDRMS_ROPE_HPL = 1, 2 or 4
        // forces it; otherwise kRopeHpl
        const int forced = knob(ADDRMS_KNOB_ROPE_HPL);
        int hpl = forced == 1 || forced == 2 || forced == 4 ? forced : kRopeHpl;
        if (!rope_built((int)G, hpl))
            hpl = 2;
        const int lh = hpl == 1 ? 0 : hpl == 2 ? 1 : 2;
        const int64_t step = (kRopeBlock / G) * hpl;
        int64_t blocks = (total + step - 1) / step;
        // ADDRMS_ROPE_BLOCKS_PER_CU caps the grid at that many blocks per CU
        // (each block then loops over several steps)
        const int bpc = knob(ADDRMS_KNOB_ROPE_BLOCKS_PER_CU);
        if (bpc > 0) {
            int cus = 0, rc;
            if ((rc = device_cus_current(&cus)) != ADDRMS_OK)
                return rc;
            if (blocks > (int64_t)cus * bpc)
                blocks = (int64_t)cus * bpc;
        }
        return launch(tab.vec[il][lg][lh],
                      dim3((unsigned)(blocks < (1 << 30) ? blocks : (1 << 30))), 0, &a, s);
    }
    return launch(tab.elem[il], dim3((unsigned)(total < (1 << 24) ? total : (1 << 24))), 0, &a, s);
}

} // namespace
} // namespace addrms

using namespace addrms;

// Scratch of the no-allocation backward: the dw partial rows live in this
// file-scope device array instead of a caller's workspace.  Each device that
// loads the library holds its own copy until the process ends.  In host code
// `scratch` only names a host-side stand-in: its device address on the
// current device comes from hipGetSymbolAddress, taken once per device and
// kept in g_scratch; only that address is ever passed to a kernel.
static __device__ __align__(256) float scratch[ADDRMS_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
std::mutex g_scratch_mu;
std::map<int, void *> g_scratch;

int scratch_ptr(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail_hip(e);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return fail_hip(e);
        if (p == nullptr)
            return fail_hip(hipErrorInvalidSymbol);
        it = g_scratch.emplace(dev, p).first;
    }
    *out = it->second;
    return ADDRMS_OK;
}
} // namespace

extern "C" {

int rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd, int64_t M, int64_t N,
                float eps, int dtype, int w_dtype, void *stream)
{
    return fwd_common(kRms, x, nullptr, w, nullptr, y, nullptr, nullptr, rstd, M, N, eps, dtype,
                      w_dtype, stream, false);
}

int add_rmsnorm_fwd(const void *x, const void *r, const void *w, void *y, void *residual_out,
                    float *rstd, int64_t M, int64_t N, float eps, int dtype, int w_dtype,
                    void *stream)
{
    return fwd_common(kRms, x, r, w, nullptr, y, residual_out, nullptr, rstd, M, N, eps, dtype,
                      w_dtype, stream, true);
}

int rmsnorm_fwd_fp8(const void *x, const void *w, void *y_fp8, float *y_scale, float *rstd,
                    int64_t M, int64_t N, float eps, int dtype, int w_dtype, void *stream)
{
    if (M != 0 && (!y_fp8 || !y_scale))
        return ADDRMS_ERR_NULL;
    return fwd_common(kRms, x, nullptr, w, nullptr, nullptr, nullptr, nullptr, rstd, M, N, eps,
                      dtype, w_dtype, stream, false, static_cast<uint8_t *>(y_fp8), y_scale);
}

int add_rmsnorm_fwd_fp8(const void *x, const void *r, const void *w, void *y_fp8, float *y_scale,
                        void *residual_out, float *rstd, int64_t M, int64_t N, float eps,
                        int dtype, int w_dtype, void *stream)
{
    if (M != 0 && (!y_fp8 || !y_scale))
        return ADDRMS_ERR_NULL;
    return fwd_common(kRms, x, r, w, nullptr, nullptr, residual_out, nullptr, rstd, M, N, eps,
                      dtype, w_dtype, stream, true, static_cast<uint8_t *>(y_fp8), y_scale);
}

int rmsnorm_fwd_fp8_grouped(const void *x, const void *w, void *y_fp8, float *y_scale,
                            int64_t group, float *rstd, int64_t M, int64_t N, float eps, int dtype,
                            int w_dtype, void *stream)
{
    if (M != 0 && (!y_fp8 || !y_scale))
        return ADDRMS_ERR_NULL;
    if (group < 1)
        return ADDRMS_ERR_SHAPE;
    return fwd_common(kRms, x, nullptr, w, nullptr, nullptr, nullptr, nullptr, rstd, M, N, eps,
                      dtype, w_dtype, stream, false, static_cast<uint8_t *>(y_fp8), y_scale, group);
}

int add_rmsnorm_fwd_fp8_grouped(const void *x, const void *r, const void *w, void *y_fp8,
                                float *y_scale, int64_t group, void *residual_out, float *rstd,
                                int64_t M, int64_t N, float eps, int dtype, int w_dtype,
                                void *stream)
{
    if (M != 0 && (!y_fp8 || !y_scale))
        return ADDRMS_ERR_NULL;
    if (group < 1)
        return ADDRMS_ERR_SHAPE;
    return fwd_common(kRms, x, r, w, nullptr, nullptr, residual_out, nullptr, rstd, M, N, eps,
                      dtype, w_dtype, stream, true, static_cast<uint8_t *>(y_fp8), y_scale, group);
}

int rmsnorm_fwd_mxfp4(const void *x, const void *w, void *y_fp4, void *y_scale, float *rstd,
                      int64_t M, int64_t N, float eps, int dtype, int w_dtype, void *stream)
{
    if (M != 0 && (!y_fp4 || !y_scale))
        return ADDRMS_ERR_NULL;
    return fwd_common(kRms, x, nullptr, w, nullptr, nullptr, nullptr, nullptr, rstd, M, N, eps,
                      dtype, w_dtype, stream, false, static_cast<uint8_t *>(y_fp4), y_scale, 32, 1);
}

int add_rmsnorm_fwd_mxfp4(const void *x, const void *r, const void *w, void *y_fp4,
                          void *y_scale, void *residual_out, float *rstd, int64_t M, int64_t N,
                          float eps, int dtype, int w_dtype, void *stream)
{
    if (M != 0 && (!y_fp4 || !y_scale))
        return ADDRMS_ERR_NULL;
    return fwd_common(kRms, x, r, w, nullptr, nullptr, residual_out, nullptr, rstd, M, N, eps,
                      dtype, w_dtype, stream, true, static_cast<uint8_t *>(y_fp4), y_scale, 32, 1);
}

int layernorm_fwd(const void *x, const void *w, const void *b, void *y, float *mean, float *rstd,
                  int64_t M, int64_t N, float eps, int dtype, int w_dtype, void *stream)
{
    return fwd_common(kLayer, x, nullptr, w, b, y, nullptr, mean, rstd, M, N, eps, dtype, w_dtype,
                      stream, false);
}

int add_layernorm_fwd(const void *x, const void *r, const void *w, const void *b, void *y,
                      void *residual_out, float *mean, float *rstd, int64_t M, int64_t N,
                      float eps, int dtype, int w_dtype, void *stream)
{
    return fwd_common(kLayer, x, r, w, b, y, residual_out, mean, rstd, M, N, eps, dtype, w_dtype,
                      stream, true);
}

size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N)
{
    if (M <= 0 || N <= 0)
        return 0;
    const uint64_t rows = (uint64_t)(M < kMaxPartials ? M : kMaxPartials);
    if ((uint64_t)N > (uint64_t)SIZE_MAX / 4u / rows)
        return 0;
    return (size_t)(rows * (uint64_t)N * 4u);
}

int rmsnorm_bwd(const void *dy, const void *x, const void *w, const float *rstd, void *dx,
                float *dw, void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                int dtype, int w_dtype, void *stream)
{
    return bwd_common(kRms, dy, nullptr, x, w, nullptr, rstd, dx, dw, nullptr, workspace,
                      workspace_bytes, M, N, dtype, w_dtype, stream);
}

int rmsnorm_bwd_noalloc(const void *dy, const void *x, const void *w, const float *rstd, void *dx,
                        float *dw, int64_t M, int64_t N, int dtype, int w_dtype, void *stream)
{
    // validate what needs no device first, so that bad arguments make no HIP call
    if (!w || !dw || (M != 0 && (!dy || !x || !rstd || !dx)))
        return ADDRMS_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(w_dtype))
        return ADDRMS_ERR_DTYPE;
    int rc = check_shape(M, N, dtype);
    if (rc != ADDRMS_OK)
        return rc;
    if ((uint64_t)N > ADDRMS_NOALLOC_SCRATCH_BYTES / sizeof(float))
        return ADDRMS_ERR_SCRATCH;
    void *ws = nullptr;
    if ((rc = scratch_ptr(&ws)) != ADDRMS_OK)
        return rc;
    return bwd_common(kRms, dy, nullptr, x, w, nullptr, rstd, dx, dw, nullptr, ws,
                      ADDRMS_NOALLOC_SCRATCH_BYTES, M, N, dtype, w_dtype, stream, true);
}

int add_rmsnorm_bwd(const void *dy, const void *dres, const void *h, const void *w,
                    const float *rstd, void *dh, float *dw, void *workspace,
                    size_t workspace_bytes, int64_t M, int64_t N, int dtype, int w_dtype,
                    void *stream)
{
    return bwd_common(kRms, dy, dres, h, w, nullptr, rstd, dh, dw, nullptr, workspace,
                      workspace_bytes, M, N, dtype, w_dtype, stream);
}

size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N)
{
    const size_t one = rmsnorm_bwd_workspace_bytes(M, N);
    return one <= SIZE_MAX / 2 ? 2 * one : 0;
}

int layernorm_bwd(const void *dy, const void *x, const void *w, const float *mean,
                  const float *rstd, void *dx, float *dw, float *db, void *workspace,
                  size_t workspace_bytes, int64_t M, int64_t N, int dtype, int w_dtype,
                  void *stream)
{
    return bwd_common(kLayer, dy, nullptr, x, w, mean, rstd, dx, dw, db, workspace,
                      workspace_bytes, M, N, dtype, w_dtype, stream);
}

int add_layernorm_bwd(const void *dy, const void *dres, const void *h, const void *w,
                      const float *mean, const float *rstd, void *dh, float *dw, float *db,
                      void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype,
                      int w_dtype, void *stream)
{
    return bwd_common(kLayer, dy, dres, h, w, mean, rstd, dh, dw, db, workspace, workspace_bytes,
                      M, N, dtype, w_dtype, stream);
}

int rmsnorm_rope_qk(const void *q, const void *k, const void *wq, const void *wk,
                    const float *cos, const float *sin, const int64_t *pos, int64_t P, void *q_out,
                    void *k_out, int64_t T, int64_t Hq, int64_t Hk, int64_t D, int64_t q_stride,
                    int64_t k_stride, int64_t q_out_stride, int64_t k_out_stride, float eps,
                    int interleaved, int dtype, int w_dtype, void *stream)
{
    return rope_common(q, k, wq, wk, cos, sin, pos, P, q_out, k_out, T, Hq, Hk, D, q_stride,
                       k_stride, q_out_stride, k_out_stride, eps, interleaved, dtype, w_dtype,
                       reinterpret_cast<hipStream_t>(stream));
}

const char *addrms_status_str(int status)
{
    switch (status) {
    case ADDRMS_OK: return "ok";
    case ADDRMS_ERR_NULL: return "a required pointer is NULL";
    case ADDRMS_ERR_SHAPE: return "invalid shape (M < 0, N <= 0, or too large)";
    case ADDRMS_ERR_DTYPE: return "unknown element type";
    case ADDRMS_ERR_EPS: return "eps must be finite and >= 0";
    case ADDRMS_ERR_ALIAS: return "output overlaps another argument";
    case ADDRMS_ERR_WORKSPACE: return "workspace missing or too small";
    case ADDRMS_ERR_HIP: return "HIP call failed";
    case ADDRMS_ERR_KNOB: return "unknown tuning knob";
    case ADDRMS_ERR_SCRATCH:
        return "a row is wider than the no-allocation backward's built-in scratch holds";
    default: return "unknown status";
    }
}

int addrms_last_hip_error(void) { return g_last_hip_error; }

int addrms_tune(int knob_id, int value)
{
    if (knob_id < 0 || knob_id >= ADDRMS_NUM_KNOBS)
        return ADDRMS_ERR_KNOB;
    if (value < 0)
        return knob(knob_id);
    return g_knobs.v[knob_id].exchange(value, std::memory_order_relaxed);
}

// The choices fwd_common and bwd_common make, through the same helpers, for
// aligned contiguous tensors and a given CU count.
int addrms_plan(int op, int norm, int fused, int qmode, int64_t qgroup, int64_t M, int64_t N,
                int dtype, int w_dtype, int cus, addrms_plan_t *out)
{
    if (!out)
        return ADDRMS_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(w_dtype))
        return ADDRMS_ERR_DTYPE;
    if (M < 1 || N < 1 || N > INT_MAX || cus < 1 || (op != ADDRMS_PLAN_FWD && op != ADDRMS_PLAN_BWD) ||
        (norm != kRms && norm != kLayer) || qmode < 0 || qmode > 3 || qgroup < 0 ||
        (qmode != 0 && (op != ADDRMS_PLAN_FWD || norm != kRms)))
        return ADDRMS_ERR_SHAPE;
    *out = addrms_plan_t{0, 0, 0, 0, 0, 0};
    const bool res = fused != 0;
    const int nv = vec_elems(dtype);
    const bool vec_ok = knob(ADDRMS_KNOB_FORCE_ELEM) == 0 && N % nv == 0;
    const int nvec = (int)(N / nv);
    int wi = 0, vi = 0;
    if (op == ADDRMS_PLAN_FWD) {
        const FwdTable &tab = fwd_table(combo(dtype, w_dtype));
        const bool q8 = qmode != 0;
        const bool mx = qmode == 3;
        int64_t g = mx ? 32 : qmode == 2 ? (qgroup >= N ? 0 : qgroup) : 0;
        int qlanes = 0;
        if (g > 0 && g % nv == 0) {
            const int64_t L = g / nv;
            if (L <= 64 && (L & (L - 1)) == 0)
                qlanes = (int)L;
        }
        const int qm = mx ? kQMx - 1 : g > 0 ? kQGroup - 1 : kQRow - 1;
        if (vec_ok && (g == 0 || qlanes > 0) &&
            pick_fwd(M, nvec, cus, norm, res, q8 ? qm + 1 : (int)kQNone, &wi, &vi) &&
            (!q8 || tab.vec_q8[res ? 1 : 0][qm][wi][vi].fn != nullptr)) {
            out->vector = 1;
            out->waves_per_row = kWprList[wi];
            out->vectors_per_lane = kVplList[vi];
        }
        return ADDRMS_OK;
    }
    const BwdTable &tab = bwd_table(combo(dtype, w_dtype));
    int m_wpr = 0, m_pf = 0;
    bool measured =
        vec_ok && bwd_measured_choice(norm, res, dtype != ADDRMS_F32, M, nvec, cus, &m_wpr, &m_pf);
    if (measured) {
        vi = vpl_index((nvec + 64 * m_wpr - 1) / (64 * m_wpr));
        wi = m_wpr == 2 ? 1 : m_wpr == 4 ? 2 : m_wpr == 8 ? 3 : -1;
        measured = vi >= 0 && wi >= 0 && bwd_built(norm, res, m_wpr, kVplList[vi]) &&
                   (size_t)(bwd_rpb(m_wpr) / 2) * (size_t)N * 4u <= kMaxDynLds &&
                   (m_pf == 1 ? tab.pf[norm][res ? 1 : 0][wi][vi].fn
                              : tab.vec[norm][res ? 1 : 0][wi][vi].fn) != nullptr;
    }
    if (measured || (vec_ok && pick_bwd(norm, res, M, (int)N, nvec, cus, &wi, &vi))) {
        const bool wide = !measured && use_wide_bwd(tab, norm, res, M, N, wi, vi, cus);
        out->vector = 1;
        out->waves_per_row = wide ? kBwdWideWpr : kWprList[wi];
        out->vectors_per_lane = kVplList[vi];
        out->wide = wide ? 1 : 0;
        out->prefetch = (measured ? m_pf == 1 : !wide && use_prefetch_bwd(tab, norm, res, wi, vi)) ? 1 : 0;
        const bool two = measured || (norm == kRms && !wide && knob(ADDRMS_KNOB_BLOCKS_PER_CU) == 0 &&
                                      nvec >= (dtype == ADDRMS_F32 ? 512 : 256) && M >= 48LL * cus);
        out->blocks_per_cu = two ? 2 : 0;
    }
    return ADDRMS_OK;
}

} // extern "C"
