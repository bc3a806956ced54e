// Internal interface between the C-ABI dispatcher and the kernel translation
// units: argument blocks and the per-dtype kernel tables.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace addrms {

// Forward arguments (plain op: r and residual_out are unused).
struct FwdArgs {
    const void *x;
    const void *r;
    const void *w;
    const void *b; // LayerNorm bias (w's dtype); may be null
    void *y;
    void *res;
    float *mean; // LayerNorm only; may be null
    float *rstd; // may be null
    uint8_t *q;     // quantised output: E4M3 codes [M, N] or packed E2M1 [M, N/2]
    void *qscale;   // its scales: float32 [M] or [M, qgroups] (E4M3), E8M0 bytes
                    // [M, qgroups] (MXFP4)
    int64_t M;
    int N;
    int nvec; // 16-byte vectors per row (vector path)
    float eps;
    // FP8 scale groups: qgroup = columns per scale (0: one scale per row),
    // qgroups = scales per row, qlanes = lanes per group on the vector path
    // (qgroup / values per vector, a power of two up to 64).
    int qgroup;
    int qgroups;
    int qlanes;
};

// Per-head RMSNorm + RoPE arguments.  Head h of token t is the D contiguous
// values at q + t*q_stride + h*D (h < Hq) or k + t*k_stride + (h-Hq)*D;
// strides are in elements.  cos/sin: float32 [P, D/2]; pos: int64 [T].
struct RopeArgs {
    const void *q;
    const void *k;
    const void *wq;
    const void *wk;
    const float *cos;
    const float *sin;
    const int64_t *pos;
    void *qo;
    void *ko;
    int64_t q_stride, k_stride, qo_stride, ko_stride;
    int64_t T;
    int64_t P;
    int Hq, Hk, D;
    float eps;
};

// Which normalisation a kernel computes.
enum Norm : int { kRms = 0, kLayer = 1 };

// Backward arguments.  For the fused op's backward, x is the saved residual
// h, dres the gradient of residual_out (added to dx), and dx receives dh.
struct BwdArgs {
    const void *dy;
    const void *dres; // fused backward only
    const void *x;
    const void *w;
    const float *mean; // LayerNorm only
    const float *rstd;
    void *dx;
    float *ws;  // [P, N] float partial sums of dw
    float *ws2; // [P, N] float partial sums of db (LayerNorm)
    int64_t M;
    int N;
    int nvec;
    int P;          // partial rows (element-wise path: row chunks)
    int64_t chunk;  // rows per chunk (element-wise dw path)
};

// Supported shapes of the vector kernels: waves per row and 16-byte vectors per
// lane.  A row of nvec vectors needs WPR * 64 * VPL >= nvec.
constexpr int kWprList[] = {1, 2, 4, 8, 16};
constexpr int kNumWpr = 5;
constexpr int kVplList[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16};
constexpr int kNumVpl = 12;
constexpr int kMaxVpl = 16;

// Backward vector kernels use 256-thread blocks and WPR in {1, 2, 4}.
constexpr int kBwdNumWpr = 4; // backward: WPR in {1, 2, 4, 8}

constexpr int kBlockFwd(int wpr) { return wpr == 1 ? 256 : 64 * wpr; }

// Forward (WPR, VPL) pairs that are built: 512- and 1024-thread blocks get at
// most 256 / 128 VGPRs per lane, so they only take rows short enough per lane
// to stay in registers.
// Quantised outputs with per-group scales (E4M3 groups, MXFP4 blocks) on the
// vector path: instantiated for at most this many vectors per lane (with 8,
// some variants spill registers); bf16 rows up to 32768 qualify, longer rows
// take the element-wise path.
constexpr int kQGroupMaxVpl = 4;
constexpr int kMxMaxVpl = 4;
constexpr bool fwd_built(int wpr, int vpl)
{
    return wpr <= 4 || (wpr == 8 && vpl <= 8) || (wpr == 16 && vpl <= 4);
}
// Quantised outputs of the forward (RMSNorm): none; E4M3 with one float32
// scale per row; E4M3 with one per group of columns; MXFP4 (E2M1 codes two
// per byte, one E8M0 scale byte per 32 values).  Each is its own kernel.
enum QMode : int { kQNone = 0, kQRow = 1, kQGroup = 2, kQMx = 3 };
constexpr bool q_built(int qm, int wpr, int vpl)
{
    return fwd_built(wpr, vpl) && (qm != kQGroup || vpl <= kQGroupMaxVpl) &&
           (qm != kQMx || vpl <= kMxMaxVpl);
}
// Backward variants that are instantiated.  The LayerNorm backward with the
// residual gradient at 16 vectors per lane needs more than the 512 VGPRs a
// lane can hold and would spill to scratch; those rows take the element-wise
// path instead.  8 waves per row (512-thread blocks, at most 256 VGPRs a
// lane) is built up to 4 vectors per lane.
constexpr bool bwd_built(int norm, bool res, int wpr, int vpl)
{
    return !(norm == kLayer && res && vpl > 14) && !(wpr == 8 && vpl > 4);
}
constexpr int kBwdBlock = 256;
constexpr int kBwdWideBlock = 1024;
// Backward vector kernels: 256-thread blocks holding 4 / WPR rows per step,
// except WPR = 8, whose 512-thread blocks hold one row.  The wide variant
// (WIDE) is one 1024-thread block per CU with 2 waves per row, 8 rows per
// step: a quarter of the dw partial rows of four 256-thread blocks.
constexpr int kBwdBlockOf(int wpr, bool wide = false)
{
    return wide ? kBwdWideBlock : wpr == 8 ? 512 : kBwdBlock;
}
constexpr int bwd_rpb(int wpr, bool wide = false)
{
    return wide ? kBwdWideBlock / (64 * wpr) : wpr == 8 ? 1 : 4 / wpr;
}
constexpr int kBwdWideWpr = 2;
constexpr int kColReduceCols = 16;    // dw columns per element-wise column-reduce block
constexpr int kColReduceVecCols = 32; // per vector column-reduce block (128-byte rows)
constexpr int kColReduceVecBlock = 1024;

// A kernel entry: function, block size, dynamic LDS bytes (backward: per
// column of N), and whether it is an element-wise fallback.
struct KernelRef {
    const void *fn;
    int block;
};

// Dtype combination index: (row dtype, weight dtype) -> 0..8, with
// dtype codes ADDRMS_F32 = 0, ADDRMS_BF16 = 1, ADDRMS_F16 = 2.
inline int combo(int dtype, int w_dtype) { return dtype * 3 + w_dtype; }

// Kernel tables, one translation unit per dtype combination.
// fwd vec: [norm][fused][wpr_idx][vpl_idx]; fwd elem: [norm][fused].
struct FwdTable {
    KernelRef vec[2][2][kNumWpr][kNumVpl];
    KernelRef elem[2][2];
    // RMSNorm with a quantised output: [fused][mode - 1][wpr][vpl], [fused][mode - 1]
    KernelRef vec_q8[2][3][kNumWpr][kNumVpl];
    KernelRef elem_q8[2][3];
};
// bwd vec: [norm][with residual gradient][wpr_idx][vpl_idx]; elem_dx:
// [norm][with residual gradient]; elem_dw: [norm].
struct BwdTable {
    KernelRef vec[2][2][kBwdNumWpr][kNumVpl];
    KernelRef wide[2][2][kNumVpl]; // WPR = kBwdWideWpr in 1024-thread blocks; null where not built
    KernelRef pf[2][2][kBwdNumWpr][kNumVpl]; // next-row prefetch (2 waves per row); null where not built
    KernelRef elem_dx[2][2];
    KernelRef elem_dw[2];
};

// RMSNorm + RoPE: vec [interleaved][log2 of the lanes per head, 0..6][log2
// of the heads per lane group and loop step, 0..2] (the 16-byte vector path),
// elem [interleaved].
constexpr int kRopeNumGroups = 7;
constexpr int kRopeNumHpl = 3;
// With one lane per head, four heads per step spill scalar registers: not
// instantiated (two are used instead).
constexpr bool rope_built(int g, int hpl) { return !(g == 1 && hpl == 4); }
constexpr int kRopeBlock = 256;
struct RopeTable {
    KernelRef vec[2][kRopeNumGroups][kRopeNumHpl];
    KernelRef elem[2];
};

const FwdTable &fwd_table(int combo_idx);
const RopeTable &rope_table(int combo_idx);
const BwdTable &bwd_table(int combo_idx);
KernelRef colreduce_kernel(bool vec);

} // namespace addrms
