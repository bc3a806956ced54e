// Kernel tables for one (row dtype, weight dtype) combination, selected at
// compile time by ADDRMS_COMBO = 2 * row_dtype + weight_dtype (0 = float32,
// 1 = bfloat16).  The build compiles this file once per combination so the
// instantiations compile in parallel.
#include "kernels.hpp"

#ifndef ADDRMS_COMBO
#error "define ADDRMS_COMBO (0..3)"
#endif

#if ADDRMS_COMBO == 0
#define ADDRMS_ROW_T float
#define ADDRMS_W_T float
#elif ADDRMS_COMBO == 1
#define ADDRMS_ROW_T float
#define ADDRMS_W_T addrms::bf16_t
#elif ADDRMS_COMBO == 2
#define ADDRMS_ROW_T addrms::bf16_t
#define ADDRMS_W_T float
#else
#define ADDRMS_ROW_T addrms::bf16_t
#define ADDRMS_W_T addrms::bf16_t
#endif

#define ADDRMS_CAT2(a, b) a##b
#define ADDRMS_CAT(a, b) ADDRMS_CAT2(a, b)

namespace addrms {

const FwdTable &ADDRMS_CAT(fwd_table_, ADDRMS_COMBO)()
{
    static const FwdTable t = TableBuilder<ADDRMS_ROW_T, ADDRMS_W_T>::fwd();
    return t;
}

const BwdTable &ADDRMS_CAT(bwd_table_, ADDRMS_COMBO)()
{
    static const BwdTable t = TableBuilder<ADDRMS_ROW_T, ADDRMS_W_T>::bwd();
    return t;
}

#if ADDRMS_COMBO == 0
KernelRef colreduce_kernel(bool vec)
{
    return vec ? KernelRef{reinterpret_cast<const void *>(&dw_colreduce_vec_kernel<0>), kColReduceVecBlock}
               : KernelRef{reinterpret_cast<const void *>(&dw_colreduce_kernel<0>), 256};
}
#endif

} // namespace addrms
