// Kernel tables for one (row dtype, weight dtype) combination, selected at
// compile time by ADDRMS_COMBO (combo_types.hpp).
#include "kernels.hpp"

#include "combo_types.hpp"

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
