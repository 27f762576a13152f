// sm_rows_f16.hip -- row-softmax kernel instances for the f16 dtype.
#define SM_DT ::smx::kF16
#define SM_ROW_FN row_kernel_f16
#include "sm_rows_inst.inl"
