// sm_rows_bf16.hip -- row-softmax kernel instances for the bf16 dtype.
#define SM_DT ::smx::kBF16
#define SM_ROW_FN row_kernel_bf16
#include "sm_rows_inst.inl"
