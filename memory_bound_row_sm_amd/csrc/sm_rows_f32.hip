// sm_rows_f32.hip -- row-softmax kernel instances for the f32 dtype.
#define SM_DT ::smx::kF32
#define SM_ROW_FN row_kernel_f32
#include "sm_rows_inst.inl"
