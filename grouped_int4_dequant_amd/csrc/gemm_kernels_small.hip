// The grouped GEMM of gemm_kernels.hip compiled for work units of at most
// 32 rows (two 16-row MFMA blocks) at three workgroups per CU, exported as
// launch_gemm_small. When a call's experts hold few rows each (short
// prompts), its items are short and stream their weights; the smaller
// register and LDS footprint lets a third workgroup share each CU, so more
// weight requests are in flight.
#define MOE_UNIT_ROWS 32
#define MOE_GEMM_WGS_PER_CU 3
#define MOE_GEMM_LAUNCH launch_gemm_small
#define MOE_GEMM_SMALL_BUILD 1
#include "gemm_kernels.hip"

static_assert(moe::kUnitRows == moe::kUnitRowsSmall, "the small build's unit size");
