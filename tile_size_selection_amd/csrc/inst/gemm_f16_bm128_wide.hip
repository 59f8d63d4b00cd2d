// Kernels with 256 accumulators per lane for gemm with f16 inputs and block rows BM = 128.
#define TSS_T _Float16
#define TSS_DT TSS_F16
#define TSS_OP 0
#define TSS_BM 128
#define TSS_TABLE table_gemm_f16_bm128_wide
#define TSS_WIDE 1
#include "../instances.inc"
