// Kernels with 256 accumulators per lane for gemm with bf16 inputs and block rows BM = 128.
#define TSS_T __bf16
#define TSS_DT TSS_BF16
#define TSS_OP 0
#define TSS_BM 128
#define TSS_TABLE table_gemm_bf16_bm128_wide
#define TSS_WIDE 1
#include "../instances.inc"
