// Kernels for gemm with bf16 inputs and block rows BM = 64.
#define TSS_T __bf16
#define TSS_DT TSS_BF16
#define TSS_OP 0
#define TSS_BM 64
#define TSS_TABLE table_gemm_bf16_bm64
#define TSS_WIDE 0
#include "../instances.inc"
