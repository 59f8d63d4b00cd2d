// Kernels for conv with bf16 inputs and block rows BM = 64.
#define TSS_T __bf16
#define TSS_DT TSS_BF16
#define TSS_OP 1
#define TSS_BM 64
#define TSS_TABLE table_conv_bf16_bm64
#define TSS_WIDE 0
#include "../instances.inc"
