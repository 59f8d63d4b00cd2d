// Kernels for conv with f16 inputs and block rows BM = 64.
#define TSS_T _Float16
#define TSS_DT TSS_F16
#define TSS_OP 1
#define TSS_BM 64
#define TSS_TABLE table_conv_f16_bm64
#define TSS_WIDE 0
#include "../instances.inc"
