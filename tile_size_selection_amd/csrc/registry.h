// Table of compiled kernels.  Each instantiation unit contributes the kernels
// of one (input dtype, operation, BM) slice of the gfx950 candidate space;
// a shape is compiled exactly when the planner's C3/C1/C2/occupancy checks
// pass for it at the lightest pipeline depth (planner.h,
// kernel_shape_needed), so every feasible configuration has a kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gemm_kernel.h"

namespace tss {

using Launch = hipError_t (*)(const KernelArgs &, dim3 grid, int lds_bytes, hipStream_t s);
// code object attributes of the kernel, and the blocks per CU the runtime
// allows at its block size with lds_bytes of dynamic LDS
using Usage = hipError_t (*)(hipFuncAttributes *attr, int *blocks_per_cu, int lds_bytes);

struct KernelEntry {
  int32_t bm, bn, bk, stages, threads, instr, dtype, op;  // op 0 = GEMM, 1 = conv
  Launch launch;
  int32_t lds_bytes;  // dynamic LDS of one block
  Usage usage;
};

struct KernelTable {
  const KernelEntry *entries;
  int n;
};

// Defined by the instantiation units.
KernelTable table_gemm_f16_bm64();
KernelTable table_gemm_f16_bm128();
KernelTable table_gemm_f16_bm256();
KernelTable table_gemm_bf16_bm64();
KernelTable table_gemm_bf16_bm128();
KernelTable table_gemm_bf16_bm256();
KernelTable table_conv_f16_bm64();
KernelTable table_conv_f16_bm128();
KernelTable table_conv_f16_bm256();
KernelTable table_conv_bf16_bm64();
KernelTable table_conv_bf16_bm128();
KernelTable table_conv_bf16_bm256();
KernelTable table_gemm_f16_bm128_wide();
KernelTable table_gemm_f16_bm256_wide();
KernelTable table_gemm_bf16_bm128_wide();
KernelTable table_gemm_bf16_bm256_wide();
KernelTable table_conv_f16_bm128_wide();
KernelTable table_conv_f16_bm256_wide();
KernelTable table_conv_bf16_bm128_wide();
KernelTable table_conv_bf16_bm256_wide();

// Dynamic LDS above 64 KiB needs a per-kernel attribute, which HIP keeps per
// device: it is set on the first launch on each device (up to 64 devices).
template <typename G, typename T, bool CONV>
hipError_t launch_kernel(const KernelArgs &a, dim3 grid, int lds_bytes, hipStream_t s) {
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)tiled_gemm_kernel<G, T, CONV>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            163840);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((tiled_gemm_kernel<G, T, CONV>), grid, dim3(G::THREADS), lds_bytes, s, a);
  return hipGetLastError();
}

template <typename G, typename T, bool CONV>
hipError_t kernel_usage(hipFuncAttributes *attr, int *blocks_per_cu, int lds_bytes) {
  const void *f = (const void *)tiled_gemm_kernel<G, T, CONV>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  if (e == hipSuccess) e = hipFuncGetAttributes(attr, f);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, G::THREADS, lds_bytes);
  return e;
}

}  // namespace tss
