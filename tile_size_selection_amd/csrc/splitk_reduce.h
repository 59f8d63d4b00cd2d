// Split-K reduction: the second pass of a GEMM (or convolution) whose K
// loop was cut into `splits` ranges computed by separate blocks.  Each range
// wrote its fp32 partial sums into its own slice of a workspace; this pass
// adds the slices of every output element in range order (0, 1, ...,
// splits-1), converts the sum to the output type (round to nearest even)
// and writes it.  A fixed order of the additions makes the result the same
// bits on every run (no atomics).
//
// Layout: P[b][s][i] for batch entry b < batch, range s < splits and element
// i < mn (the GEMM's (b * splits + s) output slices; a convolution has
// batch = 1 and mn = its whole output).  out[b][i].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace tss {

constexpr int kReduceThreads = 256;

// VEC: each thread takes 4 consecutive elements (mn % 4 == 0: 16-byte loads
// of every slice, one 4-element store); otherwise one element.
template <typename O, bool VEC>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const float *__restrict__ P, O *__restrict__ out,
                                                                       int64_t batch, int64_t mn, int32_t splits) {
  constexpr int V = VEC ? 4 : 1;
  const int64_t per_b = mn / V;
  const int64_t total = batch * per_b;
  for (int64_t u = int64_t(blockIdx.x) * kReduceThreads + threadIdx.x; u < total;
       u += int64_t(gridDim.x) * kReduceThreads) {
    const int64_t b = u / per_b, i = (u - b * per_b) * V;
    const float *src = P + b * splits * mn + i;
    if constexpr (VEC) {
      f32x4 acc = *(const f32x4 *)src;
      for (int s = 1; s < splits; ++s) {
        const f32x4 v = *(const f32x4 *)(src + int64_t(s) * mn);
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
      }
      typename Vec4<O>::type r;
      r[0] = convert_out<O>(acc[0]);
      r[1] = convert_out<O>(acc[1]);
      r[2] = convert_out<O>(acc[2]);
      r[3] = convert_out<O>(acc[3]);
      *(typename Vec4<O>::type *)(out + b * mn + i) = r;
    } else {
      float acc = src[0];
      for (int s = 1; s < splits; ++s) acc += src[int64_t(s) * mn];
      out[b * mn + i] = convert_out<O>(acc);
    }
  }
}

// Launch on `s`: out (dtype out_dtype) = the sum over ranges of P.
inline hipError_t launch_splitk_reduce(const float *P, void *out, int32_t out_dtype, int64_t batch, int64_t mn,
                                       int32_t splits, hipStream_t s) {
  const bool vec = mn % 4 == 0 && (reinterpret_cast<uintptr_t>(out) % (out_dtype == TSS_F32 ? 16 : 8)) == 0;
  const int64_t work = batch * (vec ? mn / 4 : mn);
  if (work == 0) return hipSuccess;
  const int64_t want = (work + kReduceThreads - 1) / kReduceThreads;
  const dim3 grid(uint32_t(want < 8192 ? want : 8192)), block(kReduceThreads);
  if (out_dtype == TSS_F32) {
    if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<float, true>), grid, block, 0, s, P, (float *)out, batch, mn, splits);
    else hipLaunchKernelGGL((splitk_reduce_kernel<float, false>), grid, block, 0, s, P, (float *)out, batch, mn, splits);
  } else if (out_dtype == TSS_F16) {
    if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<_Float16, true>), grid, block, 0, s, P, (_Float16 *)out, batch, mn, splits);
    else hipLaunchKernelGGL((splitk_reduce_kernel<_Float16, false>), grid, block, 0, s, P, (_Float16 *)out, batch, mn, splits);
  } else {
    if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<__bf16, true>), grid, block, 0, s, P, (__bf16 *)out, batch, mn, splits);
    else hipLaunchKernelGGL((splitk_reduce_kernel<__bf16, false>), grid, block, 0, s, P, (__bf16 *)out, batch, mn, splits);
  }
  return hipGetLastError();
}

}  // namespace tss
