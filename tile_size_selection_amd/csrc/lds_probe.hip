// LDS bank microbenchmark: the gfx950 analogue of the Tiling page's bank
// conflict table (section on shared-memory bank conflicts and the XOR
// swizzle: lanes reading words `stride` apart conflict when they fall in the
// same bank, and a row-xor-column swizzle removes it).
//
// Every wave of `blocks` 512-thread blocks times, with the shader clock
// (s_memtime), `iters` x 8 LDS reads of one address pattern:
//   strided patterns: lane l reads at byte l * stride_words * 4, with 4-byte
//     (ds_read_b32), 16-byte (ds_read_b128) or 8-byte transposing
//     (ds_read_b64_tr_b16) reads;
//   the GEMM's own fragment patterns (256x256x64 tile, 8 waves, 16x16x32
//     MFMA): the A fragment read (K-contiguous rows, ds_read_b128) and the B
//     fragment read (N-contiguous rows, ds_read_b64_tr_b16), with the XOR
//     swizzle the kernel uses and without it.
// The 8 reads of an iteration step by 2 KiB, a multiple of the 256-byte bank
// span, so each sees the same bank pattern.
#include "gemm_kernel.h"

namespace tss {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBytes = 65536;  // LDS the reads cover
using ProbeGeometry = Geometry<256, 256, 64, 2, 8, 16>;

template <int P>
__global__ __launch_bounds__(kProbeThreads) void lds_probe_kernel(int stride_words, int iters, int64_t *cycles) {
  extern __shared__ __attribute__((aligned(16))) char buf[];
  typedef int i32x4v __attribute__((ext_vector_type(4)));
  for (int i = threadIdx.x * 16; i < kProbeBytes + 16384; i += kProbeThreads * 16)
    *(__attribute__((address_space(3))) i32x4v *)(buf + i) = i32x4v{i, i + 1, i + 2, i + 3};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  using G = ProbeGeometry;
  uint32_t base;
  if constexpr (P == TSS_LDS_GEMM_A || P == TSS_LDS_GEMM_A_PLAIN)
    base = G::frag_k_rows((wave / G::WN) * G::WTM, lane, 0, P == TSS_LDS_GEMM_A);
  else if constexpr (P == TSS_LDS_GEMM_B || P == TSS_LDS_GEMM_B_PLAIN)
    base = G::frag_n_rows((wave % G::WN) * G::WTN, lane, P == TSS_LDS_GEMM_B);
  else
    base = uint32_t(lane * stride_words * 4) % uint32_t(kProbeBytes);
  int acc = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    // the addresses do not change between iterations: keep the reads inside
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const char *a = buf + (base + uint32_t(u) * 2048u) % uint32_t(kProbeBytes);
      if constexpr (P == TSS_LDS_B32) {
        acc ^= *(const __attribute__((address_space(3))) int *)a;
      } else if constexpr (P == TSS_LDS_B128 || P == TSS_LDS_GEMM_A || P == TSS_LDS_GEMM_A_PLAIN) {
        const i16x8 v = *(const lds_i16x8 *)a;
        acc ^= int(v[0]) ^ int(v[7]);
      } else {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)a);
        acc ^= int(v[0]) ^ int(v[3]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every read has returned
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  // the data decides nothing; the comparison keeps the reads alive
  if (lane == 0) cycles[blockIdx.x * (kProbeThreads / 64) + wave] = acc == 0x7fffffff ? -1 : int64_t(t1 - t0);
}

template <int P>
hipError_t launch_probe(int stride_words, int iters, int blocks, int64_t *cycles, hipStream_t s) {
  const int lds = kProbeBytes + 16384;
  hipError_t e = hipFuncSetAttribute((const void *)lds_probe_kernel<P>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lds_probe_kernel<P>, dim3(blocks), dim3(kProbeThreads), lds, s, stride_words, iters, cycles);
  return hipGetLastError();
}

}  // namespace
}  // namespace tss

extern "C" int32_t tss_lds_probe(int32_t pattern, int32_t stride_words, int32_t iters, int32_t blocks,
                                 int64_t *cycles, void *stream) {
  using namespace tss;
  if (!cycles || stride_words < 0 || stride_words > 4096 || iters < 1 || iters > (1 << 20) || blocks < 1 ||
      blocks > 65536)
    return TSS_E_ARG;
  // each read's natural alignment: 16 bytes for ds_read_b128, 8 for the transpose read
  if ((pattern == TSS_LDS_B128 && stride_words % 4) || (pattern == TSS_LDS_TR_B64 && stride_words % 2))
    return TSS_E_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (pattern) {
    case TSS_LDS_B32: e = launch_probe<TSS_LDS_B32>(stride_words, iters, blocks, cycles, s); break;
    case TSS_LDS_B128: e = launch_probe<TSS_LDS_B128>(stride_words, iters, blocks, cycles, s); break;
    case TSS_LDS_TR_B64: e = launch_probe<TSS_LDS_TR_B64>(stride_words, iters, blocks, cycles, s); break;
    case TSS_LDS_GEMM_A: e = launch_probe<TSS_LDS_GEMM_A>(stride_words, iters, blocks, cycles, s); break;
    case TSS_LDS_GEMM_A_PLAIN: e = launch_probe<TSS_LDS_GEMM_A_PLAIN>(stride_words, iters, blocks, cycles, s); break;
    case TSS_LDS_GEMM_B: e = launch_probe<TSS_LDS_GEMM_B>(stride_words, iters, blocks, cycles, s); break;
    case TSS_LDS_GEMM_B_PLAIN: e = launch_probe<TSS_LDS_GEMM_B_PLAIN>(stride_words, iters, blocks, cycles, s); break;
    default: return TSS_E_ARG;
  }
  return e == hipSuccess ? TSS_OK : TSS_E_HIP;
}
