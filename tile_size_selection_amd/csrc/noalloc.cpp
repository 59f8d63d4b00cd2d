// tss_conv2d_splitk_noalloc: the convolution with its workspace in a static
// device array of the library, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Nothing here allocates: the array is part of the code
// object, loaded once per GPU, and its address on a GPU is read once, with
// that GPU current, through hipGetSymbolAddress.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/tss.h"

namespace {

// The scratch array.  In host code its name stands for the symbol, not for a
// device address: only the pointer read by hipGetSymbolAddress is ever handed
// to a kernel or a copy.
static __device__ __attribute__((aligned(256))) char scratch[TSS_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void *> g_ptr[kMaxDevices];

// The array's address on the current device (set up on the first call there).
int32_t scratch_on_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TSS_E_HIP;
  void *p = g_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(g_mu);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TSS_E_HIP;
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TSS_OK;
}

}  // namespace

extern "C" int32_t tss_conv2d_splitk_noalloc(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                                             int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                                             int64_t dw, int64_t tile_n, int64_t tile_oh, int64_t tile_ow,
                                             int32_t dtype, int32_t out_dtype, const void *x, const void *w, void *y,
                                             int32_t splits, const tss_tile_config *cfg, void *stream) {
  if (splits < 0 || splits > 256) return TSS_E_ARG;
  int32_t S = splits;
  if (S == 0) {
    // the count the convolution will take: the split-K plan's
    if (sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || N < 1 || H < 1 || W < 1 || kh < 1 || kw < 1 ||
        H + 2 * ph < (kh - 1) * dh + 1 || W + 2 * pw < (kw - 1) * dw + 1)
      return TSS_E_ARG;
    const int64_t OH = (H + 2 * ph - (kh - 1) * dh - 1) / sh + 1;
    const int64_t OW = (W + 2 * pw - (kw - 1) * dw - 1) / sw + 1;
    tss_verdict v;
    int32_t st = tss_conv_splitk_plan(Cout, N * OH * OW, C, kh * kw, 2, nullptr, &v, &S);
    if (st != TSS_OK) return st;
  }
  const int64_t need = tss_conv2d_splitk_workspace_size(N, C, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, S);
  if (need < 0) return int32_t(need);
  if (need > TSS_SCRATCH_BYTES) return TSS_E_SCRATCH;
  void *ws = nullptr;
  int32_t st = scratch_on_current_device(&ws);
  if (st != TSS_OK) return st;
  return tss_conv2d_splitk(N, C, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, tile_n, tile_oh, tile_ow, dtype,
                           out_dtype, x, w, y, splits, ws, TSS_SCRATCH_BYTES, cfg, stream);
}
