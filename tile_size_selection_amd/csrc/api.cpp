// C ABI of the device operations: tss_gemm, tss_conv2d and their helpers.
// Argument checks happen before any launch; nothing here allocates device
// memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "conv_layout.h"
#include "planner.h"
#include "registry.h"
#include "splitk_reduce.h"

using namespace tss;

namespace {

struct Key {
  int32_t bm, bn, bk, stages, threads, instr, dtype, op;
  bool operator<(const Key &o) const {
    return std::tie(bm, bn, bk, stages, threads, instr, dtype, op) <
           std::tie(o.bm, o.bn, o.bk, o.stages, o.threads, o.instr, o.dtype, o.op);
  }
};

const std::map<Key, KernelEntry> &registry() {
  static const std::map<Key, KernelEntry> reg = [] {
    std::map<Key, KernelEntry> m;
    KernelTable (*tables[])() = {table_gemm_f16_bm64,  table_gemm_f16_bm128,  table_gemm_f16_bm256,
                                 table_gemm_bf16_bm64, table_gemm_bf16_bm128, table_gemm_bf16_bm256,
                                 table_conv_f16_bm64,  table_conv_f16_bm128,  table_conv_f16_bm256,
                                 table_conv_bf16_bm64, table_conv_bf16_bm128, table_conv_bf16_bm256,
                                 table_gemm_f16_bm128_wide,  table_gemm_f16_bm256_wide,
                                 table_gemm_bf16_bm128_wide, table_gemm_bf16_bm256_wide,
                                 table_conv_f16_bm128_wide,  table_conv_f16_bm256_wide,
                                 table_conv_bf16_bm128_wide, table_conv_bf16_bm256_wide};
    for (auto fn : tables) {
      KernelTable t = fn();
      for (int i = 0; i < t.n; ++i) {
        const KernelEntry &e = t.entries[i];
        if (!e.launch) continue;
        m[Key{e.bm, e.bn, e.bk, e.stages, e.threads, e.instr, e.dtype, e.op}] = e;
      }
    }
    return m;
  }();
  return reg;
}

const KernelEntry *find_kernel(const tss_tile_config &c, int32_t dtype, int32_t op) {
  const auto &r = registry();
  auto it = r.find(Key{c.bm, c.bn, c.bk, c.stages, c.threads, c.instr, dtype, op});
  return it == r.end() ? nullptr : &it->second;
}

// Planner choice per problem, cached (planning evaluates every candidate).
// conv = false: the GEMM (a, b, c, d) = (batch, M, N, K); conv = true: the
// implicit GEMM of a convolution, (Cout, pixels, C, taps).
int32_t planned_config(bool conv, int64_t a, int64_t b, int64_t c, int64_t d, tss_tile_config *out) {
  using PKey = std::tuple<bool, int64_t, int64_t, int64_t, int64_t>;
  static std::mutex mu;
  static std::map<PKey, tss_tile_config> cache;
  PKey key{conv, a, b, c, d};
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *out = it->second;
      return TSS_OK;
    }
  }
  tss_verdict best{};
  int32_t st = conv ? tss_conv_plan(a, b, c, d, 2, nullptr, &best, nullptr, 0, nullptr)
                    : tss_tile_plan(a, b, c, d, 2, nullptr, 0, &best, nullptr, 0, nullptr);
  if (st != TSS_OK) return st;
  {
    std::lock_guard<std::mutex> g(mu);
    if (cache.size() >= 4096) cache.clear();  // bounded for long-running callers with many shapes
    cache[key] = best.cfg;
  }
  *out = best.cfg;
  return TSS_OK;
}

// The split-K plan per problem, cached like planned_config: (tile, splits).
int32_t planned_split(bool conv, int64_t a, int64_t b, int64_t c, int64_t d, tss_tile_config *out, int32_t *splits) {
  using PKey = std::tuple<bool, int64_t, int64_t, int64_t, int64_t>;
  static std::mutex mu;
  static std::map<PKey, std::pair<tss_tile_config, int32_t>> cache;
  PKey key{conv, a, b, c, d};
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *out = it->second.first;
      *splits = it->second.second;
      return TSS_OK;
    }
  }
  tss_verdict best{};
  int32_t S = 0;  // let the plan choose
  int32_t st = conv ? tss_conv_splitk_plan(a, b, c, d, 2, nullptr, &best, &S)
                    : tss_splitk_plan(a, b, c, d, 2, nullptr, &best, &S);
  if (st != TSS_OK) return st;
  {
    std::lock_guard<std::mutex> g(mu);
    if (cache.size() >= 4096) cache.clear();
    cache[key] = {best.cfg, S};
  }
  *out = best.cfg;
  *splits = S;
  return TSS_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_config(const tss_tile_config &c) {
  const tss_device d = gfx950_device();
  if (c.bm <= 0 || c.bn <= 0 || c.bk <= 0 || c.stages <= 0 || c.threads <= 0 || !instr_on_device(c.instr, d))
    return TSS_E_ARG;
  if (evaluate_block(c, d, 2).failures) return TSS_E_INFEASIBLE;
  return TSS_OK;
}

int group_m_for(int tiles_m) {
  int g = 4;
  return tiles_m < g ? (tiles_m > 0 ? tiles_m : 1) : g;
}

constexpr int64_t kTwoGiB = int64_t(1) << 31;
constexpr int64_t kConvChannelAlignMax = 64;  // the largest BK of the gfx950 candidate space

// Workspace of tss_conv2d: the channel-last input copy xc, then (at a
// 256-byte aligned offset) the reordered weights wr.
struct ConvWorkspace {
  int64_t Cp, xc_bytes, wr_offset, wr_bytes, total;
};
// Cp = C rounded up to a multiple of `align` (the tile's BK when launching,
// so that a K tile never straddles two taps; 64, the largest BK, for the
// size a caller allocates).
ConvWorkspace conv_workspace(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw,
                             int64_t align) {
  ConvWorkspace ws;
  ws.Cp = (C + align - 1) / align * align;
  ws.xc_bytes = N * H * W * ws.Cp * 2;
  ws.wr_offset = (ws.xc_bytes + 255) / 256 * 256;
  ws.wr_bytes = Cout * kh * kw * ws.Cp * 2;
  ws.total = ws.wr_offset + ws.wr_bytes;
  return ws;
}

constexpr int32_t kMaxSplits = 256;

// K ranges of a split-K launch: at most `splits` ranges of equal length in
// whole K steps of bk (the last one holds the rest); fewer when K is short.
struct SplitK {
  int32_t n;        // ranges actually launched (1: no split)
  int32_t k_split;  // K elements per range
};
SplitK split_k(int64_t K, int32_t splits, int32_t bk) {
  if (splits <= 1 || K == 0) return SplitK{1, int32_t(K)};
  const int64_t per = (K + splits - 1) / splits;
  const int64_t ks = (per + bk - 1) / bk * bk;
  const int64_t n = (K + ks - 1) / ks;
  return n <= 1 ? SplitK{1, int32_t(K)} : SplitK{int32_t(n), int32_t(ks)};
}

// tss_gemm, tss_gemm_splitk: splits == 1 is the one-pass GEMM (no workspace).
int32_t gemm_impl(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B, void *C,
                  int64_t batch, int32_t out_dtype, const tss_tile_config *cfg, int32_t splits, void *workspace,
                  int64_t workspace_bytes, void *stream) {
  if (batch < 1 || M < 0 || N < 0 || K < 0) return TSS_E_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || batch > INT32_MAX) return TSS_E_ARG;
  if (dtype != TSS_F16 && dtype != TSS_BF16) return TSS_E_DTYPE;
  if (out_dtype != TSS_F32 && out_dtype != dtype) return TSS_E_DTYPE;
  if (K % 8 || N % 8) return TSS_E_ALIGN;
  if (M * K * 2 >= kTwoGiB || K * N * 2 >= kTwoGiB) return TSS_E_ARG;
  if (M == 0 || N == 0) return TSS_OK;
  if (!C || (K > 0 && (!A || !B))) return TSS_E_ARG;  // with K == 0, A and B are never read
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return TSS_E_ALIGN;
  tss_tile_config c{};
  if (splits == 0) {
    // the split-K plan: its split count, and its tile unless one is given
    int32_t st = planned_split(false, batch, M, N, K, &c, &splits);
    if (st != TSS_OK) return st;
  }
  if (cfg) {
    c = *cfg;
    int32_t st = check_config(c);
    if (st != TSS_OK) return st;
  } else if (c.bm == 0) {
    // the tile plan of the problem each K range is: batch * splits GEMMs of
    // M x N x ceil(K / splits) (the one-pass plan for splits == 1)
    int32_t st = planned_config(false, batch * splits, M, N, (K + splits - 1) / splits, &c);
    if (st != TSS_OK) return st;
  }
  const KernelEntry *e = find_kernel(c, dtype, 0);
  if (!e) return TSS_E_UNSUPPORTED;
  const SplitK sk = split_k(K, splits, c.bk);
  if (sk.n > 1) {
    // every range's fp32 partial output in the workspace, then the reduction
    const unsigned __int128 need = (unsigned __int128)sk.n * uint64_t(batch) * uint64_t(M) * uint64_t(N) * 4u;
    if (!workspace || (unsigned __int128)workspace_bytes < need) return TSS_E_ARG;
    if (!aligned16(workspace)) return TSS_E_ALIGN;
  }
  KernelArgs a{};
  a.A = A;
  a.B = B;
  a.C = sk.n > 1 ? workspace : C;
  a.M = int32_t(M);
  a.N = int32_t(N);
  a.K = int32_t(K);
  a.lda = int32_t(K);
  a.splits = sk.n;
  a.k_split = sk.k_split;
  a.tiles_m = int32_t((M + c.bm - 1) / c.bm);
  a.tiles_n = int32_t((N + c.bn - 1) / c.bn);
  a.group_m = group_m_for(a.tiles_m);
  a.out_dtype = sk.n > 1 ? TSS_F32 : out_dtype;
  a.batch_stride_a = M * K;
  a.batch_stride_b = K * N;
  a.batch_stride_c = M * N;
  const int64_t blocks = batch * sk.n * a.tiles_m * a.tiles_n;
  if (blocks * c.threads > int64_t(UINT32_MAX) || blocks > INT32_MAX) return TSS_E_ARG;
  hipError_t err = e->launch(a, dim3(uint32_t(blocks)), e->lds_bytes, (hipStream_t)stream);
  if (err == hipSuccess && sk.n > 1)
    err = launch_splitk_reduce(static_cast<const float *>(workspace), C, out_dtype, batch, M * N, sk.n,
                               (hipStream_t)stream);
  return err == hipSuccess ? TSS_OK : TSS_E_HIP;
}

}  // namespace

extern "C" {

int32_t tss_device_query(int32_t hip_device, tss_device *out) {
  if (!out) return TSS_E_ARG;
  hipDeviceProp_t pr;
  if (hipGetDeviceProperties(&pr, hip_device) != hipSuccess) return TSS_E_HIP;
  if (std::strncmp(pr.gcnArchName, "gfx950", 6) != 0) return TSS_E_UNSUPPORTED;
  tss_device d{};
  tss_device_gfx950(&d);  // the model with its ranking's cost parameters
  d.cores = pr.multiProcessorCount;
  d.onchip_per_core = int32_t(pr.maxSharedMemoryPerMultiProcessor);
  d.onchip_per_block_max = int32_t(pr.sharedMemPerBlock);
  d.max_threads_per_core = pr.maxThreadsPerMultiProcessor;
  d.max_threads_per_block = pr.maxThreadsPerBlock;
  if (pr.maxBlocksPerMultiProcessor > 0) d.max_blocks_per_core = pr.maxBlocksPerMultiProcessor;
  *out = d;
  return TSS_OK;
}

int32_t tss_kernel_available(const tss_tile_config *cfg, int32_t dtype, int32_t op) {
  if (!cfg || (op != 0 && op != 1)) return 0;
  return find_kernel(*cfg, dtype, op) ? 1 : 0;
}

int32_t tss_kernel_usage_query(const tss_tile_config *cfg, int32_t dtype, int32_t op, tss_kernel_usage *out) {
  if (!cfg || !out || (op != 0 && op != 1)) return TSS_E_ARG;
  const KernelEntry *e = find_kernel(*cfg, dtype, op);
  if (!e) return TSS_E_UNSUPPORTED;
  hipFuncAttributes attr{};
  int blocks = 0;
  if (e->usage(&attr, &blocks, e->lds_bytes) != hipSuccess) return TSS_E_HIP;
  tss_kernel_usage u{};
  u.regs_per_lane = attr.numRegs;
  u.lds_bytes = int32_t(attr.sharedSizeBytes) + e->lds_bytes;
  u.scratch_bytes = int32_t(attr.localSizeBytes);
  u.max_threads = attr.maxThreadsPerBlock;
  u.blocks_per_cu = blocks;
  *out = u;
  return TSS_OK;
}

int32_t tss_tile_plan_measured(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t op,
                               tss_verdict *best, tss_verdict *list, int32_t cap, int32_t *n_feasible) {
  if (op != 0 && op != 1) return TSS_E_ARG;
  if (dtype != TSS_F16 && dtype != TSS_BF16) return TSS_E_DTYPE;
  // the registers of every compiled kernel of (dtype, op), read once
  static std::mutex mu;
  static std::map<std::pair<int32_t, int32_t>, std::vector<tss_measured_usage>> tables;
  std::vector<tss_measured_usage> table;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = tables.find({dtype, op});
    if (it != tables.end()) table = it->second;
  }
  if (table.empty()) {
    for (const auto &kv : registry()) {
      const KernelEntry &e = kv.second;
      if (e.dtype != dtype || e.op != op) continue;
      tss_tile_config c{e.bm, e.bn, e.bk, e.stages, e.threads, e.instr};
      tss_kernel_usage u{};
      int32_t st = tss_kernel_usage_query(&c, dtype, op, &u);
      if (st != TSS_OK) return st;
      table.push_back(tss_measured_usage{c, u.regs_per_lane, u.scratch_bytes});
    }
    std::lock_guard<std::mutex> g(mu);
    tables[{dtype, op}] = table;
  }
  return tss_tile_plan_usage(batch, M, N, K, 2, table.data(), int32_t(table.size()), best, list, cap, n_feasible);
}

int32_t tss_gemm_default_config(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t dtype,
                                tss_tile_config *out) {
  if (!out || batch < 1 || M < 0 || N < 0 || K < 0) return TSS_E_ARG;
  if (dtype != TSS_F16 && dtype != TSS_BF16) return TSS_E_DTYPE;
  return planned_config(false, batch, M, N, K, out);
}

int32_t tss_gemm(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B, void *C,
                 int64_t batch, int32_t out_dtype, const tss_tile_config *cfg, void *stream) {
  return gemm_impl(M, N, K, dtype, A, B, C, batch, out_dtype, cfg, 1, nullptr, 0, stream);
}

int64_t tss_gemm_splitk_workspace_size(int64_t batch, int64_t M, int64_t N, int32_t splits) {
  if (batch < 1 || M < 0 || N < 0 || splits < 1 || splits > kMaxSplits) return TSS_E_ARG;
  if (M > INT32_MAX || N > INT32_MAX || batch > INT32_MAX) return TSS_E_ARG;
  if (splits == 1) return 0;
  const unsigned __int128 bytes = (unsigned __int128)splits * uint64_t(batch) * uint64_t(M) * uint64_t(N) * 4u;
  if (bytes > (unsigned __int128)INT64_MAX) return TSS_E_ARG;
  return int64_t(bytes);
}

int32_t tss_gemm_autotune(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B, void *C,
                          int64_t batch, int32_t out_dtype, int32_t topk, int32_t iters, void *stream,
                          tss_tile_config *best, float *best_us) {
  if (!best || topk < 1 || topk > 1024 || iters < 1 || iters > 100000) return TSS_E_ARG;
  std::vector<tss_verdict> list(static_cast<size_t>(topk));
  int32_t n = 0;
  int32_t st = tss_tile_plan(batch, M, N, K, 2, nullptr, 0, nullptr, list.data(), topk, &n);
  if (st != TSS_OK) return st;
  const int32_t cand = n < topk ? n : topk;
  hipStream_t s = (hipStream_t)stream;
  auto launch = [&](const tss_tile_config &c) {
    return gemm_impl(M, N, K, dtype, A, B, C, batch, out_dtype, &c, 1, nullptr, 0, stream);
  };
  st = launch(list[0].cfg);  // also every argument check, before any event exists
  if (st != TSS_OK) return st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return TSS_E_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return TSS_E_HIP;
  }
  // time `reps` launches of c on the stream: microseconds per launch, or < 0 on an error
  auto time_cfg = [&](const tss_tile_config &c, int32_t reps) -> float {
    if (hipEventRecord(e0, s) != hipSuccess) return -1.f;
    for (int32_t r = 0; r < reps; ++r)
      if (launch(c) != TSS_OK) return -1.f;
    float ms = 0.f;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      return -1.f;
    return ms * 1000.f / float(reps);
  };
  // bring the engine clock up first: the plan's first tile for at least 20 ms (at most 50 rounds)
  float spent = 0.f;
  for (int round = 0; round < 50 && spent < 20000.f; ++round) {
    const float us = time_cfg(list[0].cfg, 20);
    if (us < 0.f) {
      st = TSS_E_HIP;
      break;
    }
    spent += 20.f * us;
    if (us == 0.f) break;  // nothing launched (M or N is 0)
  }
  // two interleaved rounds over the candidates, each candidate's best round
  // (a drift of the clock or a slow round then favours no candidate)
  std::vector<float> t(size_t(cand), -1.f);
  for (int round = 0; round < 2 && st == TSS_OK; ++round)
    for (int32_t i = 0; i < cand; ++i) {
      if (launch(list[i].cfg) != TSS_OK) {  // one warm-up launch of this kernel
        st = TSS_E_HIP;
        break;
      }
      const float us = time_cfg(list[i].cfg, iters);
      if (us < 0.f) {
        st = TSS_E_HIP;
        break;
      }
      if (t[i] < 0.f || us < t[i]) t[i] = us;
    }
  float best_t = 0.f;
  int32_t best_i = -1;
  for (int32_t i = 0; st == TSS_OK && i < cand; ++i)
    if (best_i < 0 || t[i] < best_t) {  // the first of equal times: the better-ranked candidate
      best_t = t[i];
      best_i = i;
    }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != TSS_OK) return st;
  *best = list[best_i].cfg;
  if (best_us) *best_us = best_t;
  return TSS_OK;
}

int32_t tss_gemm_splitk(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B, void *C,
                        int64_t batch, int32_t out_dtype, const tss_tile_config *cfg, int32_t splits,
                        void *workspace, int64_t workspace_bytes, void *stream) {
  if (splits < 0 || splits > kMaxSplits || workspace_bytes < 0) return TSS_E_ARG;
  return gemm_impl(M, N, K, dtype, A, B, C, batch, out_dtype, cfg, splits, workspace, workspace_bytes, stream);
}

int64_t tss_conv2d_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                                  int64_t kw) {
  const int64_t lim = int64_t(1) << 30;
  if (N < 1 || C < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1) return TSS_E_ARG;
  if (N > lim || C > lim || H > lim || W > lim || Cout > lim || kh > lim || kw > lim) return TSS_E_ARG;
  return conv_workspace(N, C, H, W, Cout, kh, kw, kConvChannelAlignMax).total;
}

}  // extern "C"

// Consecutive NCHW calls whose workspace holds two sets of operand copies
// alternate between them: the layout pass then writes the set the previous
// call's GEMM did not read (rewriting lines a kernel has just read made the
// pass ~40% slower on MI355X).  Any order of calls is correct; the counter only
// picks the set.
static std::atomic<uint32_t> g_layout_flip{0};

// tss_conv2d_tiled, tss_conv2d_splitk, tss_conv2d_nhwc: splits == 1 is the
// one-pass implicit GEMM.  NCHW (nhwc false): the workspace holds the operand
// layout copies (sized for any tile; a second set at the next 256-byte
// boundary when the workspace has room for both and the partial outputs),
// then at a 256-byte boundary the K ranges' fp32 partial outputs.  NHWC (nhwc true): x is [N][H][W][C], w is
// [Cout][kh][kw][C] and y is [N][OH][OW][Cout]; the implicit GEMM reads x and
// w in place (C a multiple of 8; the channels past C up to the K step's
// multiple read as zero) and the workspace holds only the partial outputs.
static int32_t conv_impl(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw,
                         int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t tile_n,
                         int64_t tile_oh, int64_t tile_ow, int32_t dtype, int32_t out_dtype, const void *x,
                         const void *w, void *y, int32_t splits, void *workspace, int64_t workspace_bytes,
                         const tss_tile_config *cfg, void *stream, bool nhwc = false) {
  const int64_t lim = int64_t(1) << 30;
  if (splits < 0 || splits > kMaxSplits) return TSS_E_ARG;
  if (N < 1 || C < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 || sh < 1 || sw < 1 || ph < 0 || pw < 0 ||
      dh < 1 || dw < 1)
    return TSS_E_ARG;
  if (N > lim || C > lim || H > lim || W > lim || Cout > lim || kh > lim || kw > lim || sh > lim || sw > lim ||
      ph > lim || pw > lim || dh > lim || dw > lim)
    return TSS_E_ARG;
  if (dtype != TSS_F16 && dtype != TSS_BF16) return TSS_E_DTYPE;
  if (out_dtype != TSS_F32 && out_dtype != dtype) return TSS_E_DTYPE;
  const int64_t OH = (H + 2 * ph - (kh - 1) * dh - 1) / sh + 1;
  const int64_t OW = (W + 2 * pw - (kw - 1) * dw - 1) / sw + 1;
  if (H + 2 * ph < (kh - 1) * dh + 1 || W + 2 * pw < (kw - 1) * dw + 1) return TSS_E_ARG;
  if (tile_oh < 1 || tile_oh > OH || tile_ow < 1 || tile_ow > OW || tile_n < 1 || tile_n > N) return TSS_E_ARG;
  if (nhwc && C % 8 != 0) return TSS_E_ARG;  // 16-byte pixels in place
  // sizes with the largest channel padding any tile can ask for (NHWC: none)
  const ConvWorkspace wmax = conv_workspace(N, C, H, W, Cout, kh, kw, nhwc ? 1 : kConvChannelAlignMax);
  // every operand, and both layout copies, addressable with 32-bit byte offsets
  if (N * C * H * W * 2 >= kTwoGiB || Cout * C * kh * kw * 2 >= kTwoGiB || wmax.xc_bytes >= kTwoGiB ||
      wmax.wr_bytes >= kTwoGiB || kh * kw * wmax.Cp > INT32_MAX)
    return TSS_E_ARG;
  const int64_t out_bytes = out_dtype == TSS_F32 ? 4 : 2;
  if (N * Cout * OH * OW * out_bytes >= (int64_t(1) << 40)) return TSS_E_ARG;
  const int64_t tile_pixels = tile_n * tile_oh * tile_ow;
  if (tile_pixels > INT32_MAX) return TSS_E_ARG;
  const int64_t layout_bytes = nhwc ? 0 : wmax.total;  // the operand copies in the workspace
  if (!x || !w || !y) return TSS_E_ARG;
  if (layout_bytes > 0 && (!workspace || workspace_bytes < layout_bytes)) return TSS_E_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (workspace && !aligned16(workspace))) return TSS_E_ALIGN;
  tss_tile_config c{};
  if (splits == 0) {
    // the split-K plan: its split count, and its tile unless one is given
    int32_t st = planned_split(true, Cout, N * OH * OW, C, kh * kw, &c, &splits);
    if (st != TSS_OK) return st;
  }
  if (cfg) {
    c = *cfg;
    int32_t st = check_config(c);
    if (st != TSS_OK) return st;
  } else if (c.bm == 0 && splits == 1) {
    // The implicit GEMM: M = Cout, N = every output pixel, K = kh*kw*C with
    // the channels padded to the candidate's K step (tss_conv_plan).
    int32_t st = planned_config(true, Cout, N * OH * OW, C, kh * kw, &c);
    if (st != TSS_OK) return st;
  } else if (c.bm == 0) {
    // the tile plan of the problem each of the `splits` K ranges is
    tss_verdict v{};
    int32_t S = splits;
    int32_t st = tss_conv_splitk_plan(Cout, N * OH * OW, C, kh * kw, 2, nullptr, &v, &S);
    if (st != TSS_OK) return st;
    c = v.cfg;
  }
  const KernelEntry *e = find_kernel(c, dtype, 1);
  if (!e) return TSS_E_UNSUPPORTED;
  const ConvWorkspace ws = conv_workspace(N, C, H, W, Cout, kh, kw, c.bk);
  const int64_t Kc = kh * kw * ws.Cp;       // K of the implicit GEMM, over (r, s, ci), ci padded to Cp
  const int64_t Cs = nhwc ? C : ws.Cp;      // channels per pixel (and per tap of a weight row) in memory
  const SplitK sk = split_k(Kc, splits, c.bk);
  const int64_t out_elems = N * Cout * OH * OW;
  const int64_t set_bytes = (layout_bytes + 255) / 256 * 256;  // one set of operand copies
  const unsigned __int128 part_bytes = sk.n > 1 ? (unsigned __int128)sk.n * uint64_t(out_elems) * 4u : 0;
  const bool two_sets = layout_bytes > 0 && (unsigned __int128)workspace_bytes >= 2 * (unsigned __int128)set_bytes + part_bytes;
  const int64_t part_offset = two_sets ? 2 * set_bytes : set_bytes;
  if (sk.n > 1 && (!workspace || (unsigned __int128)workspace_bytes < (unsigned __int128)part_offset + part_bytes))
    return TSS_E_ARG;
  float *partials = sk.n > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + part_offset) : nullptr;

  hipError_t err = hipSuccess;
  const void *opA = w, *opB = x;
  if (!nhwc) {
    // 1. operands in (r, s, ci) order: channel-last input, reordered weights
    char *set = static_cast<char *>(workspace);
    if (two_sets && (g_layout_flip.fetch_add(1, std::memory_order_relaxed) & 1u)) set += set_bytes;
    uint16_t *xc = reinterpret_cast<uint16_t *>(set);
    uint16_t *wr = reinterpret_cast<uint16_t *>(set + ws.wr_offset);
    LayoutArgs la{};
    la.x = static_cast<const uint16_t *>(x);
    la.xc = xc;
    la.w = static_cast<const uint16_t *>(w);
    la.wr = wr;
    la.N = int32_t(N);
    la.C = int32_t(C);
    la.HW = int32_t(H * W);
    la.Cp = int32_t(ws.Cp);
    la.Cout = int32_t(Cout);
    la.KHW = int32_t(kh * kw);
    la.c_tiles = int32_t((ws.Cp + 63) / 64);
    la.p_tiles = int32_t((H * W + 63) / 64);
    const int64_t x_blocks = N * la.c_tiles * la.p_tiles;
    const int64_t w_blocks = Cout;  // one block per output channel
    if (x_blocks + w_blocks > int64_t(INT32_MAX)) return TSS_E_ARG;
    hipLaunchKernelGGL(conv_layout_kernel, dim3(uint32_t(w_blocks + x_blocks)), dim3(kLayoutThreads), 0,
                       (hipStream_t)stream, la);
    err = hipGetLastError();
    if (err != hipSuccess) return TSS_E_HIP;
    opA = wr;
    opB = xc;
  }

  // 2. the implicit GEMM over the tiles
  KernelArgs a{};
  a.A = opA;
  a.B = opB;
  a.y_nhwc = nhwc ? 1 : 0;
  a.C = sk.n > 1 ? static_cast<void *>(partials) : y;
  a.M = int32_t(Cout);
  a.N = int32_t(tile_pixels);
  a.K = int32_t(Kc);
  a.lda = int32_t(kh * kw * Cs);  // a weight row in memory
  a.splits = sk.n;
  a.k_split = sk.k_split;
  a.batch_stride_c = out_elems;  // between the K ranges' partial outputs
  a.tiles_m = int32_t((Cout + c.bm - 1) / c.bm);
  a.tiles_n = int32_t((tile_pixels + c.bn - 1) / c.bn);
  a.group_m = group_m_for(a.tiles_m);
  a.out_dtype = sk.n > 1 ? TSS_F32 : out_dtype;
  a.Nb = int32_t(N);
  a.Cin = int32_t(C);
  a.H = int32_t(H);
  a.W = int32_t(W);
  a.kh = int32_t(kh);
  a.kw = int32_t(kw);
  a.sh = int32_t(sh);
  a.sw = int32_t(sw);
  a.ph = int32_t(ph);
  a.pw = int32_t(pw);
  a.dh = int32_t(dh);
  a.dw = int32_t(dw);
  a.OH = int32_t(OH);
  a.OW = int32_t(OW);
  a.tile_oh = int32_t(tile_oh);
  a.Cp = int32_t(ws.Cp);
  a.Cs = int32_t(Cs);
  a.tile_ow = int32_t(tile_ow);
  a.tile_n = int32_t(tile_n);
  a.n_ht = int32_t((OH + tile_oh - 1) / tile_oh);
  a.n_wt = int32_t((OW + tile_ow - 1) / tile_ow);
  const int64_t n_tiles = (N + tile_n - 1) / tile_n * a.n_ht * a.n_wt;
  const int64_t blocks = n_tiles * sk.n * a.tiles_m * a.tiles_n;
  if (blocks * c.threads > int64_t(UINT32_MAX) || blocks > INT32_MAX) return TSS_E_ARG;
  err = e->launch(a, dim3(uint32_t(blocks)), e->lds_bytes, (hipStream_t)stream);
  if (err == hipSuccess && sk.n > 1)
    err = launch_splitk_reduce(partials, y, out_dtype, 1, out_elems, sk.n, (hipStream_t)stream);
  return err == hipSuccess ? TSS_OK : TSS_E_HIP;
}

extern "C" {

int32_t tss_conv2d_tiled(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw,
                         int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t tile_n,
                         int64_t tile_oh, int64_t tile_ow, int32_t dtype, int32_t out_dtype, const void *x,
                         const void *w, void *y, void *workspace, int64_t workspace_bytes,
                         const tss_tile_config *cfg, void *stream) {
  return conv_impl(N, C, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, tile_n, tile_oh, tile_ow, dtype, out_dtype, x,
                   w, y, 1, workspace, workspace_bytes, cfg, stream);
}

int64_t tss_conv2d_splitk_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                                         int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                                         int64_t dw, int32_t splits) {
  const int64_t base = tss_conv2d_workspace_size(N, C, H, W, Cout, kh, kw);
  if (base < 0) return base;
  const int64_t lim = int64_t(1) << 30;
  if (sh < 1 || sw < 1 || ph < 0 || pw < 0 || dh < 1 || dw < 1 || sh > lim || sw > lim || ph > lim || pw > lim ||
      dh > lim || dw > lim || splits < 1 || splits > kMaxSplits)
    return TSS_E_ARG;
  if (H + 2 * ph < (kh - 1) * dh + 1 || W + 2 * pw < (kw - 1) * dw + 1) return TSS_E_ARG;
  if (splits == 1) return base;
  const int64_t OH = (H + 2 * ph - (kh - 1) * dh - 1) / sh + 1;
  const int64_t OW = (W + 2 * pw - (kw - 1) * dw - 1) / sw + 1;
  const unsigned __int128 bytes = (unsigned __int128)((base + 255) / 256 * 256) +
                                  (unsigned __int128)splits * uint64_t(N) * uint64_t(Cout) * uint64_t(OH) *
                                      uint64_t(OW) * 4u;
  if (bytes > (unsigned __int128)INT64_MAX) return TSS_E_ARG;
  return int64_t(bytes);
}

int32_t tss_conv2d_splitk(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw,
                          int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t tile_n,
                          int64_t tile_oh, int64_t tile_ow, int32_t dtype, int32_t out_dtype, const void *x,
                          const void *w, void *y, int32_t splits, void *workspace, int64_t workspace_bytes,
                          const tss_tile_config *cfg, void *stream) {
  return conv_impl(N, C, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, tile_n, tile_oh, tile_ow, dtype, out_dtype, x,
                   w, y, splits, workspace, workspace_bytes, cfg, stream);
}

int32_t tss_conv2d_nhwc(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw, int64_t sh,
                        int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t tile_n, int64_t tile_oh,
                        int64_t tile_ow, int32_t dtype, int32_t out_dtype, const void *x, const void *w, void *y,
                        int32_t splits, void *workspace, int64_t workspace_bytes, const tss_tile_config *cfg,
                        void *stream) {
  return conv_impl(N, C, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, tile_n, tile_oh, tile_ow, dtype, out_dtype, x,
                   w, y, splits, workspace, workspace_bytes, cfg, stream, true);
}

int64_t tss_conv2d_nhwc_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                                       int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                                       int64_t dw, int32_t splits) {
  const int64_t lim = int64_t(1) << 30;
  if (N < 1 || C < 1 || H < 1 || W < 1 || Cout < 1 || kh < 1 || kw < 1 || sh < 1 || sw < 1 || ph < 0 || pw < 0 ||
      dh < 1 || dw < 1 || splits < 1 || splits > kMaxSplits)
    return TSS_E_ARG;
  if (N > lim || C > lim || H > lim || W > lim || Cout > lim || kh > lim || kw > lim || sh > lim || sw > lim ||
      ph > lim || pw > lim || dh > lim || dw > lim)
    return TSS_E_ARG;
  if (H + 2 * ph < (kh - 1) * dh + 1 || W + 2 * pw < (kw - 1) * dw + 1) return TSS_E_ARG;
  if (splits == 1) return 0;
  const int64_t OH = (H + 2 * ph - (kh - 1) * dh - 1) / sh + 1;
  const int64_t OW = (W + 2 * pw - (kw - 1) * dw - 1) / sw + 1;
  const unsigned __int128 bytes =
      (unsigned __int128)splits * uint64_t(N) * uint64_t(Cout) * uint64_t(OH) * uint64_t(OW) * 4u;
  if (bytes > (unsigned __int128)INT64_MAX) return TSS_E_ARG;
  return int64_t(bytes);
}

int32_t tss_conv2d(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw, int64_t sh,
                   int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t tile_oh, int32_t dtype,
                   int32_t out_dtype, const void *x, const void *w, void *y, void *workspace,
                   int64_t workspace_bytes, const tss_tile_config *cfg, void *stream) {
  // H-tiles only: every tile spans the whole batch and the whole output width
  const int64_t lim = int64_t(1) << 30;
  if (N < 1 || W < 1 || kw < 1 || sw < 1 || pw < 0 || dw < 1) return TSS_E_ARG;
  if (N > lim || W > lim || kw > lim || sw > lim || pw > lim || dw > lim) return TSS_E_ARG;
  if (W + 2 * pw < (kw - 1) * dw + 1) return TSS_E_ARG;
  const int64_t OW = (W + 2 * pw - (kw - 1) * dw - 1) / sw + 1;
  return tss_conv2d_tiled(N, C, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, N, tile_oh, OW, dtype, out_dtype, x, w,
                          y, workspace, workspace_bytes, cfg, stream);
}

}  // extern "C"
