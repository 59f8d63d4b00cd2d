// Tile planner: constraints C0..C4 evaluated on a device description, and the
// ranked sweep over candidate tiles.  Header-only and constexpr so that the
// same code decides at compile time which GEMM kernels get instantiated and
// at run time which one a problem gets.
//
// Constraint definitions: "tile_decision.py" page (tilelang tutorial ch. 28
// sec. 4) -- C3 instruction shape (checked first), C1 on-chip capacity
// stages*(BM*BK + BK*BN)*elem_bytes, C2 accumulator registers per thread
// rounded to the allocation granule, occupancy from registers / on-chip memory
// / threads, C4 waves of tiles and last-wave fill; C0 DRAM traffic
// b*M*N*K*(1/BN + 1/BM) + b*M*N from the "04-tile-size-decision/README.md"
// page (b = bytes per element).  The gfx950 register model adds the fixed
// per-thread overhead of the "Tiling（分块）" page's register example and
// works per SIMD; its ranking follows that page's rules of thumb (spare
// on-chip memory goes to a larger BK or a deeper pipeline).
#pragma once
#include <stdint.h>

#include "../../include/tss.h"

namespace tss {

struct Shape {
  int32_t m, n, k, threads;
};

constexpr bool instr_shape(int32_t instr, Shape &s) {
  switch (instr) {
    case TSS_INSTR_MFMA32: s = {32, 32, 16, 64}; return true;
    case TSS_INSTR_MFMA16: s = {16, 16, 32, 64}; return true;
    case TSS_INSTR_NV_MMA: s = {16, 8, 16, 32}; return true;
    case TSS_INSTR_NV_WGMMA: s = {64, 8, 16, 128}; return true;
    case TSS_INSTR_NV_SIMT: s = {1, 1, 1, 32}; return true;
    default: return false;
  }
}

constexpr bool instr_on_device(int32_t instr, const tss_device &d) {
  bool amd = d.lane_count == 64;
  return amd ? (instr == TSS_INSTR_MFMA32 || instr == TSS_INSTR_MFMA16)
             : (instr == TSS_INSTR_NV_MMA || instr == TSS_INSTR_NV_WGMMA || instr == TSS_INSTR_NV_SIMT);
}

// rows x cols of waves for a block of `waves` waves; false if not supported
constexpr bool wave_grid(int32_t waves, int32_t &wm, int32_t &wn) {
  switch (waves) {
    case 1: wm = 1; wn = 1; return true;
    case 2: wm = 1; wn = 2; return true;
    case 4: wm = 2; wn = 2; return true;
    case 8: wm = 2; wn = 4; return true;
    case 16: wm = 4; wn = 4; return true;
    default: return false;
  }
}

constexpr tss_device gfx950_device() {
  tss_device d{};
  d.cores = 256;
  d.onchip_per_core = 163840;
  d.onchip_per_block_max = 163840;
  d.max_threads_per_core = 2048;
  d.max_threads_per_block = 1024;
  d.max_blocks_per_core = 32;
  d.lane_count = 64;
  d.reg_granule_per_lane = 8;
  d.acc_regs_max = 256;
  d.reg_overhead = 32;
  d.reg_model = TSS_REG_PER_SIMD;
  d.regs_per_core = 0;
  d.simds_per_core = 4;
  d.regs_per_lane_per_simd = 512;
  d.max_waves_per_simd = 8;
  d.wave_grid_rule = 1;
  d.load_bytes_per_lane = 16;
  d.ranking = TSS_RANK_GFX950;
  // the ranking's cost parameters are set by gfx950_costs (planner.cpp):
  // they rank candidates, they never decide which kernels exist
  return d;
}

constexpr tss_device pages_device(int32_t sm_count, int32_t smem_kb) {
  tss_device d{};
  d.cores = sm_count;
  d.onchip_per_core = smem_kb * 1024;
  d.onchip_per_block_max = smem_kb * 1024 - 1024;
  d.max_threads_per_core = 2048;
  d.max_threads_per_block = 1024;
  d.max_blocks_per_core = 32;
  d.lane_count = 32;
  d.reg_granule_per_lane = 256 / 32;  // 256 registers per warp of 32
  d.acc_regs_max = 255;
  d.reg_overhead = 0;
  d.reg_model = TSS_REG_POOLED;
  d.regs_per_core = 65536;
  d.ranking = TSS_RANK_PAGES;
  d.step_cost_k = 0;
  d.tile_cost_k = 0;
  d.split_byte_cost = 0;
  d.launch_cost_k = 0;
  d.target_waves_per_simd = 0;
  return d;
}

constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// C3 + C1 + C2 + occupancy: the parts that do not depend on the problem.
// regs_measured > 0: the registers per lane of the compiled kernel, which then
// replace the model's estimate for occupancy (rounded up to the allocation
// granule); scratch_measured > 0: the compiled kernel spills that many bytes
// per lane, which fails C2 whatever the accumulator count says.
constexpr tss_verdict evaluate_block(const tss_tile_config &c, const tss_device &d, int32_t eb,
                                     int64_t regs_measured = 0, int64_t scratch_measured = 0) {
  tss_verdict v{};
  v.cfg = c;
  Shape s{};
  instr_shape(c.instr, s);
  // C3: whole intrinsic tiles, whole issuing groups, block size cap
  if (c.bm % s.m) v.failures |= TSS_FAIL_C3_M;
  if (c.bn % s.n) v.failures |= TSS_FAIL_C3_N;
  if (c.bk % s.k) v.failures |= TSS_FAIL_C3_K;
  if (c.threads % s.threads) v.failures |= TSS_FAIL_C3_THREADS;
  if (c.threads > d.max_threads_per_block) v.failures |= TSS_FAIL_C3_MAXTHREADS;
  if (d.wave_grid_rule) {
    int32_t wm = 0, wn = 0;
    bool ok = c.threads % d.lane_count == 0 && wave_grid(c.threads / d.lane_count, wm, wn);
    if (!ok || c.bm % (wm * s.m) || c.bn % (wn * s.n)) v.failures |= TSS_FAIL_C3_WAVEGRID;
  }
  if (d.load_bytes_per_lane) {
    int64_t waves = c.threads / d.lane_count;
    if (waves < 1) waves = 1;
    int64_t unit = int64_t(d.load_bytes_per_lane) * d.lane_count * waves;
    if ((int64_t(c.bm) * c.bk * eb) % unit || (int64_t(c.bk) * c.bn * eb) % unit)
      v.failures |= TSS_FAIL_C3_LOAD;
  }
  // C1: one A tile and one B tile per pipeline stage
  v.smem_per_stage = (int64_t(c.bm) * c.bk + int64_t(c.bk) * c.bn) * eb;
  v.smem_total = v.smem_per_stage * c.stages;
  if (v.smem_total > d.onchip_per_block_max) v.failures |= TSS_FAIL_C1;
  // C2: fp32 accumulators per thread, allocation granule, fixed overhead
  v.accum_per_thread = cdiv(int64_t(c.bm) * c.bn, c.threads);
  int64_t raw = v.accum_per_thread * 4 / 4;
  int64_t acc_regs = cdiv(raw, d.reg_granule_per_lane) * d.reg_granule_per_lane;
  v.regs_per_thread = acc_regs + d.reg_overhead;
  if (regs_measured > 0) v.regs_per_thread = cdiv(regs_measured, d.reg_granule_per_lane) * d.reg_granule_per_lane;
  if (acc_regs > d.acc_regs_max || scratch_measured > 0) v.failures |= TSS_FAIL_C2;
  v.regs_per_block = v.regs_per_thread * c.threads;
  // occupancy
  if (d.reg_model == TSS_REG_POOLED) {
    v.blocks_by_regs = d.regs_per_core / (v.regs_per_block > 0 ? v.regs_per_block : 1);
  } else {
    int64_t wps = d.regs_per_lane_per_simd / v.regs_per_thread;
    if (wps > d.max_waves_per_simd) wps = d.max_waves_per_simd;
    int64_t wpb = cdiv(c.threads, d.lane_count);
    v.blocks_by_regs = (d.simds_per_core * wps) / (wpb > 0 ? wpb : 1);
  }
  v.blocks_by_smem = d.onchip_per_core / (v.smem_total > 0 ? v.smem_total : 1);
  v.blocks_by_threads = d.max_threads_per_core / (c.threads > 0 ? c.threads : 1);
  int64_t b = v.blocks_by_regs;
  if (v.blocks_by_smem < b) b = v.blocks_by_smem;
  if (v.blocks_by_threads < b) b = v.blocks_by_threads;
  if (d.max_blocks_per_core < b) b = d.max_blocks_per_core;
  v.blocks_per_core = b > 0 ? b : 0;
  if (v.blocks_per_core == 0) {
    v.failures |= TSS_FAIL_OCC0;
    v.binding = TSS_BIND_NONE;
  } else {
    int64_t least = v.blocks_by_regs;
    if (v.blocks_by_smem < least) least = v.blocks_by_smem;
    if (v.blocks_by_threads < least) least = v.blocks_by_threads;
    v.binding = v.blocks_by_regs == least ? TSS_BIND_REGS
                : v.blocks_by_smem == least ? TSS_BIND_SMEM : TSS_BIND_THREADS;
  }
  return v;
}

using u128 = unsigned __int128;

constexpr u128 gcd128(u128 a, u128 b) {
  while (b) {
    u128 t = a % b;
    a = b;
    b = t;
  }
  return a;
}

constexpr u128 round_half_even(u128 num, u128 den) {
  u128 q = num / den, r = num % den;
  if (2 * r > den || (2 * r == den && (q & 1))) q += 1;
  return q;
}

// C4 and C0 for one problem (the verdict must come from evaluate_block).
// The caller keeps batch * M * N <= 2^62 and K <= 2^40, so that the grid fits
// int64 and C0's numerator (below 2^62 * 8 * 2^40 * 2^10) fits 128 bits.
constexpr void finish(tss_verdict &v, const tss_device &d, int64_t batch, int64_t M, int64_t N,
                      int64_t K, int32_t eb) {
  const tss_tile_config &c = v.cfg;
  v.grid = batch * cdiv(M, c.bm) * cdiv(N, c.bn);
  int64_t resident = v.blocks_per_core * d.cores;
  if (resident < 1) resident = 1;
  v.waves = cdiv(v.grid, resident);
  int64_t rem = v.grid % resident;
  if (rem) {
    int64_t g = rem, h = resident;
    while (h) {
      int64_t t = g % h;
      g = h;
      h = t;
    }
    v.fill_num = rem / g;
    v.fill_den = resident / g;
  } else {
    v.fill_num = 1;
    v.fill_den = 1;
  }
  v.warnings = 0;
  if (v.waves > 1 && rem && 2 * rem < resident) v.warnings |= TSS_WARN_TAIL;
  if (v.grid < d.cores) v.warnings |= TSS_WARN_IDLE;
  // C0 = batch*eb*(M*N*K*(BM+BN) + M*N*BM*BN) / (BM*BN), in lowest terms
  u128 num = u128(batch) * u128(eb) *
             (u128(M) * u128(N) * u128(K) * u128(c.bm + c.bn) + u128(M) * u128(N) * u128(c.bm) * u128(c.bn));
  u128 den = u128(c.bm) * u128(c.bn);
  u128 g = num ? gcd128(num, den) : den;
  num /= g;
  den /= g;
  v.traffic_num_hi = uint64_t(num >> 64);
  v.traffic_num_lo = uint64_t(num);
  v.traffic_den = uint64_t(den);
  const u128 q = round_half_even(num, den);
  v.traffic_rounded = q > u128(UINT64_MAX) ? UINT64_MAX : uint64_t(q);  // saturated; exact in num / den
}

// C0 of a finished verdict, rounded half to even, without the saturation of
// traffic_rounded.
constexpr u128 traffic_rounded_exact(const tss_verdict &v) {
  const u128 num = (u128(v.traffic_num_hi) << 64) | u128(v.traffic_num_lo);
  return round_half_even(num, u128(v.traffic_den));
}

// ---- candidate space -------------------------------------------------------

struct Space {
  int32_t bm[5], nbm, bn[5], nbn, bk[4], nbk, stages[3], nst, threads[3], nthr, instr[3], ninstr;
};

constexpr Space space_for(const tss_device &d, int32_t instr_filter) {
  Space s{};
  if (d.ranking == TSS_RANK_PAGES) {
    int32_t sizes[5] = {16, 32, 64, 128, 256};
    for (int i = 0; i < 5; ++i) s.bm[i] = s.bn[i] = sizes[i];
    s.nbm = s.nbn = 5;
    int32_t ks[4] = {16, 32, 64, 128};
    for (int i = 0; i < 4; ++i) s.bk[i] = ks[i];
    s.nbk = 4;
    int32_t nv[3] = {TSS_INSTR_NV_MMA, TSS_INSTR_NV_SIMT, TSS_INSTR_NV_WGMMA};
    for (int i = 0; i < 3; ++i) s.instr[i] = nv[i];
    s.ninstr = 3;
  } else {
    // largest first: of two otherwise equal tiles the taller one comes first
    // (it copies fewer B chunks per FLOP; in the convolution those are the
    // copies that carry per-lane pad and slice tests)
    int32_t sizes[3] = {256, 128, 64};
    for (int i = 0; i < 3; ++i) s.bm[i] = s.bn[i] = sizes[i];
    s.nbm = s.nbn = 3;
    int32_t ks[3] = {16, 32, 64};
    for (int i = 0; i < 3; ++i) s.bk[i] = ks[i];
    s.nbk = 3;
    // 16x16x32 first: it wins ties, keeping the 16x16 output tile of the
    // MMA level of the Tiling page's multi-level tiling
    s.instr[0] = TSS_INSTR_MFMA16;
    s.instr[1] = TSS_INSTR_MFMA32;
    s.ninstr = 2;
  }
  if (instr_filter) {
    s.instr[0] = instr_filter;
    s.ninstr = 1;
  }
  s.stages[0] = 2; s.stages[1] = 3; s.stages[2] = 4; s.nst = 3;
  s.threads[0] = 128; s.threads[1] = 256; s.threads[2] = 512; s.nthr = 3;
  return s;
}

// Lexicographic rank key; smaller is preferred.  128-bit terms: the
// traffic and time terms of problems near the accepted bounds exceed 64 bits.
using i128 = __int128;
struct Key {
  i128 k[8];
};

// The gfx950 time term of a candidate whose K loop runs over K elements
// (K_loop: the GEMM's K, or the convolution's K with each tap's channels
// padded to whole K steps).  On the busiest CU, C4 deals out
// W = ceil(grid / CUs) tiles, at most u = min(blocks per CU, W) of them
// resident at once, so in R = ceil(W / u) rounds.  Each tile streams its
// C0 panels, (BM + BN) elements per K element (the README page's per-tile
// traffic), over n = ceil(K_loop / BK) K steps, each step costing
// BK + step_cost_k K elements; each round pays tile_cost_k more (prologue,
// epilogue, output write):
//   T = W * (BM + BN) * n * (BK + step_cost_k) + R * (BM + BN) * tile_cost_k.
// Every candidate's intensity 2*BM*BN / ((BM + BN) * b) (the Tiling page's
// tiled-intensity formula, at most 128 FLOP/B) is below MI355X's ridge
// (2516.6 TFLOP/s over 8 TB/s, about 315 FLOP/B), which is why panel
// traffic is the unit of time.
constexpr i128 busiest_core_time(const tss_verdict &v, const tss_device &d, int64_t K_loop) {
  const tss_tile_config &c = v.cfg;
  const int64_t W = cdiv(v.grid, d.cores);
  if (W == 0) return 0;
  const int64_t u = v.blocks_per_core < W ? v.blocks_per_core : W;
  const int64_t R = cdiv(W, u > 0 ? u : 1);
  const int64_t n = cdiv(K_loop, c.bk);
  const i128 panel = i128(c.bm + c.bn);
  return i128(W) * panel * i128(n) * i128(c.bk + d.step_cost_k) + i128(R) * panel * i128(d.tile_cost_k);
}

constexpr Key rank_key(const tss_verdict &v, const tss_device &d, int64_t K_loop) {
  Key r{};
  const i128 t = i128(traffic_rounded_exact(v));
  if (d.ranking == TSS_RANK_PAGES) {
    r.k[0] = t;
    r.k[1] = -v.blocks_per_core;
    r.k[2] = v.smem_total;
  } else {
    // the busiest CU's time (above); then total C0, larger BK, most resident
    // blocks; resident waves per SIMD closest to target_waves_per_simd (in
    // whole waves per CU: |u * waves - SIMDs * target|), then the most
    // resident waves; deeper pipeline, less LDS.  Residency counts only the
    // blocks the grid can supply: with ceil(grid / CUs) waves of tiles no CU
    // ever holds more than that many blocks at once, whatever its capacity.
    const int64_t W = cdiv(v.grid, d.cores);
    const int64_t usable = v.blocks_per_core < W ? v.blocks_per_core : W;
    const int64_t waves = usable * (v.cfg.threads / d.lane_count);
    const int64_t off = waves - int64_t(d.simds_per_core) * d.target_waves_per_simd;
    r.k[0] = busiest_core_time(v, d, K_loop);
    r.k[1] = t;
    r.k[2] = -v.cfg.bk;
    r.k[3] = -usable;
    r.k[4] = d.target_waves_per_simd > 0 ? (off < 0 ? -off : off) : 0;
    r.k[5] = -waves;
    r.k[6] = -v.cfg.stages;
    r.k[7] = v.smem_total;
  }
  return r;
}

// Split counts the split-K plan considers.
constexpr int32_t kSplitCandidates[] = {1, 2, 3, 4, 6, 8, 12, 16};

// Ranges a split of K into S parts of whole K steps of bk gives (the kernel's
// cut: ceil(K / S) rounded up to a multiple of bk per range).
constexpr int64_t split_ranges(int64_t K, int64_t S, int64_t bk) {
  if (K == 0 || S <= 1) return 1;
  const int64_t ks = cdiv(cdiv(K, S), bk) * bk;
  return cdiv(K, ks);
}

// The split-K plan's total for S ranges whose tile plan has busiest-CU time
// T_S, scaled by elem_bytes * cores to stay an integer:
//   (T_S + [S > 1] * (8 * S * batch * M * N * split_byte_cost / (eb * cores) + launch_cost_k)) * eb * cores
constexpr i128 split_total(i128 T_S, int64_t S, int64_t batch, int64_t M, int64_t N, int32_t eb,
                           const tss_device &d) {
  const i128 scale = i128(eb) * i128(d.cores);
  i128 t = T_S * scale;
  if (S > 1)
    t += i128(8) * i128(S) * i128(batch) * i128(M) * i128(N) * i128(d.split_byte_cost) +
         i128(d.launch_cost_k) * scale;
  return t;
}

constexpr bool key_less(const Key &a, const Key &b) {
  for (int i = 0; i < 8; ++i) {
    if (a.k[i] != b.k[i]) return a.k[i] < b.k[i];
  }
  return false;
}

// A configuration gets a compiled kernel exactly when it is feasible on the
// gfx950 model (C3, C1, C2 and occupancy pass); C4 and C0 only rank it.
constexpr bool kernel_needed(int32_t bm, int32_t bn, int32_t bk, int32_t stages, int32_t threads,
                             int32_t instr) {
  tss_device d = gfx950_device();
  tss_tile_config c{bm, bn, bk, stages, threads, instr};
  return evaluate_block(c, d, 2).failures == 0;
}

}  // namespace tss
