// C ABI of the tile planner (host only).  The arithmetic lives in planner.h.
#include <algorithm>
#include <vector>

#include "planner.h"

using namespace tss;

namespace {

// The gfx950 model with its ranking's cost parameters (include/tss.h,
// tss_device), properties of this library's kernels:
//  step_cost_k 22: with a fixed cost of 22 K elements per K step, the 32-
//    and 16-wide steps take 1.24x and 1.76x the 64-wide step's time per
//    FLOP at equal K (measured on the convolution workload);
//  tile_cost_k 900: the 4096^3 GEMM's prologue and epilogue take about
//    10 us of one round against 1.41 us per 64-wide K step (86 K elements
//    of cost), about 7 steps or 600 K elements; 900 is past 824, where the
//    K = 200 GEMM's 128x128 tiles (measured faster there) overtake the
//    256x256 tile;
//  target_waves_per_simd 4: among tiles equal in time, traffic, K step and
//    resident blocks, 256-thread blocks at 4 waves per SIMD ran 8-16%
//    faster than their 512-thread twins on K loops of 2 to 4 steps;
//  split_byte_cost 6, launch_cost_k 67000: the split-K plan's costs, with
//    which its split count measured within 5% of the fastest on nine GEMM
//    shapes (2 us of reduction launch at the rate the time term converts at).
tss_device gfx950_with_costs() {
  tss_device d = gfx950_device();
  d.step_cost_k = 22;
  d.tile_cost_k = 900;
  d.split_byte_cost = 6;
  d.launch_cost_k = 67000;
  d.target_waves_per_simd = 4;
  return d;
}

bool valid_device(const tss_device &d) {
  if (d.cores <= 0 || d.onchip_per_core <= 0 || d.onchip_per_block_max <= 0 || d.max_threads_per_core <= 0 ||
      d.max_threads_per_block <= 0 || d.max_blocks_per_core <= 0 || d.lane_count <= 0 ||
      d.reg_granule_per_lane <= 0 || d.acc_regs_max <= 0 || d.reg_overhead < 0 || d.step_cost_k < 0 ||
      d.tile_cost_k < 0 || d.split_byte_cost < 0 || d.launch_cost_k < 0 || d.target_waves_per_simd < 0)
    return false;
  if (d.reg_model == TSS_REG_POOLED) return d.regs_per_core > 0;
  if (d.reg_model == TSS_REG_PER_SIMD)
    return d.simds_per_core > 0 && d.regs_per_lane_per_simd > 0 && d.max_waves_per_simd > 0;
  return false;
}

bool valid_config(const tss_tile_config &c, const tss_device &d) {
  return c.bm > 0 && c.bn > 0 && c.bk > 0 && c.stages > 0 && c.threads > 0 && instr_on_device(c.instr, d);
}


// K of the problem for a candidate: a plain GEMM's K (the same for every
// candidate), or the implicit GEMM of a convolution whose channels the kernel
// pads to a multiple of the candidate's K step: taps * ceil(C / BK) * BK.
struct FixedK {
  int64_t K;
  int64_t operator()(int32_t) const { return K; }
};
struct ConvK {
  int64_t C, taps;
  int64_t operator()(int32_t bk) const { return taps * ((C + bk - 1) / bk) * bk; }
};
// One of S ranges of a K: ceil(K / S), with the convolution's K depending on BK.
template <typename KOf>
struct RangeK {
  KOf k_of;
  int64_t S;
  int64_t operator()(int32_t bk) const { return (k_of(bk) + S - 1) / S; }
};

constexpr int64_t kLim40 = int64_t(1) << 40;

// Sizes every planner entry point accepts: batch <= 2^20, M, N, K <= 2^40
// and batch * M * N <= 2^62, so that the grid fits 64 bits and C0's
// numerator 128 bits.
bool sizes_ok(int64_t batch, int64_t M, int64_t N, int64_t K) {
  if (batch < 1 || M < 0 || N < 0 || K < 0) return false;
  if (M > kLim40 || N > kLim40 || K > kLim40 || batch > (int64_t(1) << 20)) return false;
  const unsigned __int128 bmn = (unsigned __int128)batch * (unsigned __int128)M * (unsigned __int128)N;
  return bmn <= ((unsigned __int128)1 << 62);
}

// The shared sweep: every candidate of the device's space that passes
// C3/C1/C2/occupancy, finished for the problem with its own K (k_of) and
// ranked by rank_key.  usage_of (may be null) gives the compiled kernel's
// measured usage for a configuration (null to leave the candidate out).
template <typename UsageOf, typename KOf>
int32_t plan_sweep(int64_t batch, int64_t M, int64_t N, const KOf &k_of, int32_t elem_bytes, const tss_device &d,
                   int32_t instr_filter, const UsageOf *usage_of, tss_verdict *best, tss_verdict *list, int32_t cap,
                   int32_t *n_feasible) {
  const int64_t K = k_of(1);
  if (!sizes_ok(batch, M, N, K) || elem_bytes < 1 || elem_bytes > 8 || cap < 0) return TSS_E_ARG;
  if (!valid_device(d)) return TSS_E_ARG;
  if (instr_filter && !instr_on_device(instr_filter, d)) return TSS_E_ARG;
  const Space s = space_for(d, instr_filter);
  std::vector<tss_verdict> feas;
  std::vector<int64_t> feas_k;
  feas.reserve(512);
  feas_k.reserve(512);
  for (int ii = 0; ii < s.ninstr; ++ii) {
    Shape sh{};
    instr_shape(s.instr[ii], sh);
    for (int a = 0; a < s.nbm; ++a)
      for (int b = 0; b < s.nbn; ++b)
        for (int c = 0; c < s.nbk; ++c) {
          // A K step longer than K is skipped, unless K is shorter than every
          // candidate step: then the shortest one is kept (its tail is masked).
          const int64_t Kc = k_of(s.bk[c]);
          if (Kc > kLim40) return TSS_E_ARG;
          if (s.bk[c] > (Kc > s.bk[0] ? Kc : s.bk[0])) continue;
          for (int e = 0; e < s.nst; ++e)
            for (int f = 0; f < s.nthr; ++f) {
              if (s.threads[f] % sh.threads) continue;
              tss_tile_config cfg{s.bm[a], s.bn[b], s.bk[c], s.stages[e], s.threads[f], s.instr[ii]};
              int64_t regs = 0, scratch = 0;
              if (usage_of) {
                if (evaluate_block(cfg, d, elem_bytes).failures) continue;  // the model decides what exists
                const tss_measured_usage *u = (*usage_of)(cfg);
                if (!u) continue;
                regs = u->regs_per_lane;
                scratch = u->scratch_bytes;
              }
              tss_verdict v = evaluate_block(cfg, d, elem_bytes, regs, scratch);
              if (v.failures) continue;
              finish(v, d, batch, M, N, Kc, elem_bytes);
              feas.push_back(v);
              feas_k.push_back(Kc);
            }
        }
  }
  std::vector<int32_t> order(feas.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = int32_t(i);
  auto key_of = [&](int32_t i) { return rank_key(feas[i], d, feas_k[i]); };
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return key_less(key_of(x), key_of(y)); });
  if (n_feasible) *n_feasible = int32_t(feas.size());
  if (list)
    for (int32_t i = 0; i < cap && i < int32_t(feas.size()); ++i) list[i] = feas[order[i]];
  if (feas.empty()) return TSS_E_INFEASIBLE;
  if (best) *best = feas[order[0]];
  return TSS_OK;
}

struct NoUsage {
  const tss_measured_usage *operator()(const tss_tile_config &) const { return nullptr; }
};

// The split-K plan over kSplitCandidates (tss_splitk_plan): the tile plan of
// the split problem for each S, its busiest-CU time plus the split's costs.
template <typename KOf>
int32_t splitk_sweep(int64_t batch, int64_t M, int64_t N, const KOf &k_of, int32_t elem_bytes, const tss_device &d,
                     tss_verdict *best, int32_t *splits) {
  if (!splits || d.ranking != TSS_RANK_GFX950 || *splits < 0 || *splits > 256) return TSS_E_ARG;
  // *splits > 0: the tile plan for that many ranges only
  const int32_t fixed = *splits;
  bool found = false;
  i128 best_total = 0;
  tss_verdict best_v{};
  int32_t best_s = 0;
  const int32_t one[1] = {fixed};
  const int32_t *cands = fixed ? one : kSplitCandidates;
  const int ncand = fixed ? 1 : int(sizeof(kSplitCandidates) / sizeof(kSplitCandidates[0]));
  for (int ci = 0; ci < ncand; ++ci) {
    const int32_t S = cands[ci];
    if (batch * S > (int64_t(1) << 20)) {  // beyond the planner's batch bound
      if (fixed) return TSS_E_ARG;
      break;
    }
    tss_verdict v{};
    int32_t st = plan_sweep<NoUsage>(batch * S, M, N, RangeK<KOf>{k_of, S}, elem_bytes, d, 0, nullptr, &v, nullptr, 0,
                                     nullptr);
    if (st == TSS_E_INFEASIBLE) continue;
    if (st != TSS_OK) return st;
    if (!fixed && S > 1 && split_ranges(k_of(v.cfg.bk), S, v.cfg.bk) != S) continue;  // the kernel would cut fewer
    const i128 total =
        split_total(rank_key(v, d, RangeK<KOf>{k_of, S}(v.cfg.bk)).k[0], S, batch, M, N, elem_bytes, d);
    if (!found || total < best_total) {
      found = true;
      best_total = total;
      best_v = v;
      best_s = S;
    }
  }
  if (!found) return TSS_E_INFEASIBLE;
  if (best) *best = best_v;
  *splits = best_s;
  return TSS_OK;
}

}  // namespace

extern "C" {

int32_t tss_instr_shape(int32_t instr, int32_t out[4]) {
  Shape s{};
  if (!out || !instr_shape(instr, s)) return TSS_E_ARG;
  out[0] = s.m;
  out[1] = s.n;
  out[2] = s.k;
  out[3] = s.threads;
  return TSS_OK;
}

int32_t tss_device_gfx950(tss_device *out) {
  if (!out) return TSS_E_ARG;
  *out = gfx950_with_costs();
  return TSS_OK;
}

int32_t tss_device_pages(int32_t sm_count, int32_t smem_kb, tss_device *out) {
  if (!out || sm_count <= 0 || smem_kb <= 1 || smem_kb > (1 << 20)) return TSS_E_ARG;
  *out = pages_device(sm_count, smem_kb);
  return TSS_OK;
}

int32_t tss_evaluate(const tss_tile_config *cfg, const tss_device *dev, int64_t batch, int64_t M, int64_t N,
                     int64_t K, int32_t elem_bytes, tss_verdict *out) {
  const tss_device d = dev ? *dev : gfx950_with_costs();
  if (!cfg || !out || !sizes_ok(batch, M, N, K) || elem_bytes < 1 || elem_bytes > 8) return TSS_E_ARG;
  if (!valid_device(d) || !valid_config(*cfg, d)) return TSS_E_ARG;
  tss_verdict v = evaluate_block(*cfg, d, elem_bytes);
  finish(v, d, batch, M, N, K, elem_bytes);
  *out = v;
  return TSS_OK;
}


int32_t tss_tile_plan(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t elem_bytes, const tss_device *dev,
                      int32_t instr_filter, tss_verdict *best, tss_verdict *list, int32_t cap,
                      int32_t *n_feasible) {
  const tss_device d = dev ? *dev : gfx950_with_costs();
  return plan_sweep<NoUsage>(batch, M, N, FixedK{K}, elem_bytes, d, instr_filter, nullptr, best, list, cap,
                             n_feasible);
}

int32_t tss_conv_plan(int64_t Cout, int64_t pixels, int64_t C, int64_t taps, int32_t elem_bytes,
                      const tss_device *dev, tss_verdict *best, tss_verdict *list, int32_t cap,
                      int32_t *n_feasible) {
  const tss_device d = dev ? *dev : gfx950_with_costs();
  if (C < 1 || taps < 1 || C > (int64_t(1) << 30) || taps > (int64_t(1) << 20)) return TSS_E_ARG;
  if (d.ranking != TSS_RANK_GFX950 || d.lane_count != 64) return TSS_E_ARG;
  return plan_sweep<NoUsage>(1, Cout, pixels, ConvK{C, taps}, elem_bytes, d, 0, nullptr, best, list, cap,
                             n_feasible);
}

int32_t tss_splitk_plan(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t elem_bytes, const tss_device *dev,
                        tss_verdict *best, int32_t *splits) {
  const tss_device d = dev ? *dev : gfx950_with_costs();
  if (!sizes_ok(batch, M, N, K) || !valid_device(d)) return TSS_E_ARG;
  return splitk_sweep(batch, M, N, FixedK{K}, elem_bytes, d, best, splits);
}

int32_t tss_conv_splitk_plan(int64_t Cout, int64_t pixels, int64_t C, int64_t taps, int32_t elem_bytes,
                             const tss_device *dev, tss_verdict *best, int32_t *splits) {
  const tss_device d = dev ? *dev : gfx950_with_costs();
  if (C < 1 || taps < 1 || C > (int64_t(1) << 30) || taps > (int64_t(1) << 20) || !valid_device(d)) return TSS_E_ARG;
  if (d.lane_count != 64) return TSS_E_ARG;
  return splitk_sweep(1, Cout, pixels, ConvK{C, taps}, elem_bytes, d, best, splits);
}

int32_t tss_tile_plan_usage(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t elem_bytes,
                            const tss_measured_usage *table, int32_t n_table, tss_verdict *best, tss_verdict *list,
                            int32_t cap, int32_t *n_feasible) {
  if (n_table < 0 || (n_table > 0 && !table)) return TSS_E_ARG;
  for (int32_t i = 0; i < n_table; ++i)
    if (table[i].regs_per_lane <= 0 || table[i].scratch_bytes < 0) return TSS_E_ARG;
  auto usage_of = [&](const tss_tile_config &c) -> const tss_measured_usage * {
    for (int32_t i = 0; i < n_table; ++i) {
      const tss_tile_config &t = table[i].cfg;
      if (t.bm == c.bm && t.bn == c.bn && t.bk == c.bk && t.stages == c.stages && t.threads == c.threads &&
          t.instr == c.instr)
        return &table[i];
    }
    return nullptr;
  };
  return plan_sweep(batch, M, N, FixedK{K}, elem_bytes, gfx950_with_costs(), 0, &usage_of, best, list, cap,
                    n_feasible);
}

int32_t tss_hw_tile(int64_t H, int64_t kh, int64_t sh, int64_t pt, int64_t d, int64_t o0, int64_t o1,
                    tss_hw_slice *out) {
  if (!out || H <= 0 || kh <= 0 || sh <= 0 || pt < 0 || d <= 0 || o0 < 0 || o1 <= o0) return TSS_E_ARG;
  const int64_t lim = int64_t(1) << 40;
  if (H > lim || kh > lim || sh > lim || pt > lim || d > lim || o1 > lim) return TSS_E_ARG;
  // "Tiling（分块）" page, H/W tiling formulas (1)..(5)
  const int64_t window = (kh - 1) * d + 1;
  tss_hw_slice s{};
  s.o0 = o0;
  s.o1 = o1;
  s.in_start = std::max<int64_t>(0, o0 * sh - pt);
  s.in_end = (o1 - 1) * sh - pt + window;
  s.in_span = s.in_end - s.in_start;
  s.pt = std::max<int64_t>(0, pt - o0 * sh);
  s.pb = std::max<int64_t>(0, s.in_end - H);
  s.halo = window - sh;
  *out = s;
  return TSS_OK;
}

const char *tss_status_string(int32_t status) {
  switch (status) {
    case TSS_OK: return "ok";
    case TSS_E_ARG: return "invalid argument";
    case TSS_E_DTYPE: return "unsupported dtype";
    case TSS_E_ALIGN: return "pointer or row stride not 16-byte aligned";
    case TSS_E_INFEASIBLE: return "tile configuration infeasible";
    case TSS_E_HIP: return "HIP runtime error";
    case TSS_E_UNSUPPORTED: return "no compiled kernel for this configuration";
    case TSS_E_SCRATCH: return "the problem needs more scratch than the library's static array holds";
    default: return "unknown status";
  }
}

}  // extern "C"
