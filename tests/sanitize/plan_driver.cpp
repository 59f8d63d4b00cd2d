// The planner's C entry points under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; built with g++ by
// tests/test_host_sanitizers.py).  It drives every planner call over a grid of
// problems -- the workloads, ragged, tiny, empty and at the ABI's bounds --
// on the gfx950 model, the pages' H100 model and a model with other cost
// parameters, plus the argument checks, and prints a checksum of the
// verdicts so that the calls cannot be optimised away.  Exit status 0; a
// sanitizer finding aborts with its report.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/tss.h"

namespace {

uint64_t mix(uint64_t h, uint64_t v) { return (h ^ v) * 0x100000001b3ull; }

uint64_t digest(const tss_verdict &v) {
  uint64_t h = 0xcbf29ce484222325ull;
  h = mix(h, uint64_t(v.cfg.bm) << 32 | uint32_t(v.cfg.bn));
  h = mix(h, uint64_t(v.cfg.bk) << 32 | uint32_t(v.cfg.threads));
  h = mix(h, uint64_t(v.grid));
  h = mix(h, v.traffic_rounded);
  h = mix(h, uint64_t(v.blocks_per_core));
  return h;
}

}  // namespace

int main() {
  tss_device g{}, p{}, a{}, c{};
  if (tss_device_gfx950(&g) != TSS_OK || tss_device_pages(132, 228, &p) != TSS_OK ||
      tss_device_pages(108, 164, &a) != TSS_OK || tss_device_gfx950(&c) != TSS_OK)
    return 1;
  c.step_cost_k = 40;
  c.tile_cost_k = 2000;
  c.target_waves_per_simd = 2;
  const tss_device *devs[] = {nullptr, &g, &p, &a, &c};
  const int64_t dims[] = {0, 1, 7, 72, 256, 3000, 4096, 8192, int64_t(1) << 20, int64_t(1) << 31, int64_t(1) << 40};
  const int64_t batches[] = {1, 4, int64_t(1) << 20};
  std::vector<tss_verdict> list(600);
  uint64_t sum = 0;
  long calls = 0, ok = 0;
  for (const tss_device *d : devs)
    for (int64_t b : batches)
      for (int64_t M : dims)
        for (int64_t N : dims)
          for (int64_t K : dims) {
            tss_verdict best{};
            int32_t n = 0;
            const int32_t st = tss_tile_plan(b, M, N, K, 2, d, 0, &best, list.data(), int32_t(list.size()), &n);
            ++calls;
            if (st == TSS_OK) {
              ++ok;
              sum = mix(sum, digest(best));
              for (int32_t i = 0; i < n && i < int32_t(list.size()); ++i) sum = mix(sum, digest(list[i]));
            }
            if (M == N && N == K) {  // split K and the conv plan on the cube's sizes
              for (int32_t want : {0, 3}) {
                int32_t s = want;
                if (tss_splitk_plan(b, M, N, K, 2, d, &best, &s) == TSS_OK) sum = mix(sum, digest(best) + uint64_t(s));
                s = want;
                if (tss_conv_splitk_plan(M, N, K, 9, 2, d, &best, &s) == TSS_OK)
                  sum = mix(sum, digest(best) + uint64_t(s));
              }
              if (tss_conv_plan(M, N * b, K, 9, 2, d, &best, list.data(), 8, &n) == TSS_OK) sum = mix(sum, digest(best));
              ++calls;
            }
          }
  // every configuration of a small space evaluated on both models, infeasible ones included
  const int32_t instrs[] = {TSS_INSTR_MFMA32, TSS_INSTR_MFMA16, TSS_INSTR_NV_MMA, TSS_INSTR_NV_WGMMA, TSS_INSTR_NV_SIMT, 0, 99};
  for (int32_t bm : {0, 16, 64, 96, 256, 512})
    for (int32_t bn : {8, 64, 256})
      for (int32_t bk : {16, 64, 256})
        for (int32_t st : {1, 2, 4})
          for (int32_t thr : {0, 32, 64, 128, 256, 512, 1024, 2048})
            for (int32_t ins : instrs)
              for (const tss_device *d : devs) {
                tss_tile_config cfg{bm, bn, bk, st, thr, ins};
                tss_verdict v{};
                if (tss_evaluate(&cfg, d, 3, 3000, 5000, 2048, 2, &v) == TSS_OK) sum = mix(sum, digest(v));
                ++calls;
              }
  // measured-usage plans with a table that covers part of the space
  std::vector<tss_measured_usage> table;
  for (int32_t i = 0; i < 300; ++i) {
    tss_measured_usage u{};
    const int32_t sizes[] = {64, 128, 256};
    u.cfg = {sizes[i % 3], sizes[(i / 3) % 3], 16 << (i % 3), 2 + i % 3, 128 << (i % 3),
             i % 2 ? TSS_INSTR_MFMA16 : TSS_INSTR_MFMA32};
    u.regs_per_lane = 24 + (i * 37) % 480;
    u.scratch_bytes = i % 11 == 0 ? 64 : 0;
    table.push_back(u);
  }
  for (int64_t M : dims) {
    tss_verdict best{};
    int32_t n = 0;
    if (tss_tile_plan_usage(1, M, M, M, 2, table.data(), int32_t(table.size()), &best, list.data(),
                            int32_t(list.size()), &n) == TSS_OK)
      sum = mix(sum, digest(best));
    ++calls;
  }
  // H/W tile formulas over small geometries, bounds included
  for (int64_t H = 1; H <= 12; ++H)
    for (int64_t kh = 1; kh <= 4; ++kh)
      for (int64_t sh = 1; sh <= 3; ++sh)
        for (int64_t pt = 0; pt <= 3; ++pt)
          for (int64_t d = 1; d <= 2; ++d)
            for (int64_t o0 = -1; o0 <= 6; ++o0)
              for (int64_t o1 = o0; o1 <= o0 + 3; ++o1) {
                tss_hw_slice s{};
                if (tss_hw_tile(H, kh, sh, pt, d, o0, o1, &s) == TSS_OK)
                  sum = mix(sum, uint64_t(s.in_start) ^ uint64_t(s.in_end) << 16 ^ uint64_t(s.pt) << 32 ^
                                     uint64_t(s.pb) << 48);
                ++calls;
              }
  // null pointers and bad arguments return codes, never crash
  tss_verdict v{};
  int32_t n = 0, s = 0;
  tss_tile_config cfg{256, 256, 64, 2, 512, TSS_INSTR_MFMA16};
  int32_t bad = 0;
  bad += tss_tile_plan(0, 64, 64, 64, 2, nullptr, 0, &v, nullptr, 0, &n) == TSS_OK;
  bad += tss_tile_plan(-1, 64, 64, 64, 2, nullptr, 0, &v, nullptr, 0, &n) == TSS_OK;
  bad += tss_tile_plan(1, 64, 64, 64, 9, nullptr, 0, &v, nullptr, 0, &n) == TSS_OK;
  bad += tss_tile_plan(1, int64_t(1) << 41, 64, 64, 2, nullptr, 0, &v, nullptr, 0, &n) == TSS_OK;
  bad += tss_evaluate(nullptr, nullptr, 1, 64, 64, 64, 2, &v) == TSS_OK;
  bad += tss_evaluate(&cfg, nullptr, 1, 64, 64, 64, 2, nullptr) == TSS_OK;
  bad += tss_splitk_plan(1, 64, 64, 64, 2, nullptr, &v, nullptr) == TSS_OK;
  s = 257;
  bad += tss_splitk_plan(1, 64, 64, 64, 2, nullptr, &v, &s) == TSS_OK;
  bad += tss_conv_plan(64, 64, 0, 9, 2, nullptr, &v, nullptr, 0, &n) == TSS_OK;
  bad += tss_hw_tile(0, 3, 1, 1, 1, 0, 1, nullptr) == TSS_OK;
  bad += tss_device_pages(0, 228, &p) == TSS_OK;
  for (int32_t code = -10; code <= 2; ++code) sum = mix(sum, uint64_t(tss_status_string(code)[0]));
  std::printf("calls %ld ok %ld bad %d checksum %016llx\n", calls, ok, bad, (unsigned long long)sum);
  return bad == 0 ? 0 : 2;
}
