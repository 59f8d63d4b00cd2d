/*
 * tss_plan -- command line of the tile planner, over the C ABI of libtss.so.
 *
 * The interface of the "tile_decision.py" page (tilelang tutorial ch. 28
 * sec. 4, its main() and print_verdict()): a sweep that lists the feasible
 * configurations in rank order, or (--diagnose) the constraint-by-constraint
 * verdict on one configuration.  The output lines that the
 * "04-tile-size-decision/README.md" page prints under its expected output
 * (the C1 / C2 / occupancy / FAIL lines of a diagnosis, the table rows and
 * the counts of a sweep) keep that format, so the page's printout can be
 * compared with this program's.
 *
 *   --device gfx950 (default) | pages     the MI355X model, or the pages'
 *                                         NVIDIA model (H100/H200 defaults)
 *   --m --n --k --batch                   the GEMM (default 4096^3, batch 1)
 *   --instr                               mfma16 | mfma32 (gfx950; default:
 *                                         both), mma | wgmma | simt (pages;
 *                                         default wgmma)
 *   --sm-count --smem-kb                  the pages' device override (SMs,
 *                                         shared memory per SM in KiB)
 *   --block-m --block-n --block-k --stages --threads
 *                                         the configuration to diagnose
 *   --topk                                rows of the sweep table (15)
 *   --diagnose                            diagnose instead of sweeping
 *
 * Exit status 0 whether or not the configuration is feasible (failures are
 * part of the verdict, as on the page); 2 for a bad command line.
 */
#include <getopt.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tss.h"

static const struct {
  const char *name;
  int32_t id;
} kInstr[] = {{"mfma16", TSS_INSTR_MFMA16}, {"mfma32", TSS_INSTR_MFMA32}, {"mma", TSS_INSTR_NV_MMA},
              {"wgmma", TSS_INSTR_NV_WGMMA}, {"simt", TSS_INSTR_NV_SIMT}};

static const char *instr_name(int32_t id) {
  for (size_t i = 0; i < sizeof kInstr / sizeof kInstr[0]; ++i)
    if (kInstr[i].id == id) return kInstr[i].name;
  return "?";
}

static int32_t instr_id(const char *name) {
  for (size_t i = 0; i < sizeof kInstr / sizeof kInstr[0]; ++i)
    if (strcmp(kInstr[i].name, name) == 0) return kInstr[i].id;
  return -1;
}

static const char *binding_name(int32_t b) {
  switch (b) {
    case TSS_BIND_REGS: return "regs";
    case TSS_BIND_SMEM: return "smem";
    case TSS_BIND_THREADS: return "threads";
    default: return "";
  }
}

struct Ctx {
  tss_device dev;
  int gfx;            /* 1: gfx950 model */
  const char *core;   /* "SM" or "CU" */
};

/* C0 in bytes as a double (the value is an exact rational in the verdict) */
static double traffic_bytes(const tss_verdict *v) {
  const double two64 = 18446744073709551616.0;
  return ((double)v->traffic_num_hi * two64 + (double)v->traffic_num_lo) / (double)v->traffic_den;
}

static double fill_of(const tss_verdict *v) { return v->fill_den ? (double)v->fill_num / (double)v->fill_den : 0.0; }

/* The failure and warning lines of a verdict, in the order the constraints
   are checked. */
static void print_problems(const struct Ctx *x, const tss_verdict *v, const char *indent) {
  const tss_tile_config *c = &v->cfg;
  int32_t sh[4] = {0, 0, 0, 0};
  tss_instr_shape(c->instr, sh);
  const char *in = instr_name(c->instr);
  const uint32_t f = v->failures;
  if (f & TSS_FAIL_C3_M) printf("%sFAIL  C3 block_M=%d is not a multiple of %d (%s)\n", indent, c->bm, sh[0], in);
  if (f & TSS_FAIL_C3_N) printf("%sFAIL  C3 block_N=%d is not a multiple of %d (%s)\n", indent, c->bn, sh[1], in);
  if (f & TSS_FAIL_C3_K) printf("%sFAIL  C3 block_K=%d is not a multiple of %d (%s)\n", indent, c->bk, sh[2], in);
  if (f & TSS_FAIL_C3_THREADS)
    printf("%sFAIL  C3 threads=%d is not a multiple of %d (%s)\n", indent, c->threads, sh[3], in);
  if (f & TSS_FAIL_C3_MAXTHREADS)
    printf("%sFAIL  C3 threads=%d exceeds %d per block\n", indent, c->threads, x->dev.max_threads_per_block);
  if (f & TSS_FAIL_C3_WAVEGRID)
    printf("%sFAIL  C3 block (%d,%d) does not split into whole %dx%d tiles per wave for %d waves\n", indent,
           c->bm, c->bn, sh[0], sh[1], c->threads / x->dev.lane_count);
  if (f & TSS_FAIL_C3_LOAD) {
    int32_t waves = c->threads / x->dev.lane_count;
    if (waves < 1) waves = 1;
    printf("%sFAIL  C3 operand tiles are not whole %d-byte block loads\n", indent,
           x->dev.load_bytes_per_lane * x->dev.lane_count * waves);
  }
  if (f & TSS_FAIL_C1)
    printf("%sFAIL  C1 shared %lld B > %d B per block at stages=%d\n", indent, (long long)v->smem_total,
           x->dev.onchip_per_block_max, c->stages);
  if (f & TSS_FAIL_C2)
    printf("%sFAIL  C2 accumulators alone need %lld registers/thread (> %d); expect spilling to local memory\n",
           indent, (long long)(v->regs_per_thread - x->dev.reg_overhead), x->dev.acc_regs_max);
  if (f & TSS_FAIL_OCC0) printf("%sFAIL  C1/C2 no resident block fits: blocks_per_SM = 0\n", indent);
  if (v->warnings & TSS_WARN_TAIL) {
    int64_t resident = v->blocks_per_core * x->dev.cores;
    if (resident < 1) resident = 1;
    printf("%swarn  C4 last wave only %.0f%% full (%lld tiles / %lld resident): tail effect\n", indent,
           fill_of(v) * 100.0, (long long)v->grid, (long long)resident);
  }
  if (v->warnings & TSS_WARN_IDLE)
    printf("%swarn  C4 only %lld tiles for %d %ss: more than half the machine is idle\n", indent,
           (long long)v->grid, x->dev.cores, x->core);
}

static void print_verdict(const struct Ctx *x, const tss_verdict *v) {
  const tss_tile_config *c = &v->cfg;
  const int lanes = x->dev.lane_count;
  printf("block=(%4d,%4d,%3d)  stages=%d  threads=%4d  instr=%s\n", c->bm, c->bn, c->bk, c->stages, c->threads,
         instr_name(c->instr));
  printf("  C1 shared/stage %8.1f KB -> total %8.1f KB\n", v->smem_per_stage / 1024.0, v->smem_total / 1024.0);
  printf("  C2 accumulators %5lld/thread -> %4lld regs/thread (%s-rounded), %6lld regs/block\n",
         (long long)v->accum_per_thread, (long long)v->regs_per_thread, x->gfx ? "granule" : "warp",
         (long long)v->regs_per_block);
  printf("     occupancy: regs -> %lld blk/%s, smem -> %lld, threads -> %lld  => %lld blk/%s (%lld of the %d-block "
         "hardware limit), binding=%s\n",
         (long long)v->blocks_by_regs, x->core, (long long)v->blocks_by_smem, (long long)v->blocks_by_threads,
         (long long)v->blocks_per_core, x->core, (long long)v->blocks_per_core, x->dev.max_blocks_per_core,
         binding_name(v->binding));
  printf("  C0 DRAM traffic %9.1f MB  (b*M*N*K*(1/block_N + 1/block_M) + b*M*N)\n", traffic_bytes(v) / 1e6);
  printf("  C4 grid %6lld tiles over %3lld-%s blocks -> %lld wave(s), last wave %5.1f%% full\n", (long long)v->grid,
         (long long)(v->blocks_per_core * c->threads / lanes), x->gfx ? "wave" : "warp", (long long)v->waves,
         fill_of(v) * 100.0);
  print_problems(x, v, "  ");
  if (!v->failures) printf("  OK    all four constraints satisfied\n");
  printf("\n");
}

static int sweep(const struct Ctx *x, int64_t batch, int64_t m, int64_t n, int64_t k, int32_t instr, int topk) {
  int32_t count = 0;
  int32_t st = tss_tile_plan(batch, m, n, k, 2, &x->dev, instr, NULL, NULL, 0, &count);
  if (st != TSS_OK && st != TSS_E_INFEASIBLE) {
    fprintf(stderr, "tss_plan: %s\n", tss_status_string(st));
    return 2;
  }
  tss_verdict *list = (tss_verdict *)calloc(count > 0 ? (size_t)count : 1, sizeof(tss_verdict));
  if (!list) return 2;
  if (count > 0) tss_tile_plan(batch, m, n, k, 2, &x->dev, instr, NULL, list, count, &count);
  printf("feasible configurations found: %d\n", count);
  printf("%8s%8s%8s%3s%5s%10s%8s%9s%7s%6s%7s  binding\n", "block_M", "block_N", "block_K", "st", "thr",
         "trafficMB", x->gfx ? "ldsKB" : "smemKB", "regs/thr", x->gfx ? "blk/CU" : "blk/SM", "waves", "tail");
  for (int i = 0; i < count && i < topk; ++i) {
    const tss_verdict *v = &list[i];
    const tss_tile_config *c = &v->cfg;
    printf("%8d%8d%8d%3d%5d%10.1f%8.1f%9lld%7lld%6lld%6.0f%%  %s", c->bm, c->bn, c->bk, c->stages, c->threads,
           traffic_bytes(v) / 1e6, v->smem_total / 1024.0, (long long)v->regs_per_thread,
           (long long)v->blocks_per_core, (long long)v->waves, fill_of(v) * 100.0, binding_name(v->binding));
    if (x->gfx) printf("  %s", instr_name(c->instr));
    printf("\n");
  }
  printf("\n");
  /* how many configurations share the least C0 traffic, and the fullest last wave */
  uint64_t least = UINT64_MAX;
  double best_fill = 0.0;
  for (int i = 0; i < count; ++i) {
    if (list[i].traffic_rounded < least) least = list[i].traffic_rounded;
    if (fill_of(&list[i]) > best_fill) best_fill = fill_of(&list[i]);
  }
  int tied = 0;
  for (int i = 0; i < count; ++i) tied += list[i].traffic_rounded == least;
  printf("configurations tied at the minimum traffic: %d\n", count ? tied : 0);
  printf("best last-wave fill among feasible configurations: %.0f%%\n", best_fill * 100.0);
  if (count) {
    const tss_tile_config *c = &list[0].cfg;
    printf("\nfirst choice, diagnosed in full by: tss_plan%s --diagnose --block-m %d --block-n %d --block-k %d "
           "--stages %d --threads %d --instr %s\n",
           x->gfx ? "" : " --device pages", c->bm, c->bn, c->bk, c->stages, c->threads, instr_name(c->instr));
  }
  free(list);
  return 0;
}

static void usage(void) {
  fprintf(stderr,
          "usage: tss_plan [--device gfx950|pages] [--m M] [--n N] [--k K] [--batch B] [--instr NAME]\n"
          "                [--sm-count S] [--smem-kb KB] [--topk T] [--diagnose --block-m BM --block-n BN\n"
          "                --block-k BK --stages ST --threads TH]\n");
}

static int parse_i64(const char *s, int64_t *out) {
  char *end = NULL;
  long long v = strtoll(s, &end, 10);
  if (!s[0] || *end) return 0;
  *out = (int64_t)v;
  return 1;
}

int main(int argc, char **argv) {
  enum { O_DEVICE = 1, O_M, O_N, O_K, O_BATCH, O_INSTR, O_SMS, O_SMEM, O_BM, O_BN, O_BK, O_ST, O_THR, O_TOPK, O_DIAG };
  static struct option opts[] = {{"device", required_argument, 0, O_DEVICE}, {"m", required_argument, 0, O_M},
                                 {"n", required_argument, 0, O_N},           {"k", required_argument, 0, O_K},
                                 {"batch", required_argument, 0, O_BATCH},   {"instr", required_argument, 0, O_INSTR},
                                 {"sm-count", required_argument, 0, O_SMS},  {"smem-kb", required_argument, 0, O_SMEM},
                                 {"block-m", required_argument, 0, O_BM},    {"block-n", required_argument, 0, O_BN},
                                 {"block-k", required_argument, 0, O_BK},    {"stages", required_argument, 0, O_ST},
                                 {"threads", required_argument, 0, O_THR},   {"topk", required_argument, 0, O_TOPK},
                                 {"diagnose", no_argument, 0, O_DIAG},       {0, 0, 0, 0}};
  int64_t m = 4096, n = 4096, k = 4096, batch = 1, sms = 132, smem_kb = 228, topk = 15;
  int64_t bm = 128, bn = 128, bk = 32, stages = 3, threads = 256;
  const char *device = "gfx950", *instr = NULL;
  int diagnose = 0, sm_given = 0;
  int c;
  while ((c = getopt_long(argc, argv, "", opts, NULL)) != -1) {
    int64_t *dst = NULL;
    switch (c) {
      case O_DEVICE: device = optarg; continue;
      case O_INSTR: instr = optarg; continue;
      case O_DIAG: diagnose = 1; continue;
      case O_M: dst = &m; break;
      case O_N: dst = &n; break;
      case O_K: dst = &k; break;
      case O_BATCH: dst = &batch; break;
      case O_SMS: dst = &sms; sm_given = 1; break;
      case O_SMEM: dst = &smem_kb; sm_given = 1; break;
      case O_BM: dst = &bm; break;
      case O_BN: dst = &bn; break;
      case O_BK: dst = &bk; break;
      case O_ST: dst = &stages; break;
      case O_THR: dst = &threads; break;
      case O_TOPK: dst = &topk; break;
      default: usage(); return 2;
    }
    if (!parse_i64(optarg, dst)) {
      usage();
      return 2;
    }
  }
  if (optind < argc) {
    usage();
    return 2;
  }
  struct Ctx x;
  memset(&x, 0, sizeof x);
  if (strcmp(device, "gfx950") == 0) {
    x.gfx = 1;
    x.core = "CU";
    tss_device_gfx950(&x.dev);
    if (sm_given) {
      fprintf(stderr, "tss_plan: --sm-count / --smem-kb describe the pages' device (--device pages)\n");
      return 2;
    }
  } else if (strcmp(device, "pages") == 0) {
    x.core = "SM";
    if (sms < 1 || sms > INT32_MAX || smem_kb < 2 || smem_kb > (1 << 20) ||
        tss_device_pages((int32_t)sms, (int32_t)smem_kb, &x.dev) != TSS_OK) {
      usage();
      return 2;
    }
  } else {
    usage();
    return 2;
  }
  int32_t iid = 0;
  if (instr) {
    iid = instr_id(instr);
  } else if (!x.gfx) {
    iid = TSS_INSTR_NV_WGMMA;
  } else if (diagnose) {
    iid = TSS_INSTR_MFMA16;
  }
  if (iid < 0 || (iid && ((x.gfx != 0) != (iid == TSS_INSTR_MFMA16 || iid == TSS_INSTR_MFMA32)))) {
    fprintf(stderr, "tss_plan: instruction %s is not one of this device's\n", instr ? instr : "?");
    return 2;
  }
  if (x.gfx)
    printf("device: MI355X (gfx950)  CUs=%d  LDS/CU=%d KB  LDS/block<=%d KB  VGPRs/lane/SIMD=%d\n", x.dev.cores,
           x.dev.onchip_per_core / 1024, x.dev.onchip_per_block_max / 1024, x.dev.regs_per_lane_per_simd);
  else
    printf("device: H100/H200 (sm_90)  SMs=%d  shared/SM=%d KB  shared/block<=%d KB  regs/SM=%d\n", x.dev.cores,
           x.dev.onchip_per_core / 1024, x.dev.onchip_per_block_max / 1024, x.dev.regs_per_core);
  printf("target: %s%lldx%lldx%lld fp16 -> fp32 accum, intrinsic=%s\n\n", "", (long long)m, (long long)n,
         (long long)k, iid ? instr_name(iid) : "mfma16+mfma32");
  if (batch != 1) printf("batch: %lld\n\n", (long long)batch);

  if (diagnose) {
    if (bm < 1 || bn < 1 || bk < 1 || stages < 1 || threads < 1 || bm > INT32_MAX || bn > INT32_MAX ||
        bk > INT32_MAX || stages > INT32_MAX || threads > INT32_MAX) {
      usage();
      return 2;
    }
    tss_tile_config cfg = {(int32_t)bm, (int32_t)bn, (int32_t)bk, (int32_t)stages, (int32_t)threads, iid};
    tss_verdict v;
    int32_t st = tss_evaluate(&cfg, &x.dev, batch, m, n, k, 2, &v);
    if (st != TSS_OK) {
      fprintf(stderr, "tss_plan: %s\n", tss_status_string(st));
      return 2;
    }
    printf("the requested configuration, constraint by constraint\n");
    printf("------------------------------------------------------------------------------\n");
    print_verdict(&x, &v);
    return 0;
  }
  if (topk < 0 || topk > INT32_MAX) {
    usage();
    return 2;
  }
  return sweep(&x, batch, m, n, k, iid, (int)topk);
}
