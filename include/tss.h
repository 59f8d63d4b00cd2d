/*
 * tss.h -- C ABI of the tile-size-selected GEMM / convolution library for
 * MI355X (gfx950), libtss.so.
 *
 * Three families of entry points:
 *
 *  1. The tile planner (host only, no GPU needed): the constraint check of the
 *     "tile_decision.py" page (tilelang tutorial ch. 28 sec. 4) -- C3
 *     instruction shape, C1 on-chip capacity, C2 register pressure, occupancy,
 *     C4 parallelism -- and the C0 DRAM-traffic model of the
 *     "04-tile-size-decision/README.md" page, evaluated on a device
 *     description, plus the sweep that ranks every candidate.
 *  2. The H-tile slice formulas of the "Tiling（分块）" page (section on the
 *     general H/W tiling formulas).
 *  3. The device operations: a tiled fp16/bf16 GEMM with fp32 accumulation,
 *     and a convolution computed as an implicit GEMM over H-tiles with halo
 *     (block -> wave -> MFMA tiling as in the Tiling page's multi-level
 *     tiling section).
 *
 * Conventions for every function:
 *  - Return value: a tss_status (0 = TSS_OK, negative = error).  No function
 *    throws, aborts or prints.  Arguments are validated before any launch;
 *    on error nothing is launched and output buffers are untouched.
 *  - Device operations are asynchronous on the given stream (a hipStream_t
 *    passed as void*, NULL = the null stream) and allocate nothing: the
 *    caller owns every buffer and keeps it alive until the stream reaches
 *    the work.
 *  - Device buffers are dense, row-major, 16-byte aligned.
 *  - Thread safety: every function may be called concurrently.
 */
#ifndef TSS_H_
#define TSS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
enum {
  TSS_OK = 0,
  TSS_E_ARG = -1,          /* null pointer, negative or oversized dimension, bad enum */
  TSS_E_DTYPE = -2,        /* unsupported input / output dtype combination */
  TSS_E_ALIGN = -3,        /* pointer or row stride not 16-byte aligned */
  TSS_E_INFEASIBLE = -4,   /* the tile config fails C1..C3 or fits no block on a CU */
  TSS_E_HIP = -5,          /* HIP runtime error (launch, device query) */
  TSS_E_UNSUPPORTED = -6,  /* feasible config with no compiled kernel */
  TSS_E_SCRATCH = -7       /* needs more scratch than the library's static array holds */
};

/* ---- element types ------------------------------------------------------- */
enum { TSS_F16 = 1, TSS_BF16 = 2, TSS_F32 = 3 };

/* ---- instruction shapes (C3) -------------------------------------------- */
enum {
  TSS_INSTR_MFMA32 = 1,    /* v_mfma_f32_32x32x16_{f16,bf16}: multiples (32, 32, 16), 64 lanes */
  TSS_INSTR_MFMA16 = 2,    /* v_mfma_f32_16x16x32_{f16,bf16}: multiples (16, 16, 32), 64 lanes */
  /* The NVIDIA shapes of the tile_decision.py page, for the pages' own
     device model only (no kernels): */
  TSS_INSTR_NV_MMA = 16,   /* mma m16n8k16: (16, 8, 16), 32 threads */
  TSS_INSTR_NV_WGMMA = 17, /* wgmma m64nNk16: (64, 8, 16), 128 threads */
  TSS_INSTR_NV_SIMT = 18   /* (1, 1, 1), 32 threads */
};

enum { TSS_REG_POOLED = 0, TSS_REG_PER_SIMD = 1 };
enum { TSS_RANK_PAGES = 0, TSS_RANK_GFX950 = 1 };

/*
 * Device description used by the planner.  Two register models:
 *  POOLED   (the tile_decision.py page): blocks by registers =
 *           regs_per_core / (regs_per_thread * threads).
 *  PER_SIMD (gfx950): waves per SIMD = min(max_waves_per_simd,
 *           regs_per_lane_per_simd / regs_per_thread); blocks by registers =
 *           simds_per_core * waves per SIMD / waves per block.
 * regs_per_thread = ceil(accumulators * 4 B / 4 B / granule) * granule +
 * reg_overhead; C2 fails when the accumulator registers exceed acc_regs_max.
 */
typedef struct {
  int32_t cores;                  /* SMs or CUs */
  int32_t onchip_per_core;        /* shared memory / LDS bytes per SM or CU */
  int32_t onchip_per_block_max;   /* usable bytes per block */
  int32_t max_threads_per_core;
  int32_t max_threads_per_block;
  int32_t max_blocks_per_core;
  int32_t lane_count;             /* warp or wavefront size */
  int32_t reg_granule_per_lane;
  int32_t acc_regs_max;
  int32_t reg_overhead;
  int32_t reg_model;              /* TSS_REG_* */
  int32_t regs_per_core;          /* POOLED only */
  int32_t simds_per_core;         /* PER_SIMD only */
  int32_t regs_per_lane_per_simd; /* PER_SIMD only */
  int32_t max_waves_per_simd;     /* PER_SIMD only */
  int32_t wave_grid_rule;         /* 1: block must split into whole MFMA tiles per wave */
  int32_t load_bytes_per_lane;    /* >0: each wave issues whole 64-lane loads per stage */
  int32_t ranking;                /* TSS_RANK_* */
  /* Cost parameters of the gfx950 ranking (ignored by the pages' ranking),
     in units of K elements of one tile's K loop:
     step_cost_k: what one K step costs beyond its BK elements of work (the
       barrier, the waits, the restart of the fragment pipeline); a tile's
       K loop of n steps of BK costs n * (BK + step_cost_k).  gfx950 model:
       22, the value at which a fixed per-step cost reproduces the measured
       time per FLOP of the 32- and 16-wide K steps relative to the 64-wide
       step at equal K (1.24x and 1.76x, convolution workload).  0 turns the
       term off: the loop then costs its padded K alone.
     tile_cost_k: the fixed cost of one round of co-resident tiles on a CU
       (prologue, epilogue, output write), as a K-loop length of the same
       tile.  gfx950 model: 900 (a round of a 256x256 tile weighs about 10
       K steps of 64; at 4096^3 its prologue and epilogue take about 10 us
       against 1.4 us per step, and the value is set above 824, where the
       K = 200 sweep's 128x128 tiles, measured faster, overtake the 256x256
       tile).  0 turns it off.
     Cost parameters of the split-K plan (tss_splitk_plan), in the same
     units (one streamed panel element):
     split_byte_cost: what one byte of the partial sums' extra traffic (each
       range's fp32 output written once and read once by the reduction)
       costs, as bytes of streamed panel; the partial sums of S ranges add
       8 * S * batch * M * N * split_byte_cost / (elem_bytes * cores).
     launch_cost_k: the fixed cost of the reduction launch.
     target_waves_per_simd: the occupancy the gfx950 ranking's tie-break
       prefers among candidates of equal time, traffic, K step and resident
       blocks: resident waves per SIMD closest to this first, then the most
       (0: the most resident waves first).  gfx950 model: 4. */
  int32_t step_cost_k;
  int32_t tile_cost_k;
  int32_t split_byte_cost;
  int32_t launch_cost_k;
  int32_t target_waves_per_simd;
} tss_device;

/* One tile configuration (block tile BM x BN, K step BK, pipeline stages,
   threads per block, instruction shape). */
typedef struct {
  int32_t bm, bn, bk, stages, threads, instr;
} tss_tile_config;

/* failure bits, in the order the constraints are checked */
enum {
  TSS_FAIL_C3_M = 1 << 0, TSS_FAIL_C3_N = 1 << 1, TSS_FAIL_C3_K = 1 << 2,
  TSS_FAIL_C3_THREADS = 1 << 3, TSS_FAIL_C3_MAXTHREADS = 1 << 4,
  TSS_FAIL_C3_WAVEGRID = 1 << 5, TSS_FAIL_C3_LOAD = 1 << 6,
  TSS_FAIL_C1 = 1 << 7, TSS_FAIL_C2 = 1 << 8, TSS_FAIL_OCC0 = 1 << 9
};
enum { TSS_WARN_TAIL = 1, TSS_WARN_IDLE = 2 };
enum { TSS_BIND_NONE = 0, TSS_BIND_REGS = 1, TSS_BIND_SMEM = 2, TSS_BIND_THREADS = 3 };

/*
 * Verdict on one configuration for one problem.  All figures are exact:
 * last-wave fill = fill_num / fill_den; C0 traffic in bytes =
 * (traffic_num_hi * 2^64 + traffic_num_lo) / traffic_den in lowest terms,
 * traffic_rounded its round-half-to-even integer value.
 */
typedef struct {
  tss_tile_config cfg;
  int64_t smem_per_stage, smem_total;
  int64_t accum_per_thread, regs_per_thread, regs_per_block;
  int64_t blocks_by_regs, blocks_by_smem, blocks_by_threads, blocks_per_core;
  int64_t grid, waves, fill_num, fill_den;
  uint64_t traffic_num_hi, traffic_num_lo, traffic_den, traffic_rounded;
  uint32_t failures;   /* TSS_FAIL_* bits; 0 = feasible */
  uint32_t warnings;   /* TSS_WARN_* bits (C4) */
  int32_t binding;     /* TSS_BIND_*: the first of regs, smem, threads at the minimum */
  int32_t pad_;
} tss_verdict;

/* The multiples an instruction shape imposes (C3): out[0..3] = block M, block
   N and block K multiples and the thread-count multiple (the lanes that issue
   it).  Errors: TSS_E_ARG (out NULL, unknown instr). */
int32_t tss_instr_shape(int32_t instr, int32_t out[4]);

/* The MI355X (gfx950) model: 256 CUs, 160 KiB LDS per CU and per block,
   wave64, 4 SIMDs x 8 waves, 512-deep unified VGPR file (256 accumulation
   registers), 32 blocks per CU.  out: non-null. */
int32_t tss_device_gfx950(tss_device *out);

/* The tile_decision.py page's device model (H100/H200 defaults: sm_count
   132, smem_kb 228; the per-block limit is smem_kb KiB minus 1 KiB).
   sm_count, smem_kb > 0. */
int32_t tss_device_pages(int32_t sm_count, int32_t smem_kb, tss_device *out);

/* The gfx950 model with the CU count and LDS sizes read from HIP device
   hip_device.  Needs a GPU; TSS_E_HIP otherwise. */
int32_t tss_device_query(int32_t hip_device, tss_device *out);

/*
 * C3, C1, C2, occupancy, C4 and C0 for cfg on dev, for a batch of M x N x K
 * GEMMs whose operands take elem_bytes per element.  dev NULL = gfx950.
 * Infeasibility is reported in out->failures, not as an error.
 * Errors: TSS_E_ARG (null cfg/out, dimensions < 0 or batch < 1, elem_bytes
 * not 1..8, non-positive config fields, unknown instr for the device).
 */
int32_t tss_evaluate(const tss_tile_config *cfg, const tss_device *dev, int64_t batch, int64_t M,
                     int64_t N, int64_t K, int32_t elem_bytes, tss_verdict *out);

/*
 * Sweep every candidate of the device's space, keep the feasible ones and
 * rank them (stable over the enumeration order instr, BM, BN, BK, stages,
 * threads).  Candidates with BK > K are skipped, unless K is below the
 * smallest BK of the space, in which case that smallest BK is kept.
 *   pages model : BM, BN in {16..256}, BK in {16..128}, stages 2..4,
 *                 threads {128, 256, 512}, instr fixed by *instr_filter;
 *                 key (round(traffic), -blocks/SM, shared memory).
 *   gfx950 model: BM, BN in {256, 128, 64} (largest first), BK in
 *                 {16, 32, 64}, stages 2..4, threads {128, 256, 512}, both
 *                 MFMA shapes, 16x16x32 first (or the one in instr_filter);
 *                 key (T, round(traffic), -BK, -u,
 *                 |u * waves/block - SIMDs * dev->target_waves_per_simd|
 *                 (0 when the target is 0), -u * waves/block, -stages, LDS
 *                 bytes).  T is the busiest CU's time in units
 *                 of streamed panel elements: with W = ceil(grid / CUs)
 *                 tiles on that CU, u = min(blocks/CU, W) of them resident
 *                 at once (R = ceil(W / u) rounds) and n = ceil(K / BK) K
 *                 steps per tile,
 *                   T = W * (BM + BN) * n * (BK + dev->step_cost_k)
 *                     + R * (BM + BN) * dev->tile_cost_k.
 * instr_filter: 0 = every shape of the device, else one TSS_INSTR_*.
 * best (nullable) receives the top verdict; list (nullable) the first
 * min(cap, n) verdicts in rank order; *n_feasible (nullable) the count.
 * Sizes: batch in [1, 2^20], M, N, K in [0, 2^40], batch * M * N <= 2^62
 * (TSS_E_ARG otherwise); traffic_rounded saturates at 2^64 - 1 (the exact
 * value stays in traffic_num / traffic_den and ranks the candidates).
 * Returns TSS_E_INFEASIBLE when nothing is feasible (best then untouched).
 */
int32_t tss_tile_plan(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t elem_bytes,
                      const tss_device *dev, int32_t instr_filter, tss_verdict *best,
                      tss_verdict *list, int32_t cap, int32_t *n_feasible);

/*
 * The gfx950 plan for a convolution computed as an implicit GEMM ("Tiling（分块）"
 * page: a convolution is a GEMM with M = output channels, N = output pixels,
 * K = C * kh * kw).  The kernel pads the channels of each tap to a multiple
 * of the tile's K step, so a candidate with step BK computes
 * K = taps * ceil(C / BK) * BK; each candidate is finished (C4, C0) and
 * ranked (tss_tile_plan's gfx950 key) with its own K.  With the step cost
 * (dev->step_cost_k) a shorter K step is chosen only where the padding it
 * saves outweighs the steps it adds; with step_cost_k = 0 a candidate's K
 * loop costs its padded K alone.  Where C is a multiple of 64 every BK
 * gives K = taps * C.
 * Cout: output channels (M); pixels: output pixels of the whole problem (N);
 * C: input channels; taps: kh * kw; dev: a device with the gfx950 ranking
 * (NULL = tss_device_gfx950).  best, list, cap, n_feasible as for
 * tss_tile_plan (the verdicts' traffic uses each candidate's own K).
 * Errors: TSS_E_ARG (C < 1, taps < 1, sizes out of range, dev not ranked
 * the gfx950 way), TSS_E_INFEASIBLE.
 */
int32_t tss_conv_plan(int64_t Cout, int64_t pixels, int64_t C, int64_t taps, int32_t elem_bytes,
                      const tss_device *dev, tss_verdict *best, tss_verdict *list, int32_t cap,
                      int32_t *n_feasible);

/*
 * The split-K plan (gfx950 ranking): for S in {1, 2, 3, 4, 6, 8, 12, 16},
 * the tile plan of the split problem -- batch * S GEMMs of M x N x
 * ceil(K / S) (tss_tile_plan) -- whose busiest-CU time T_S (the first term
 * of the rank key) is charged, for S > 1, the partial sums' traffic and the
 * reduction launch (dev->split_byte_cost, dev->launch_cost_k); S is kept only
 * when its tile's K steps cut K into exactly S ranges.  The least total
 * wins, the smaller S on a tie.  *splits: on entry 0 (choose S as above) or
 * the S to plan the tile for (1..256); on return the S; best (nullable)
 * receives the verdict of the tile for the split problem.  The tile and S
 * are what tss_gemm_splitk takes for splits = 0 (its tile for a given S and
 * a NULL cfg is this plan's with *splits = S).  dev NULL = gfx950 (it must
 * rank the gfx950 way).
 * Errors: TSS_E_ARG (as tss_tile_plan, splits NULL or out of range),
 * TSS_E_INFEASIBLE.
 */
int32_t tss_splitk_plan(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t elem_bytes, const tss_device *dev,
                        tss_verdict *best, int32_t *splits);

/* The same for a convolution's implicit GEMM (as tss_conv_plan: each
   candidate's K is taps * ceil(C / BK) * BK, split into S ranges). */
int32_t tss_conv_splitk_plan(int64_t Cout, int64_t pixels, int64_t C, int64_t taps, int32_t elem_bytes,
                             const tss_device *dev, tss_verdict *best, int32_t *splits);

/*
 * The planner with feedback from the compiled kernels.  The tile_decision.py
 * page's C2 counts only the accumulators, and its README lists the register
 * model as a known limitation.  Here each candidate takes what its compiled
 * kernel uses: the registers per lane replace the model's estimate (rounded
 * up to the allocation granule) in the occupancy, and so in C4's resident
 * blocks, waves and fill and in the ranking; a kernel that spills to scratch
 * fails C2 (the page's "expect spilling to local memory").  Which
 * configurations are candidates is still the model's decision (C3, C1, C2 on
 * the accumulators, occupancy).
 * table: n_table entries (configuration, registers per lane > 0, scratch
 * bytes per lane >= 0); a candidate absent from the table is left out.
 * gfx950 model and ranking (as tss_tile_plan with dev = NULL, instr_filter
 * = 0).
 * Errors: TSS_E_ARG (bad sizes, n_table < 0, table NULL with n_table > 0, a
 * register count <= 0 or negative scratch), TSS_E_INFEASIBLE (no candidate).
 */
typedef struct {
  tss_tile_config cfg;
  int32_t regs_per_lane, scratch_bytes;
} tss_measured_usage;

int32_t tss_tile_plan_usage(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t elem_bytes,
                            const tss_measured_usage *table, int32_t n_table, tss_verdict *best,
                            tss_verdict *list, int32_t cap, int32_t *n_feasible);

/* One H-tile of a convolution ("Tiling（分块）" page, H/W tiling formulas):
   output rows [o0, o1) need input rows [in_start, in_end) (in_end exclusive,
   may exceed H), sub-operator pads pt' (top) and pb' (bottom), and share
   halo rows with the next tile.  The slice read from the input is
   [in_start, min(in_end, H)); it is empty (min(in_end, H) <= in_start) for a
   tile whose windows lie wholly in the padding, and pt' + (min(in_end, H) -
   in_start) + pb' is the tile's window span in every case. */
typedef struct {
  int64_t o0, o1, in_start, in_end, in_span, pt, pb, halo;
} tss_hw_slice;

/* H > 0, kh > 0, sh > 0, pt >= 0, d > 0, 0 <= o0 < o1.  TSS_E_ARG otherwise. */
int32_t tss_hw_tile(int64_t H, int64_t kh, int64_t sh, int64_t pt, int64_t d, int64_t o0,
                    int64_t o1, tss_hw_slice *out);

/*
 * C[b] = A[b] x B[b] for b < batch: A is M x K, B is K x N, C is M x N, all
 * row-major and batch-major (A[b][M][K], B[b][K][N], C[b][M][N]).
 * dtype: TSS_F16 or TSS_BF16 (A and B); fp32 accumulation; out_dtype
 * TSS_F32, or the input dtype (rounded to nearest even).
 * cfg: the tile configuration to use, or NULL to take the planner's choice
 * (tss_tile_plan on the gfx950 model, cached per shape).
 * Requirements: batch >= 1, M, N, K >= 0; K and N multiples of 8 (16-byte
 * rows); A, B, C 16-byte aligned; each operand slice below 2 GiB.
 * M == 0 or N == 0: nothing to do.  K == 0: C is zero-filled (A and B may
 * then be NULL).
 * Errors: TSS_E_ARG, TSS_E_DTYPE, TSS_E_ALIGN, TSS_E_INFEASIBLE (cfg fails
 * C1..C3), TSS_E_UNSUPPORTED (no compiled kernel for cfg), TSS_E_HIP.
 */
int32_t tss_gemm(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B,
                 void *C, int64_t batch, int32_t out_dtype, const tss_tile_config *cfg,
                 void *stream);

/*
 * 2-D convolution, NCHW input x[N][C][H][W], OIHW weights w[Cout][C][kh][kw],
 * output y[N][Cout][OH][OW] with OH = (H + 2ph - (kh-1)dh - 1)/sh + 1 and OW
 * likewise, computed as an implicit GEMM (M = Cout, N = pixels, K over the
 * kh*kw taps and the channels) over output-row tiles of tile_oh rows.  Each
 * H-tile reads exactly its input slice [in_start, min(in_end, H)) with the
 * sub-operator pads of the Tiling page's H/W tiling formulas (tss_hw_tile);
 * the batch never crosses a tile.
 * Two launches on `stream`: the operands are first rewritten into
 * `workspace` (input channel-last x[n][h][w][c], weights w[o][r][s][c], the
 * channels zero-padded to Cp = C rounded up to a multiple of the tile's K
 * step, 16, 32 or 64), then the implicit GEMM reads them.  workspace: device memory of at least
 * tss_conv2d_workspace_size(...) bytes, 16-byte aligned, owned by the caller;
 * its contents are scratch and are overwritten on every call (calls that
 * share a workspace must be ordered on one stream).  A workspace of at least
 * twice that size holds two sets of the copies, and consecutive calls
 * alternate between them (a process-wide counter picks the set): the layout
 * pass then does not rewrite the lines the previous call's GEMM has just
 * read, which on MI355X takes it from about 9.5 to 6.5 us on an 8x256x56x56
 * input.  The results do not depend on the set.
 * dtype TSS_F16 / TSS_BF16, fp32 accumulation, out_dtype TSS_F32 or dtype.
 * tile_oh in [1, OH]; cfg NULL = tss_conv_plan's choice for the implicit
 * GEMM (Cout x N*OH*OW, K = kh*kw*C with C padded to each candidate's K
 * step).  x, w, y 16-byte aligned.
 * Errors: TSS_E_ARG (also for a missing or too small workspace), TSS_E_DTYPE,
 * TSS_E_ALIGN, TSS_E_INFEASIBLE, TSS_E_UNSUPPORTED, TSS_E_HIP.
 */
int32_t tss_conv2d(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                   int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                   int64_t dw, int64_t tile_oh, int32_t dtype, int32_t out_dtype, const void *x,
                   const void *w, void *y, void *workspace, int64_t workspace_bytes,
                   const tss_tile_config *cfg, void *stream);

/*
 * The same convolution over tiles of tile_n images x tile_oh output rows x
 * tile_ow output columns (tss_conv2d is tile_n = N, tile_ow = OW).  The H/W
 * tiling formulas of the Tiling page hold for either dimension: a tile reads
 * input rows [in_start, min(in_end, H)) and columns [w_start, min(w_end, W))
 * of its images, with the sub-operator pads pt'/pb' and pl'/pr' that
 * tss_hw_tile gives for (H, kh, sh, ph, dh) and for (W, kw, sw, pw, dw);
 * neighbouring tiles re-read the halo rows and columns.  Splitting the batch
 * (the page's batch split) needs no halo.  The tiling changes which input a
 * block reads, not the order of the sums: any tiling gives the same bits for
 * the same cfg.
 * tile_n in [1, N], tile_oh in [1, OH], tile_ow in [1, OW], and
 * tile_n * tile_oh * tile_ow < 2^31.  Everything else as tss_conv2d (one
 * GEMM batch entry per tile; cfg NULL = tss_conv_plan's choice for the
 * whole problem, Cout x N*OH*OW).
 * Errors: as tss_conv2d.
 */
int32_t tss_conv2d_tiled(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                         int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                         int64_t dw, int64_t tile_n, int64_t tile_oh, int64_t tile_ow, int32_t dtype,
                         int32_t out_dtype, const void *x, const void *w, void *y, void *workspace,
                         int64_t workspace_bytes, const tss_tile_config *cfg, void *stream);

/*
 * The same convolution on channel-last tensors, read in place: input
 * x[N][H][W][C] (NHWC), weights w[Cout][kh][kw][C] (OHWI), output
 * y[N][OH][OW][Cout] (NHWC).  The implicit GEMM's K runs over (r, s, ci), so
 * a channel-last pixel is a contiguous run of K: the kernel of
 * tss_conv2d_tiled copies its B rows (8 channels of one input pixel per
 * 16-byte chunk) and its A rows straight from x and w, one launch and no
 * operand copies.  Each tap's channels are padded to the tile's K step as in
 * tss_conv2d (the same K, the same plan, the same sum order); the padding is
 * not in memory and reads as zero.  Same tiles, H/W tiling formulas and
 * halo as tss_conv2d_tiled.
 * Requirements: C a multiple of 8 (16-byte pixels); x, w, y 16-byte aligned.
 * splits in [0, 256] as tss_conv2d_splitk: 1 = one pass (workspace unused,
 * may be NULL); 0 = the split-K plan's count; > 1 = K cut into ranges whose
 * fp32 partial outputs go to workspace (at least
 * tss_conv2d_nhwc_workspace_size(..., S) bytes for the count S used,
 * 16-byte aligned, owned by the caller).
 * Everything else, and the errors, as tss_conv2d_splitk; TSS_E_ARG also for
 * C not a multiple of 8.
 */
int32_t tss_conv2d_nhwc(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                        int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                        int64_t dw, int64_t tile_n, int64_t tile_oh, int64_t tile_ow, int32_t dtype,
                        int32_t out_dtype, const void *x, const void *w, void *y, int32_t splits,
                        void *workspace, int64_t workspace_bytes, const tss_tile_config *cfg,
                        void *stream);

/* splits * N * Cout * OH * OW * 4 bytes (0 for splits == 1), or TSS_E_ARG
   (< 0) for splits outside [1, 256] or arguments tss_conv2d_nhwc would
   reject on size alone. */
int64_t tss_conv2d_nhwc_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout,
                                       int64_t kh, int64_t kw, int64_t sh, int64_t sw, int64_t ph,
                                       int64_t pw, int64_t dh, int64_t dw, int32_t splits);

/*
 * Measured choice of the tile (the Tiling page's autotuning: enumerate the
 * candidates, time each on the device, keep the fastest), for shapes where
 * the model's ranking alone falls short (short K loops, where one tile's
 * 256- and 512-thread versions rank equal but do not run equal).  Takes the
 * first `topk` candidates of tss_tile_plan's gfx950 ranking for this
 * problem, times `iters` back-to-back launches of each on `stream` with HIP
 * events, in two interleaved rounds over all candidates (after running the
 * first candidate for at least 20 ms to bring the engine clock up; one
 * untimed launch before each timing), and returns the candidate with the
 * least time of its better round in *best (the better-ranked one of equal
 * times) and that time per launch in *best_us (may be NULL).
 * Arguments as tss_gemm; C receives the products of every candidate in
 * turn (every candidate computes the same product; C holds the last one).
 * Blocking: it synchronizes with the stream after each candidate.  The
 * choice depends on the measurement (run-to-run noise can pick either of
 * two tiles within a few percent of each other); pass it to tss_gemm as cfg.
 * topk in [1, 1024], iters in [1, 100000].
 * Errors: as tss_gemm, and TSS_E_ARG for topk or iters out of range or a
 * NULL best.
 */
int32_t tss_gemm_autotune(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A,
                          const void *B, void *C, int64_t batch, int32_t out_dtype, int32_t topk,
                          int32_t iters, void *stream, tss_tile_config *best, float *best_us);

/*
 * Split K: the same GEMM with its K loop cut into ranges computed by
 * separate blocks, for problems whose output tiles alone leave CUs idle (the
 * C4 "idle" warning of the tile_decision.py page: fewer tiles than CUs).
 * K is cut into at most `splits` ranges of equal length in whole K steps of
 * the tile (the last range holds the rest; fewer ranges when K is short).
 * Each range adds its products into its own fp32 partial output in
 * `workspace`; a second launch on `stream` adds the ranges of every output
 * element in range order (0, 1, ...) and converts the sum to out_dtype, so
 * every run gives the same bits (the sum order differs from the one-pass
 * GEMM's, the result not).
 * splits in [0, 256]; 0 = the split-K plan's count (tss_splitk_plan; with
 * its tile when cfg is NULL); 1 = tss_gemm (workspace unused, may be NULL);
 * with splits > 1 and a NULL cfg the tile is tss_splitk_plan's for that S.
 * workspace: device memory, 16-byte aligned, of at least
 * tss_gemm_splitk_workspace_size(batch, M, N, splits) bytes, owned by the
 * caller; scratch, overwritten by every call (calls sharing it must be
 * ordered on one stream).  Everything else as tss_gemm.
 * Errors: as tss_gemm; TSS_E_ARG also for splits out of range or a missing
 * or too small workspace.
 */
int32_t tss_gemm_splitk(int64_t M, int64_t N, int64_t K, int32_t dtype, const void *A, const void *B, void *C,
                        int64_t batch, int32_t out_dtype, const tss_tile_config *cfg, int32_t splits,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* splits * batch * M * N * 4 bytes (0 for splits == 1), or TSS_E_ARG (< 0)
   for sizes tss_gemm_splitk would reject. */
int64_t tss_gemm_splitk_workspace_size(int64_t batch, int64_t M, int64_t N, int32_t splits);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * tss_conv2d_splitk with its workspace (the operand layout copies and the
 * K ranges' partial outputs) in a static device array of the library,
 * TSS_SCRATCH_BYTES bytes per GPU, held from the first call on that GPU
 * until the process ends.  Allocates nothing (no hipMalloc, no allocating
 * library call); the array's address on the current device is looked up on
 * the first call on that device.  Every call on one GPU uses the same array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be ordered by the caller.  Arguments and results as tss_conv2d_splitk.
 * Errors: as tss_conv2d_splitk; TSS_E_SCRATCH when the problem needs more
 * than TSS_SCRATCH_BYTES (tss_conv2d_splitk_workspace_size for the split
 * count used); TSS_E_HIP if the array's address cannot be read.
 */
#define TSS_SCRATCH_BYTES ((int64_t)64 << 20)
int32_t tss_conv2d_splitk_noalloc(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw,
                                  int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                                  int64_t tile_n, int64_t tile_oh, int64_t tile_ow, int32_t dtype,
                                  int32_t out_dtype, const void *x, const void *w, void *y, int32_t splits,
                                  const tss_tile_config *cfg, void *stream);

/* Bytes of workspace tss_conv2d needs for these sizes with any tile
   configuration (channels padded to 64), or TSS_E_ARG (< 0) for sizes
   tss_conv2d would reject as non-positive or above 2^30. */
int64_t tss_conv2d_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout,
                                  int64_t kh, int64_t kw);

/*
 * tss_conv2d_tiled with the implicit GEMM's K loop (taps x channels) cut into
 * at most `splits` ranges of whole K steps, as tss_gemm_splitk: each range's
 * fp32 partial output goes to the workspace after the operand layout copies,
 * and a last launch adds them in range order into y.  splits in [0, 256]
 * (0: tss_conv_splitk_plan's count, and its tile for a NULL cfg); workspace
 * of at least tss_conv2d_splitk_workspace_size(...) bytes for that count
 * (with room for a second set of the operand copies as well, that is
 * tss_conv2d_workspace_size rounded up to 256 bytes more, the two sets
 * alternate as in tss_conv2d, and the partial outputs follow both).
 * Everything else as tss_conv2d_tiled.
 */
int32_t tss_conv2d_splitk(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh, int64_t kw,
                          int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t tile_n,
                          int64_t tile_oh, int64_t tile_ow, int32_t dtype, int32_t out_dtype, const void *x,
                          const void *w, void *y, int32_t splits, void *workspace, int64_t workspace_bytes,
                          const tss_tile_config *cfg, void *stream);

/* tss_conv2d_workspace_size rounded up to 256 bytes plus splits fp32 copies
   of the output (the layout part alone for splits == 1), or TSS_E_ARG. */
int64_t tss_conv2d_splitk_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Cout, int64_t kh,
                                         int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                                         int64_t dw, int32_t splits);

/* 1 if a kernel is compiled for cfg and dtype (op 0 = GEMM, 1 = conv), else 0. */
int32_t tss_kernel_available(const tss_tile_config *cfg, int32_t dtype, int32_t op);

/*
 * What the compiled kernel for (cfg, dtype, op) uses, read through the HIP
 * runtime from its code object: registers per lane (VGPRs and AGPRs of the
 * unified file), LDS per block (static plus the launch's dynamic size),
 * private memory per lane (register spills; 0 = none), the largest block it
 * accepts, and the blocks per CU the runtime's occupancy calculator allows
 * at the launch's block size and LDS.  Needs a GPU.
 * Errors: TSS_E_ARG (NULL pointer, op not 0/1), TSS_E_UNSUPPORTED (no kernel
 * compiled for cfg), TSS_E_HIP (no device, runtime error).
 */
typedef struct {
  int32_t regs_per_lane, lds_bytes, scratch_bytes, max_threads, blocks_per_cu, pad_;
} tss_kernel_usage;

int32_t tss_kernel_usage_query(const tss_tile_config *cfg, int32_t dtype, int32_t op,
                               tss_kernel_usage *out);

/* tss_tile_plan_usage with the table read from every compiled kernel of
   (dtype, op) by tss_kernel_usage_query (read once per process).  Needs a
   GPU; errors as both. */
int32_t tss_tile_plan_measured(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t op,
                               tss_verdict *best, tss_verdict *list, int32_t cap, int32_t *n_feasible);

/*
 * LDS bank microbenchmark, the gfx950 counterpart of the Tiling page's table
 * of bank conflicts by access stride and of its XOR swizzle.  Launches
 * `blocks` blocks of 8 waves; every wave times (shader clock cycles) `iters`
 * x 8 LDS reads of one pattern and writes the count to cycles[block * 8 +
 * wave] (device memory, blocks * 8 int64, owned by the caller).
 *   TSS_LDS_B32 / TSS_LDS_B128 / TSS_LDS_TR_B64: lane l reads 4 / 16 / 8
 *     bytes (ds_read_b32, ds_read_b128, ds_read_b64_tr_b16) at byte
 *     l * stride_words * 4; stride_words in [0, 4096], a multiple of 4 for
 *     B128 and of 2 for TR_B64;
 *   TSS_LDS_GEMM_A(_PLAIN): the GEMM kernel's A fragment read (256x256x64
 *     tile, 8 waves, 16x16x32 MFMA) with (without) its XOR swizzle;
 *   TSS_LDS_GEMM_B(_PLAIN): its B fragment transpose read likewise;
 *   stride_words is ignored for the GEMM patterns.
 * iters in [1, 2^20], blocks in [1, 65536].  Asynchronous on `stream`.
 * Errors: TSS_E_ARG, TSS_E_HIP.
 */
enum {
  TSS_LDS_B32 = 1, TSS_LDS_B128 = 2, TSS_LDS_TR_B64 = 3, TSS_LDS_GEMM_A = 4, TSS_LDS_GEMM_A_PLAIN = 5,
  TSS_LDS_GEMM_B = 6, TSS_LDS_GEMM_B_PLAIN = 7
};
int32_t tss_lds_probe(int32_t pattern, int32_t stride_words, int32_t iters, int32_t blocks, int64_t *cycles,
                      void *stream);

/* The configuration tss_gemm / tss_conv2d would take for a NULL cfg. */
int32_t tss_gemm_default_config(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t dtype,
                                tss_tile_config *out);

/* Static text for a status code (never NULL). */
const char *tss_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* TSS_H_ */
