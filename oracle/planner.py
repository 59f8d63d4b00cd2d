"""Tile-size constraint checker (C0..C4) and shortlist sweep -- the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the "tile_decision.py" page (tilelang tutorial chapter 28 section 4,
"Tile-size decision procedure"), whose module docstring lists the four
constraints C1..C4; the "04-tile-size-decision/README.md" page, which adds the
C0 DRAM-traffic term to the same list; and the constraint-analysis section of
the "Tiling（分块）" page (shared-memory capacity, register pressure with an
overhead term, occupancy).

Every quantity is an integer or an exact rational (``fractions.Fraction``), so
verdicts can be compared bit for bit with any other implementation.

Two families of device model share one evaluation routine:

* ``pages`` models (H100/H200 and the A100 override of the README's commands):
  the pages' own constants and register model -- registers pooled per SM,
  divided by registers per block -- and the pages' ranking key.
* the ``gfx950`` model (MI355X): 256 CUs, 160 KiB LDS per CU and per
  workgroup, wave64, 4 SIMDs per CU with a 512-entry unified VGPR file per
  lane (256 of which can be accumulation registers), v_mfma f16/bf16 shapes.
  The register model is per SIMD; accumulators are counted as on the pages
  plus the fixed per-thread overhead of the Tiling page's register example;
  the block must split into a grid of waves whose sub-tiles are whole MFMA
  tiles; and each operand tile must split into the same whole number of
  wave-wide 16-byte-per-lane loads for every wave.  These additions are
  readings, listed with their reasons in the design notes of the repository.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

# ---------------------------------------------------------------------------
# Device models
# ---------------------------------------------------------------------------

REG_POOLED = "pooled"     # regs per SM // regs per block       (tile_decision.py page)
REG_PER_SIMD = "per_simd"  # waves per SIMD from the per-lane VGPR file (gfx950)


@dataclass(frozen=True)
class DeviceModel:
    name: str
    cores: int                      # SMs (NVIDIA) or CUs (AMD)
    onchip_per_core: int            # shared memory / LDS bytes per SM or CU
    onchip_per_block_max: int       # usable bytes per block (workgroup)
    max_threads_per_core: int
    max_threads_per_block: int
    max_blocks_per_core: int
    lane_count: int                 # warp (32) or wavefront (64) size
    reg_granule_per_lane: int       # per-thread register allocation granule
    acc_regs_max: int               # C2 cap on accumulator registers per thread
    reg_overhead: int               # registers per thread beyond accumulators
    reg_model: str
    regs_per_core: int = 0          # pooled model: 32-bit registers per SM
    simds_per_core: int = 0         # per-SIMD model
    regs_per_lane_per_simd: int = 0  # per-SIMD model: unified VGPR file depth
    max_waves_per_simd: int = 0     # per-SIMD model
    instr_shapes: Tuple[Tuple[str, Tuple[int, int, int, int]], ...] = ()
    wave_grid_rule: bool = False    # gfx950: block splits into whole MFMA tiles per wave
    load_bytes_per_lane: int = 0    # gfx950: operand tiles are whole wave-wide loads
    ranking: str = "pages"
    # cost parameters of the gfx950 ranking, in K elements of a tile's K loop
    # (see busiest_core_time); the pages' ranking does not use them
    step_cost_k: int = 0            # a K step's cost beyond its BK elements
    tile_cost_k: int = 0            # a round of co-resident tiles' fixed cost
    # the gfx950 ranking's occupancy tie-break: resident waves per SIMD closest
    # to this first (0: none, the most resident waves first)
    target_waves_per_simd: int = 0
    # cost parameters of the split-K plan (see splitk_total)
    split_byte_cost: int = 0        # one byte of partial-sum traffic, in streamed panel bytes
    launch_cost_k: int = 0          # the reduction launch, in streamed panel elements
    core_name: str = "SM"           # how messages name a core

    def shape(self, instr: str) -> Tuple[int, int, int, int]:
        for k, v in self.instr_shapes:
            if k == instr:
                return v
        raise KeyError(f"instruction {instr!r} not known on {self.name}")


# The pages' instruction multiples (M, N, K, threads) for the NVIDIA paths
# (tile_decision.py page, "Instruction-shape constraints"): the warp-level mma
# m16n8k16, the warpgroup wgmma m64nNk16 with N a multiple of 8 and 128
# threads, and plain SIMT code.
NVIDIA_SHAPES = (("mma", (16, 8, 16, 32)), ("simt", (1, 1, 1, 32)), ("wgmma", (64, 8, 16, 128)))

# gfx950 dense f16/bf16 MFMA shapes: v_mfma_f32_16x16x32_{f16,bf16} and
# v_mfma_f32_32x32x16_{f16,bf16}; both are issued by one 64-lane wave.  The
# 16x16 one is listed first, so it wins ties: it keeps the 16x16 output tile
# of the MMA level in the Tiling page's multi-level tiling section.
GFX950_SHAPES = (("mfma16", (16, 16, 32, 64)), ("mfma32", (32, 32, 16, 64)))


def device_pages(sm_count: int = 132, smem_kb: int = 228) -> DeviceModel:
    """The H100/H200 defaults of the tile_decision.py page's Device record.

    The command line of that page describes other devices only through the SM
    count and the shared memory per SM; the per-block limit it derives is one
    KiB less than the per-SM figure (227 KiB for the 228 KiB default).
    """
    return DeviceModel(
        name="H100/H200 (sm_90)", cores=sm_count,
        onchip_per_core=smem_kb * 1024, onchip_per_block_max=smem_kb * 1024 - 1024,
        max_threads_per_core=2048, max_threads_per_block=1024, max_blocks_per_core=32,
        lane_count=32, reg_granule_per_lane=256 // 32, acc_regs_max=255, reg_overhead=0,
        reg_model=REG_POOLED, regs_per_core=65536,
        instr_shapes=NVIDIA_SHAPES, ranking="pages")


# The gfx950 model's cost parameters.  They are properties of the kernels
# (measured), not of the pages: a K step costs about 22 K elements beyond its
# BK (with that fixed cost per step, the 32- and 16-wide steps take 1.24x and
# 1.76x the 64-wide step's time per FLOP at equal K, as measured on the
# convolution workload); a round of co-resident tiles costs about 900 K
# elements more (the 4096^3 GEMM's prologue and epilogue, about 10 us, against
# 1.41 us per 64-wide K step of 86 K elements' cost, put the figure near 600;
# 900 is the value above 824, the point past which the K = 200 GEMM's 128x128
# tiles, measured faster there, rank ahead of the 256x256 tile).  Among
# candidates the time, traffic, K step and residency rank equal, 4 resident
# waves per SIMD is preferred (the 256-thread blocks that ran 8-16% faster
# than their 512-thread twins on K loops of 2 to 4 steps).  The functions
# below take these from the device record, so any other values can be given
# through dataclasses.replace.
GFX950_STEP_COST_K = 22
GFX950_TILE_COST_K = 900
GFX950_TARGET_WAVES_PER_SIMD = 4
# Split K: each byte of the partial sums' extra traffic costs as much as 6
# bytes of streamed panel, and the reduction launch as much as 67000 panel
# elements; with these, the split count of the split-K plan measured within
# 5% of the fastest split count on nine GEMM shapes.
GFX950_SPLIT_BYTE_COST = 6
GFX950_LAUNCH_COST_K = 67000


def device_gfx950() -> DeviceModel:
    """MI355X (gfx950).  Values confirmed on the device through hipDeviceProp_t:
    256 CUs, 163840 B LDS per CU and per block, 2048 threads per CU, 1024 per
    block, 32 blocks per CU, wave64.  From the CDNA4 ISA: 4 SIMDs per CU, 8
    waves per SIMD, a 512-deep unified VGPR file per lane with at most 256
    accumulation registers, allocation granule 8.  The per-thread overhead of
    32 registers is the Tiling page's register example (constraint two)."""
    return DeviceModel(
        name="MI355X (gfx950)", cores=256,
        onchip_per_core=163840, onchip_per_block_max=163840,
        max_threads_per_core=2048, max_threads_per_block=1024, max_blocks_per_core=32,
        lane_count=64, reg_granule_per_lane=8, acc_regs_max=256, reg_overhead=32,
        reg_model=REG_PER_SIMD, simds_per_core=4, regs_per_lane_per_simd=512,
        max_waves_per_simd=8, instr_shapes=GFX950_SHAPES,
        wave_grid_rule=True, load_bytes_per_lane=16, ranking="gfx950",
        step_cost_k=GFX950_STEP_COST_K, tile_cost_k=GFX950_TILE_COST_K,
        target_waves_per_simd=GFX950_TARGET_WAVES_PER_SIMD,
        split_byte_cost=GFX950_SPLIT_BYTE_COST, launch_cost_k=GFX950_LAUNCH_COST_K, core_name="CU")


# Wave grids (rows x cols of waves) a block of n waves is split into.
WAVE_GRIDS = {1: (1, 1), 2: (1, 2), 4: (2, 2), 8: (2, 4), 16: (4, 4)}

# ---------------------------------------------------------------------------
# Records
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class TileConfig:
    block_m: int
    block_n: int
    block_k: int
    stages: int = 3
    threads: int = 128
    instr: str = "wgmma"


@dataclass
class Verdict:
    config: TileConfig
    smem_per_stage: int = 0
    smem_total: int = 0
    accum_per_thread: int = 0
    regs_per_thread: int = 0
    regs_per_block: int = 0
    blocks_by_regs: int = 0
    blocks_by_smem: int = 0
    blocks_by_threads: int = 0
    blocks_per_core: int = 0
    grid: int = 0
    waves: int = 0
    fill: Fraction = Fraction(0)
    traffic: Fraction = Fraction(0)
    k_loop: int = 0                                     # the K the candidate's loop runs over
    failures: List[str] = field(default_factory=list)   # constraint codes, in check order
    messages: List[str] = field(default_factory=list)   # human-readable FAIL text
    warnings: List[str] = field(default_factory=list)   # C4 codes: "tail", "idle"
    warn_text: List[str] = field(default_factory=list)
    binding: str = ""

    @property
    def feasible(self) -> bool:
        return not self.failures


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ---------------------------------------------------------------------------
# C3, C1, C2, occupancy  (checked in this order, as the procedure prescribes:
# the instruction shape first because it is the cheapest mistake to make)
# ---------------------------------------------------------------------------


def _c3_checks(cfg: TileConfig, dev: DeviceModel, elem_bytes: int) -> List[Tuple[str, str]]:
    """C3, instruction-shape multiples: (failure code, message) for every
    way the block fails to be a whole number of the intrinsic's tiles, of
    its issuing group of threads, of the device's thread limit, and on gfx950
    of a wave grid of whole MFMA tiles and of whole wave-wide copies."""
    out = []
    im, inn, ik, it = dev.shape(cfg.instr)
    dims = (("C3_M", cfg.block_m, "block_M", im), ("C3_N", cfg.block_n, "block_N", inn),
            ("C3_K", cfg.block_k, "block_K", ik))
    out += [(code, f"C3 {name}={dim} is not a multiple of {mult} ({cfg.instr})")
            for code, dim, name, mult in dims if dim % mult]
    if cfg.threads % it:
        out.append(("C3_THREADS", f"C3 threads={cfg.threads} is not a multiple of {it} ({cfg.instr})"))
    if cfg.threads > dev.max_threads_per_block:
        out.append(("C3_MAXTHREADS", f"C3 threads={cfg.threads} exceeds {dev.max_threads_per_block} per block"))
    if dev.wave_grid_rule:
        waves = cfg.threads // dev.lane_count if cfg.threads % dev.lane_count == 0 else 0
        grid = WAVE_GRIDS.get(waves)
        if grid is None or cfg.block_m % (grid[0] * im) or cfg.block_n % (grid[1] * inn):
            out.append(("C3_WAVEGRID", f"C3 block ({cfg.block_m},{cfg.block_n}) does not split into whole"
                                       f" {im}x{inn} tiles per wave for {cfg.threads // dev.lane_count} waves"))
    if dev.load_bytes_per_lane:
        # each wave copies the same whole number of wave-wide loads of each operand tile per stage
        unit = dev.load_bytes_per_lane * dev.lane_count * max(cfg.threads // dev.lane_count, 1)
        if (cfg.block_m * cfg.block_k * elem_bytes) % unit or (cfg.block_k * cfg.block_n * elem_bytes) % unit:
            out.append(("C3_LOAD", f"C3 operand tiles are not whole {unit}-byte block loads"))
    return out


def _c1_bytes(cfg: TileConfig, elem_bytes: int) -> Tuple[int, int]:
    """C1's on-chip footprint: one A tile (block_M x block_K) and one B tile
    (block_K x block_N) per pipeline stage -> (bytes per stage, total)."""
    per_stage = (cfg.block_m * cfg.block_k + cfg.block_k * cfg.block_n) * elem_bytes
    return per_stage, per_stage * cfg.stages


def _c2_registers(cfg: TileConfig, dev: DeviceModel, accum_bytes: int) -> Tuple[int, int]:
    """C2's register model: the C tile's accumulators spread over the
    block's threads, in 4-byte registers rounded up to the allocation
    granule -> (accumulators per thread, accumulator registers per lane)."""
    acc = _ceil_div(cfg.block_m * cfg.block_n, cfg.threads)
    regs = _ceil_div(acc * accum_bytes // 4, dev.reg_granule_per_lane) * dev.reg_granule_per_lane
    return acc, regs


def _residency(v: Verdict, cfg: TileConfig, dev: DeviceModel) -> None:
    """Resident blocks per SM/CU allowed by registers, on-chip memory and
    threads, under the hardware block cap; the binding resource is the first
    of (regs, smem, threads) attaining the least.  Fills v."""
    if dev.reg_model == REG_POOLED:
        v.blocks_by_regs = dev.regs_per_core // max(v.regs_per_block, 1)
    else:
        waves_per_simd = min(dev.max_waves_per_simd, dev.regs_per_lane_per_simd // v.regs_per_thread)
        v.blocks_by_regs = (dev.simds_per_core * waves_per_simd) // max(_ceil_div(cfg.threads, dev.lane_count), 1)
    v.blocks_by_smem = dev.onchip_per_core // max(v.smem_total, 1)
    v.blocks_by_threads = dev.max_threads_per_core // max(cfg.threads, 1)
    limits = (("regs", v.blocks_by_regs), ("smem", v.blocks_by_smem), ("threads", v.blocks_by_threads))
    least = min(n for _, n in limits)
    v.blocks_per_core = max(min(least, dev.max_blocks_per_core), 0)
    if v.blocks_per_core > 0:
        v.binding = next(name for name, n in limits if n == least)


def evaluate(cfg: TileConfig, dev: DeviceModel, elem_bytes: int = 2, accum_bytes: int = 4,
             regs_measured: Optional[int] = None, spill_bytes: int = 0) -> Verdict:
    """C3, C1, C2 and occupancy of one configuration, failures listed in
    that order.  regs_measured: the registers per lane a compiled kernel of
    this configuration uses; given, they replace the register estimate in
    the occupancy (rounded up to the allocation granule).  spill_bytes > 0:
    that kernel spills to scratch, which fails C2 -- the README page names
    the accumulator-only register model a limitation, and C2's own message
    is the spill."""
    v = Verdict(config=cfg)
    for code, msg in _c3_checks(cfg, dev, elem_bytes):
        v.failures.append(code)
        v.messages.append(msg)

    v.smem_per_stage, v.smem_total = _c1_bytes(cfg, elem_bytes)
    if v.smem_total > dev.onchip_per_block_max:
        v.failures.append("C1")
        v.messages.append(f"C1 shared {v.smem_total} B > {dev.onchip_per_block_max} B per block"
                          f" at stages={cfg.stages}")

    v.accum_per_thread, acc_regs = _c2_registers(cfg, dev, accum_bytes)
    v.regs_per_thread = acc_regs + dev.reg_overhead
    if regs_measured:
        v.regs_per_thread = _ceil_div(regs_measured, dev.reg_granule_per_lane) * dev.reg_granule_per_lane
    if acc_regs > dev.acc_regs_max:
        v.failures.append("C2")
        v.messages.append(f"C2 accumulators alone need {acc_regs} registers/thread"
                          f" (> {dev.acc_regs_max}); expect spilling to local memory")
    elif spill_bytes > 0:
        v.failures.append("C2")
        v.messages.append(f"C2 the compiled kernel spills {spill_bytes} bytes/thread to local memory")
    v.regs_per_block = v.regs_per_thread * cfg.threads

    _residency(v, cfg, dev)
    if v.blocks_per_core == 0:
        v.failures.append("OCC0")
        v.messages.append("C1/C2 no resident block fits: blocks_per_SM = 0")
    return v


# ---------------------------------------------------------------------------
# C4 -- parallelism: how many waves of tiles the grid takes and how full the
# last one is.
# ---------------------------------------------------------------------------


def finish_parallelism(v: Verdict, m: int, n: int, dev: DeviceModel, batch: int = 1) -> Verdict:
    cfg = v.config
    v.grid = batch * _ceil_div(m, cfg.block_m) * _ceil_div(n, cfg.block_n)
    resident = max(v.blocks_per_core * dev.cores, 1)
    v.waves = _ceil_div(v.grid, resident)
    rem = v.grid % resident
    v.fill = Fraction(rem, resident) if rem else Fraction(1)
    if v.waves > 1 and v.fill < Fraction(1, 2):
        v.warnings.append("tail")
        v.warn_text.append(f"C4 last wave only {float(v.fill) * 100:.0f}% full "
                           f"({v.grid} tiles / {resident} resident): tail effect")
    if v.grid < dev.cores:
        v.warnings.append("idle")
        v.warn_text.append(f"C4 only {v.grid} tiles for {dev.cores} {dev.core_name}s: more than half the machine"
                           f" is idle")
    return v


# ---------------------------------------------------------------------------
# C0 -- DRAM traffic model: every C tile streams its A panel (block_M x K) and
# B panel (K x block_N) once, and C is written once:
#     b*M*N*K*(1/block_N + 1/block_M) + b*M*N,   b = bytes per element.
# A batch of independent GEMMs multiplies the whole expression.
# ---------------------------------------------------------------------------


def dram_traffic(m: int, n: int, k: int, cfg: TileConfig, elem_bytes: int = 2, batch: int = 1) -> Fraction:
    return batch * (elem_bytes * m * n * k * (Fraction(1, cfg.block_n) + Fraction(1, cfg.block_m))
                    + elem_bytes * m * n)


def round_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    diff = x - fl
    if diff > Fraction(1, 2):
        return fl + 1
    if diff < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


# ---------------------------------------------------------------------------
# Sweep
# ---------------------------------------------------------------------------

PAGES_SPACE = dict(bm=(16, 32, 64, 128, 256), bn=(16, 32, 64, 128, 256), bk=(16, 32, 64, 128),
                   stages=(2, 3, 4), threads=(128, 256, 512))
# gfx950: tile sides largest first, so that of two otherwise equal tiles the
# taller one comes first (it copies fewer B chunks per FLOP; in the
# convolution those are the copies that carry per-lane pad and slice tests).
GFX950_SPACE = dict(bm=(256, 128, 64), bn=(256, 128, 64), bk=(16, 32, 64),
                    stages=(2, 3, 4), threads=(128, 256, 512))


def busiest_core_time(v: Verdict, dev: DeviceModel, k_loop: Optional[int] = None) -> int:
    """The time the busiest CU needs, in units of streamed panel elements,
    for a finished gfx950 candidate whose K loop runs over k_loop elements.

    C4 deals the grid out over the cores, so the busiest one gets
    W = ceil(grid / cores) tiles, of which at most u = min(blocks_per_core, W)
    are resident at once: R = ceil(W / u) rounds.  Each tile streams the C0
    panels of its K loop, BM + BN elements per K element, over
    n = ceil(k_loop / BK) steps that cost BK + step_cost_k each, and each
    round pays tile_cost_k more K elements' worth of its panels:

        T = W * (BM + BN) * n * (BK + step_cost_k) + R * (BM + BN) * tile_cost_k

    Every candidate tile's intensity 2*BM*BN / ((BM + BN) * b) (Tiling page)
    is below the device ridge (gfx950: 2516.6 TFLOP/s over 8 TB/s, about 315
    FLOP/B), which is why streamed panel elements measure time."""
    c = v.config
    k = v.k_loop if k_loop is None else k_loop
    w = _ceil_div(v.grid, dev.cores)
    if w == 0:
        return 0
    u = min(v.blocks_per_core, w)
    rounds = _ceil_div(w, max(u, 1))
    steps = _ceil_div(k, c.block_k)
    panel = c.block_m + c.block_n
    return w * panel * steps * (c.block_k + dev.step_cost_k) + rounds * panel * dev.tile_cost_k


def rank_key(v: Verdict, dev: DeviceModel, k_loop: Optional[int] = None):
    """Order of preference among feasible candidates.

    pages: least modelled DRAM traffic, then most resident blocks, then least
    shared memory (the tile_decision.py page's shortlist order).
    gfx950: least time on the busiest CU (busiest_core_time: C0 per tile
    under C4's dealing of the grid over the cores), then least total traffic
    (C0); then, as the Tiling page's rules of thumb advise when on-chip memory
    has room, the larger block_K; then most resident blocks per CU (occupancy,
    that page's third constraint), counting only the blocks the grid can
    supply (a CU never holds more than ceil(grid / cores) blocks at once);
    then resident waves per SIMD nearest target_waves_per_simd, then the most
    resident waves; then the deeper pipeline; then less LDS.
    """
    t = round_half_even(v.traffic)
    if dev.ranking == "pages":
        return (t, -v.blocks_per_core, v.smem_total)
    c = v.config
    usable = min(v.blocks_per_core, _ceil_div(v.grid, dev.cores))
    resident_waves = usable * (c.threads // dev.lane_count)
    # distance from the target, kept in whole waves per CU:
    # |waves / simds - target| * simds
    off = abs(resident_waves - dev.simds_per_core * dev.target_waves_per_simd) if dev.target_waves_per_simd else 0
    return (busiest_core_time(v, dev, k_loop), t, -c.block_k, -usable, off, -resident_waves, -c.stages,
            v.smem_total)


def candidates(dev: DeviceModel, k: int, instrs: Sequence[str]):
    space = PAGES_SPACE if dev.ranking == "pages" else GFX950_SPACE
    # a K step longer than K is skipped -- unless K is shorter than every
    # candidate step, when the shortest one is kept (its tail is masked)
    bk_cap = max(k, min(space["bk"]))
    for instr in instrs:
        it = dev.shape(instr)[3]
        for bm in space["bm"]:
            for bn in space["bn"]:
                for bk in space["bk"]:
                    if bk > bk_cap:
                        continue
                    for st in space["stages"]:
                        for thr in space["threads"]:
                            if thr % it:
                                continue
                            yield TileConfig(bm, bn, bk, st, thr, instr)


def sweep(m: int, n: int, k: int, dev: DeviceModel, instrs: Sequence[str], batch: int = 1,
          elem_bytes: int = 2, regs: Optional[dict] = None) -> List[Verdict]:
    """All feasible candidates in preference order (a stable sort over the
    enumeration order block_M, block_N, block_K, stages, threads, with the
    instruction shape outermost).  regs: {TileConfig: (registers per lane,
    scratch bytes per lane) of its compiled kernel}; given, the model still
    decides which candidates exist, those missing from regs are left out, and
    the others take their occupancy from the measured registers and fail C2
    if they spill."""
    out = []
    for cfg in candidates(dev, k, instrs):
        v = evaluate(cfg, dev, elem_bytes=elem_bytes)
        if not v.feasible:
            continue
        if regs is not None:
            if cfg not in regs:
                continue
            r, spill = regs[cfg]
            v = evaluate(cfg, dev, elem_bytes=elem_bytes, regs_measured=r, spill_bytes=spill)
            if not v.feasible:
                continue
        finish_parallelism(v, m, n, dev, batch)
        v.traffic = dram_traffic(m, n, k, cfg, elem_bytes, batch)
        v.k_loop = k
        out.append(v)
    out.sort(key=lambda x: rank_key(x, dev))
    return out


def plan(m: int, n: int, k: int, dev: Optional[DeviceModel] = None, batch: int = 1,
         elem_bytes: int = 2, instrs: Optional[Sequence[str]] = None,
         regs: Optional[dict] = None) -> Tuple[Optional[Verdict], int]:
    dev = dev or device_gfx950()
    instrs = instrs or [s for s, _ in dev.instr_shapes]
    res = sweep(m, n, k, dev, instrs, batch, elem_bytes, regs)
    return (res[0] if res else None), len(res)


def conv_k(channels: int, taps: int, block_k: int) -> int:
    """K of a convolution's implicit GEMM as a tile with K step block_k
    computes it: each of the taps (kh * kw) runs over the channels padded up
    to a whole number of K steps."""
    return taps * _ceil_div(channels, block_k) * block_k


def sweep_conv(cout: int, pixels: int, channels: int, taps: int, dev: Optional[DeviceModel] = None,
               elem_bytes: int = 2, splits: int = 1) -> List[Verdict]:
    """The gfx950 sweep for a convolution computed as a GEMM (the Tiling page:
    M = output channels, N = output pixels, K = channels * kh * kw), where K
    depends on the candidate: conv_k(channels, taps, block_k).  Each
    candidate is finished (C4, C0) and ranked (rank_key) with its own K; the
    enumeration order is the GEMM sweep's.  splits > 1: the problem each of
    that many K ranges is, `splits` GEMMs (a batch) of K = ceil(conv_k /
    splits), a K step longer than that K being skipped as in sweep."""
    dev = dev or device_gfx950()
    assert dev.ranking != "pages"
    instrs = [s for s, _ in dev.instr_shapes]
    smallest = min(GFX950_SPACE["bk"])
    out = []
    for cfg in candidates(dev, 1 << 62, instrs):
        k = _ceil_div(conv_k(channels, taps, cfg.block_k), splits)
        if cfg.block_k > max(k, smallest):
            continue
        v = evaluate(cfg, dev, elem_bytes=elem_bytes)
        if not v.feasible:
            continue
        finish_parallelism(v, cout, pixels, dev, splits)
        v.traffic = dram_traffic(cout, pixels, k, cfg, elem_bytes, splits)
        v.k_loop = k
        out.append(v)
    out.sort(key=lambda x: rank_key(x, dev))
    return out


# ---------------------------------------------------------------------------
# Split K (C4's idle warning: fewer tiles than cores): the K loop cut into S
# ranges computed by separate blocks into fp32 partial sums, added up by a
# second pass.
# ---------------------------------------------------------------------------

SPLIT_CANDIDATES = (1, 2, 3, 4, 6, 8, 12, 16)


def split_ranges(k: int, s: int, block_k: int) -> int:
    """Ranges a kernel cutting K into S parts of whole K steps gets: each
    range ceil(K / S) rounded up to a multiple of block_k, the last one the
    rest."""
    if k == 0 or s <= 1:
        return 1
    per = _ceil_div(_ceil_div(k, s), block_k) * block_k
    return _ceil_div(k, per)


def splitk_total(t_s: int, s: int, batch: int, m: int, n: int, elem_bytes: int, dev: DeviceModel) -> Fraction:
    """The busiest CU's time with S ranges: T_S (busiest_core_time of the
    split problem's tile) plus, for S > 1, the partial sums -- S fp32 copies
    of the output, each written once and read once, 8 * S * batch * M * N
    bytes spread over the cores, each byte costing split_byte_cost bytes of
    streamed panel (elem_bytes per element) -- and the reduction launch."""
    t = Fraction(t_s)
    if s > 1:
        t += Fraction(8 * s * batch * m * n * dev.split_byte_cost, elem_bytes * dev.cores) + dev.launch_cost_k
    return t


def splitk_plan(m: int, n: int, k: int, dev: Optional[DeviceModel] = None, batch: int = 1, elem_bytes: int = 2,
                splits: int = 0) -> Tuple[int, Verdict]:
    """The split count and the tile: for each S of SPLIT_CANDIDATES (or only
    `splits` when > 0), the plan of the problem one range is (batch * S
    GEMMs of M x N x ceil(K / S)); S > 1 is kept only if that tile's K steps
    cut K into exactly S ranges; the least splitk_total wins, the smaller S
    on a tie."""
    dev = dev or device_gfx950()
    instrs = [s for s, _ in dev.instr_shapes]
    best = None
    for s in ((splits,) if splits else SPLIT_CANDIDATES):
        res = sweep(m, n, _ceil_div(k, s), dev, instrs, batch=batch * s, elem_bytes=elem_bytes)
        if not res:
            continue
        v = res[0]
        if not splits and s > 1 and split_ranges(k, s, v.config.block_k) != s:
            continue
        total = splitk_total(busiest_core_time(v, dev), s, batch, m, n, elem_bytes, dev)
        if best is None or total < best[0]:
            best = (total, s, v)
    if best is None:
        raise ValueError("no feasible tile")
    return best[1], best[2]


def conv_splitk_plan(cout: int, pixels: int, channels: int, taps: int, dev: Optional[DeviceModel] = None,
                     elem_bytes: int = 2, splits: int = 0) -> Tuple[int, Verdict]:
    """splitk_plan for a convolution's implicit GEMM, each candidate's K being
    conv_k(channels, taps, block_k) (sweep_conv)."""
    dev = dev or device_gfx950()
    best = None
    for s in ((splits,) if splits else SPLIT_CANDIDATES):
        res = sweep_conv(cout, pixels, channels, taps, dev, elem_bytes, splits=s)
        if not res:
            continue
        v = res[0]
        if not splits and s > 1 and split_ranges(conv_k(channels, taps, v.config.block_k), s, v.config.block_k) != s:
            continue
        total = splitk_total(busiest_core_time(v, dev), s, 1, cout, pixels, elem_bytes, dev)
        if best is None or total < best[0]:
            best = (total, s, v)
    if best is None:
        raise ValueError("no feasible tile")
    return best[1], best[2]


# ---------------------------------------------------------------------------
# Text report in the pages' format (used to compare with their printed output)
# ---------------------------------------------------------------------------


def sweep_rows(results: Sequence[Verdict], topk: int) -> List[str]:
    rows = []
    for v in results[:topk]:
        c = v.config
        rows.append(" ".join([str(c.block_m), str(c.block_n), str(c.block_k), str(c.stages), str(c.threads),
                              f"{float(v.traffic) / 1e6:.1f}", f"{v.smem_total / 1024:.1f}",
                              str(v.regs_per_thread), str(v.blocks_per_core), str(v.waves),
                              f"{float(v.fill) * 100:.0f}%", v.binding]))
    return rows


def sweep_summary(results: Sequence[Verdict]) -> dict:
    best = round_half_even(results[0].traffic) if results else 0
    tied = sum(1 for v in results if round_half_even(v.traffic) == best)
    best_fill = max((v.fill for v in results), default=Fraction(0))
    return {"feasible": len(results), "tied": tied, "best_fill_pct": f"{float(best_fill) * 100:.0f}%"}


def diagnose_lines(v: Verdict) -> List[str]:
    c = v.config
    lines = [
        f"C1 shared/stage {v.smem_per_stage / 1024:.1f} KB -> total {v.smem_total / 1024:.1f} KB",
        f"C2 accumulators {v.accum_per_thread}/thread -> {v.regs_per_thread} regs/thread (warp-rounded),"
        f" {v.regs_per_block} regs/block",
        f"occupancy: regs -> {v.blocks_by_regs} blk/SM, smem -> {v.blocks_by_smem},"
        f" threads -> {v.blocks_by_threads} => {v.blocks_per_core} blk/SM",
        f"C4 grid {v.grid} tiles -> {v.waves} wave(s), last wave {float(v.fill) * 100:.1f}% full",
    ]
    lines += [f"FAIL {m}" for m in v.messages]
    lines += [f"warn {w}" for w in v.warn_text]
    if v.feasible:
        lines.append("OK all four constraints satisfied")
    return lines


def diagnose(cfg: TileConfig, dev: DeviceModel, m: int, n: int, batch: int = 1) -> Verdict:
    v = evaluate(cfg, dev)
    finish_parallelism(v, m, n, dev, batch)
    return v


__all__ = ["DeviceModel", "TileConfig", "Verdict", "device_pages", "device_gfx950", "evaluate",
           "finish_parallelism", "dram_traffic", "round_half_even", "sweep", "plan", "rank_key",
           "sweep_rows", "sweep_summary", "diagnose_lines", "diagnose", "candidates", "WAVE_GRIDS",
           "busiest_core_time", "conv_k", "sweep_conv", "splitk_plan", "conv_splitk_plan", "split_ranges",
           "splitk_total", "SPLIT_CANDIDATES", "GFX950_STEP_COST_K", "GFX950_TILE_COST_K",
           "replace"]
