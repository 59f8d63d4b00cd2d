"""Pins of the planner oracle (C0..C4, sweep) to what the pages fix.

Pages-mode must reproduce the output the README page prints for its own
commands; the gfx950 model is pinned with closed forms worked by hand.
"""
import os
from fractions import Fraction

import pytest

from oracle import planner as P
from oracle import intensity as I

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        return [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]


def test_pages_sweep_matches_readme_printout():
    gold = _lines("readme_sweep_topk8.txt")
    dev = P.device_pages()
    res = P.sweep(4096, 4096, 4096, dev, ["wgmma"])
    summ = P.sweep_summary(res)
    rows = P.sweep_rows(res, 8)
    want_rows = [l.split()[1:] for l in gold if l.startswith("row ")]
    for i, w in enumerate(want_rows):
        assert rows[i].split() == w
    for l in gold:
        key, *val = l.split()
        if key == "feasible":
            assert summ["feasible"] == int(val[0])
        elif key == "tied":
            assert summ["tied"] == int(val[0])
        elif key == "best_fill":
            assert summ["best_fill_pct"] == val[0]


def test_pages_diagnose_overbudget_matches_readme_printout():
    gold = _lines("readme_diagnose_overbudget.txt")
    v = P.diagnose(P.TileConfig(256, 256, 64, 4, 256, "wgmma"), P.device_pages(), 4096, 4096)
    got = P.diagnose_lines(v)
    assert got[0].split() == gold[0].split()
    assert got[1].split() == gold[1].split()
    assert got[2].split() == gold[2].split()
    fails = [l for l in got if l.startswith("FAIL")]
    assert [f.split() for f in fails] == [g.split() for g in gold if g.startswith("FAIL")]
    assert v.failures == ["C1", "C2", "OCC0"]
    # blocks/SM = 0 leaves one resident slot, so every tile is its own wave
    assert (v.grid, v.waves, v.fill) == (256, 256, Fraction(1))


def test_pages_other_commands_cross_checked():
    """Outputs of the README's other commands, not printed on the pages: they
    were obtained by executing the tile_decision.py page's listing as printed
    (an implementation independent of this oracle)."""
    dev = P.device_pages()
    v = P.diagnose(P.TileConfig(128, 256, 64, 3, 256, "wgmma"), dev, 4096, 4096)
    assert v.feasible and v.binding == "smem"
    assert (v.smem_per_stage, v.smem_total, v.regs_per_thread, v.regs_per_block) == (49152, 147456, 128, 32768)
    assert (v.blocks_by_regs, v.blocks_by_smem, v.blocks_by_threads, v.blocks_per_core) == (2, 1, 8, 1)
    assert (v.grid, v.waves, f"{float(v.fill) * 100:.1f}") == (512, 4, "87.9")
    s = P.sweep_summary(P.sweep(4096, 4096, 4096, dev, ["mma"]))
    assert (s["feasible"], s["tied"], s["best_fill_pct"]) == (813, 8, "94%")
    a100 = P.device_pages(sm_count=108, smem_kb=164)
    res = P.sweep(4096, 4096, 4096, a100, ["wgmma"])
    s = P.sweep_summary(res)
    assert (s["feasible"], s["tied"], s["best_fill_pct"]) == (435, 7, "96%")
    assert (res[0].waves, f"{float(res[0].fill) * 100:.0f}%") == (3, "37%")


def test_tiling_page_constraint_examples():
    """Constraint analysis of the Tiling page: shared-memory bytes per config
    and the A100 block count; the register estimate with its overhead."""
    for l in _lines("tiling_numbers.txt"):
        key, *v = l.split()
        if key == "smem":
            bm, bn, bk, eb, st, want = map(int, v)
            ver = P.evaluate(P.TileConfig(bm, bn, bk, st, 256, "mma"), P.device_pages(), elem_bytes=eb)
            assert ver.smem_total == want
        elif key == "smem_blocks_a100":
            kb, tile_kb, want = map(int, v)
            assert kb // tile_kb == want
            a100 = P.device_pages(sm_count=108, smem_kb=164)
            big = P.evaluate(P.TileConfig(256, 256, 64, 3, 256, "mma"), a100)
            assert "C1" in big.failures           # 192 KB does not fit 164 KB
        elif key == "regs":
            bm, bn, thr, overhead, want = map(int, v)
            g = P.device_gfx950()
            assert g.reg_overhead == overhead
            assert -(-bm * bn // thr) + overhead == want


def test_traffic_closed_forms():
    c = P.TileConfig(256, 256, 16, 2, 512, "wgmma")
    assert P.dram_traffic(4096, 4096, 4096, c) == 2 * 4096 ** 3 * Fraction(2, 256) + 2 * 4096 ** 2
    assert P.round_half_even(P.dram_traffic(4096, 4096, 4096, c)) == 1107296256
    c128 = P.TileConfig(128, 128, 32, 2, 256, "mfma32")
    t = P.dram_traffic(4096, 4096, 4096, c128)
    assert t == 2181038080
    # link to the Tiling page's intensity: without the C write, 2MNK / traffic
    # is the tiled intensity 2*BM*BN/((BM+BN)*elem_bytes) = 64 FLOP/B
    assert Fraction(2 * 4096 ** 3) / (t - 2 * 4096 ** 2) == I.intensity_tiled(128, 128, 4096) == 64
    # a batch multiplies the whole expression
    c64 = P.TileConfig(64, 256, 32, 2, 256, "mfma32")
    assert P.dram_traffic(3000, 5000, 2048, c64, batch=4) == 4 * P.dram_traffic(3000, 5000, 2048, c64)
    assert P.round_half_even(Fraction(5, 2)) == 2 and P.round_half_even(Fraction(7, 2)) == 4
    assert P.round_half_even(Fraction(-5, 2)) == -2 and P.round_half_even(Fraction(11, 4)) == 3


def test_grid_is_not_symmetric_in_block_dims():
    g = P.device_gfx950()
    v = P.finish_parallelism(P.evaluate(P.TileConfig(64, 256, 32, 2, 256, "mfma32"), g), 3000, 5000, g, batch=4)
    assert v.grid == 4 * 47 * 20
    v2 = P.finish_parallelism(P.evaluate(P.TileConfig(256, 64, 32, 2, 256, "mfma32"), g), 3000, 5000, g, batch=4)
    assert v2.grid == 4 * 12 * 79


def test_gfx950_closed_forms():
    g = P.device_gfx950()
    v = P.evaluate(P.TileConfig(256, 256, 64, 2, 256, "mfma32"), g)
    assert v.feasible and v.smem_total == 131072 and v.accum_per_thread == 256
    assert v.regs_per_thread == 288                      # 256 accumulators + 32 overhead
    assert v.blocks_by_regs == 1                         # floor(512/288) = 1 wave/SIMD, 4 waves/block
    assert v.blocks_by_smem == 1 and v.blocks_by_threads == 8 and v.blocks_per_core == 1
    assert v.binding == "regs"
    v = P.evaluate(P.TileConfig(256, 256, 64, 3, 256, "mfma32"), g)
    assert v.failures == ["C1", "OCC0"] and v.smem_total == 196608   # no block fits either
    v = P.evaluate(P.TileConfig(256, 256, 32, 2, 128, "mfma32"), g)
    assert "C2" in v.failures and v.accum_per_thread == 512
    v = P.evaluate(P.TileConfig(256, 256, 32, 2, 512, "mfma32"), g)
    assert v.regs_per_thread == 160 and v.blocks_by_regs == (4 * (512 // 160)) // 8 == 1
    v = P.evaluate(P.TileConfig(64, 64, 32, 2, 256, "mfma32"), g)
    assert v.accum_per_thread == 16 and v.regs_per_thread == 48
    assert v.blocks_by_regs == (4 * 8) // 4 == 8 and v.blocks_by_smem == 163840 // 16384 == 10
    assert v.blocks_by_threads == 8 and v.binding == "regs"
    # wave grid: 8 waves split 2 x 4; a 64-wide block cannot hold 4 columns of 32-wide MFMA tiles
    assert "C3_WAVEGRID" in P.evaluate(P.TileConfig(64, 64, 32, 2, 512, "mfma32"), g).failures
    assert P.evaluate(P.TileConfig(64, 64, 64, 2, 512, "mfma16"), g).feasible
    # mfma16 needs block_K a multiple of 32
    assert P.evaluate(P.TileConfig(128, 128, 16, 2, 256, "mfma16"), g).failures == ["C3_K"]
    # C4 at the headline shape: 256 tiles of 256x256 on 256 CUs, one full wave
    v = P.finish_parallelism(P.evaluate(P.TileConfig(256, 256, 64, 2, 256, "mfma32"), g), 4096, 4096, g)
    assert (v.grid, v.waves, v.fill, v.warnings) == (256, 1, Fraction(1), [])
    v = P.finish_parallelism(P.evaluate(P.TileConfig(128, 128, 64, 2, 256, "mfma32"), g), 6272, 256, g)
    assert v.grid == 98 and v.warnings == ["idle"]


def test_tail_warning_threshold_exact():
    g = P.device_gfx950()
    v = P.evaluate(P.TileConfig(256, 256, 64, 2, 256, "mfma32"), g)    # 1 block/CU -> 256 resident
    P.finish_parallelism(v, 256 * 16, 256 * 24, g)                  # 384 tiles: fill 128/256 = 1/2 -> no warn
    assert v.waves == 2 and v.fill == Fraction(1, 2) and v.warnings == []
    v = P.evaluate(P.TileConfig(256, 256, 64, 2, 256, "mfma32"), g)
    P.finish_parallelism(v, 256 * 1, 256 * 383, g)                  # 383 tiles: fill 127/256 -> tail
    assert v.warnings == ["tail"]


def test_sweep_is_stable_and_sorted():
    g = P.device_gfx950()
    res = P.sweep(4096, 4096, 4096, g, ["mfma32", "mfma16"])
    keys = [P.rank_key(v, g) for v in res]
    assert keys == sorted(keys)
    order = {c: i for i, c in enumerate(P.candidates(g, 4096, ["mfma32", "mfma16"]))}
    for a, b in zip(res, res[1:]):
        if P.rank_key(a, g) == P.rank_key(b, g):
            assert order[a.config] < order[b.config]
    best = res[0].config
    assert (best.block_m, best.block_n) == (256, 256)
    # every feasible candidate was kept and nothing infeasible slipped in
    n_feasible = sum(1 for c in P.candidates(g, 4096, ["mfma32", "mfma16"]) if P.evaluate(c, g).feasible)
    assert n_feasible == len(res)


def test_bk_larger_than_k_is_skipped():
    g = P.device_gfx950()
    res = P.sweep(64, 64, 32, g, ["mfma32"])
    assert res and all(v.config.block_k <= 32 for v in res)


def test_gfx950_load_rule_per_wave():
    """64x64x16 fp16: each operand tile is 2 KiB = two 1 KiB wave loads, so a
    block of 2 waves passes and a block of 4 waves (0.5 load each) fails."""
    g = P.device_gfx950()
    assert "C3_LOAD" not in P.evaluate(P.TileConfig(64, 64, 16, 2, 128, "mfma32"), g).failures
    assert "C3_LOAD" in P.evaluate(P.TileConfig(64, 64, 16, 2, 256, "mfma32"), g).failures
    assert "C3_LOAD" not in P.evaluate(P.TileConfig(64, 64, 32, 2, 256, "mfma32"), g).failures
    assert "C3_LOAD" in P.evaluate(P.TileConfig(64, 128, 16, 2, 512, "mfma16"), g).failures


def test_short_k_keeps_the_shortest_step():
    g = P.device_gfx950()
    res = P.sweep(64, 64, 8, g, ["mfma32"])
    assert res and {v.config.block_k for v in res} == {16}
    assert P.sweep(64, 64, 0, g, ["mfma32"])
    pages = P.sweep(4096, 4096, 8, P.device_pages(), ["wgmma"])
    assert {v.config.block_k for v in pages} == {16}


def test_gfx950_rank_prefers_occupancy_then_bigger_k_step():
    """4096^3: every 256x256 tile streams 512 panel rows through its CU (one
    tile per CU) and ties on C0; the 64-deep K step wins, then 512 threads
    (8 resident waves against 4), and the 16x16x32 shape wins the tie with
    32x32x16 by coming first."""
    g = P.device_gfx950()
    res = P.sweep(4096, 4096, 4096, g, [s for s, _ in g.instr_shapes])
    c = res[0].config
    assert (c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr) == (256, 256, 64, 2, 512, "mfma16")
    # one tile per CU, 256 + 256 panel rows, 64 K steps of 64 + 22, one round of 900
    assert (g.step_cost_k, g.tile_cost_k, g.target_waves_per_simd) == (22, 900, 4)
    assert P.rank_key(res[0], g)[:1] == (1 * 512 * 64 * (64 + 22) + 1 * 512 * 900,) == (3278848,)
    # 8 resident waves on 4 SIMDs: 2 per SIMD, 2 below the target of 4 -> 8 waves off
    assert P.rank_key(res[0], g)[4:6] == (8, -8)
    d = res[1].config    # the 32x32x16 twin ties on every key and follows it
    assert (d.block_m, d.block_n, d.block_k, d.stages, d.threads, d.instr) == (256, 256, 64, 2, 512, "mfma32")


def test_gfx950_round_cost_crossover_and_waves_target():
    """K = 200 on 4096 x 4096, worked by hand.  256x256x64 (512 threads):
    256 tiles, one per CU, 4 steps of 64 + 22 over 512 panel rows, one round:
    T = 512 * 4 * 86 + 512 * f.  128x128x32 (256 threads): 1024 tiles, W = 4,
    all resident (LDS 32 KiB -> 5 blocks), 7 steps of 32 + 22 over 256 rows,
    one round: T = 4 * 256 * 7 * 54 + 256 * f.  They cross at
    256 * f = 387072 - 176128, f = 824.  Its 512-thread twin has the same T
    and residency (4 blocks of 8 waves: 8 per SIMD) and is 16 waves off a
    target of 4 per SIMD against 0: the target decides; without it the twin's
    32 waves win."""
    g = P.device_gfx950()
    ins = [s for s, _ in g.instr_shapes]

    def time_of(dev, bm, bn, bk, thr):
        res = {v.config: v for v in P.sweep(4096, 4096, 200, dev, ins)}
        return P.rank_key(res[P.TileConfig(bm, bn, bk, 2, thr, "mfma16")], dev)

    for f in (823, 824, 825, 900):
        d = P.replace(g, tile_cost_k=f)
        big, small = time_of(d, 256, 256, 64, 512)[0], time_of(d, 128, 128, 32, 256)[0]
        assert (big, small) == (176128 + 512 * f, 387072 + 256 * f)
        assert (big < small, big == small) == (f < 824, f == 824)
    first = P.sweep(4096, 4096, 200, g, ins)[0].config
    assert (first.block_m, first.block_n, first.block_k, first.threads) == (128, 128, 32, 256)
    k256, k512 = time_of(g, 128, 128, 32, 256), time_of(g, 128, 128, 32, 512)
    assert k256[:4] == k512[:4] == (617472, k256[1], -32, -4)
    assert (k256[4:6], k512[4:6]) == ((0, -16), (16, -32))
    g0 = P.replace(g, target_waves_per_simd=0)
    first0 = P.sweep(4096, 4096, 200, g0, ins)[0].config
    assert (first0.block_m, first0.block_n, first0.block_k, first0.threads) == (128, 128, 32, 512)


def test_gfx950_busiest_core_time_closed_forms():
    """T = W*(BM+BN)*n*(BK+s) + R*(BM+BN)*f, worked by hand (W tiles on the
    busiest CU, u = min(blocks/CU, W) resident, R = ceil(W/u) rounds,
    n = ceil(K/BK) steps) with the cost parameters s and f set explicitly."""
    g0 = P.replace(P.device_gfx950(), step_cost_k=0, tile_cost_k=0)
    ev = lambda bm, bn, M, N, b=1, bk=64, st=2, thr=256: P.finish_parallelism(
        P.evaluate(P.TileConfig(bm, bn, bk, st, thr, "mfma32"), g0), M, N, g0, b)
    T = P.busiest_core_time
    # s = f = 0: the busiest CU's C0 panel traffic, (BM + BN) * K per tile.
    # conv workload as a GEMM (256 x 6272, K = 2304): 128x64 -> 196 tiles, at
    # most one per CU; 64x64 -> 392 tiles, two on some CUs
    assert T(ev(128, 64, 256, 6272), g0, 2304) == 1 * 192 * 2304
    assert T(ev(64, 64, 256, 6272), g0, 2304) == 2 * 128 * 2304
    assert T(ev(256, 256, 256, 6272), g0, 2304) == 1 * 512 * 2304      # 25 tiles
    # ragged batch: 4 x 12 x 20 = 960 tiles of 256x256 -> 4 per CU; K = 2048
    assert T(ev(256, 256, 3000, 5000, 4), g0, 2048) == 4 * 512 * 2048
    assert T(ev(128, 128, 3000, 5000, 4), g0, 2048) == 15 * 256 * 2048   # 3840 tiles
    # a ragged K runs whole steps: K = 200 with BK = 64 -> 4 steps = 256
    assert T(ev(256, 256, 4096, 4096), g0, 200) == 512 * 256
    assert T(ev(256, 256, 4096, 4096, bk=16), g0, 200) == 512 * 13 * 16
    # step cost s = 22: each step costs BK + 22
    g1 = P.replace(g0, step_cost_k=22)
    v = ev(256, 256, 4096, 4096)
    assert T(v, g1, 200) == 512 * 4 * (64 + 22) == 176128
    assert T(v, g1, 4096) == 512 * 64 * 86 == 2818048
    # round cost f = 100: 128x128x64 at 2 stages holds 2 blocks per CU (LDS
    # 64 KiB of 160; registers: 64 + 32 = 96 per lane -> 5 waves per SIMD,
    # 5 blocks of 4 waves); 4096^2 -> 1024 tiles, W = 4, u = 2, R = 2
    g2 = P.replace(g0, step_cost_k=22, tile_cost_k=100)
    v = ev(128, 128, 4096, 4096)
    assert (v.blocks_per_core, v.grid) == (2, 1024)
    assert T(v, g2, 4096) == 4 * 256 * 64 * 86 + 2 * 256 * 100
    v = ev(256, 256, 4096, 4096)
    assert T(v, g2, 4096) == 512 * 64 * 86 + 1 * 512 * 100
    # no tiles (N = 0): no time
    assert T(ev(256, 256, 4096, 0), g2, 4096) == 0


def test_gfx950_conv_and_small_shape_choices():
    g = P.device_gfx950()
    ins = [s for s, _ in g.instr_shapes]
    c = P.sweep(256, 6272, 2304, g, ins)[0].config
    # 128x64 and 64x128 tie on every key but order: the taller tile comes first.  Its 196 tiles leave every CU
    # one block at most, so the LDS room for 3 blocks of a 2-stage ring buys nothing and the 4-stage ring wins
    assert (c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr) == (128, 64, 64, 4, 512, "mfma16")
    v = P.sweep(256, 6272, 2304, g, ins)[0]
    assert v.blocks_per_core == 1 and P.rank_key(v, g)[3:7] == (-1, 8, -8, -4)
    two = P.finish_parallelism(P.evaluate(P.TileConfig(128, 64, 64, 2, 512, "mfma16"), g), 256, 6272, g)
    assert two.blocks_per_core == 3 and P.rank_key(two, g)[3:7] == (-1, 8, -8, -2)   # 3 resident, 1 usable
    c = P.sweep(256, 256, 256, g, ins)[0].config
    assert (c.block_m, c.block_n) == (64, 64)     # 16 tiles over 16 CUs beat one 256x256 tile
    c = P.sweep(3000, 5000, 2048, g, ins, batch=4)[0].config
    assert (c.block_m, c.block_n, c.block_k, c.stages, c.threads) == (256, 256, 64, 2, 512)


def test_pages_register_granule_closed_form():
    """tile_decision.py page, C2: 256 registers per warp of 32 threads, so
    8 accumulators per thread take 8 registers and 9 take 16."""
    dev = P.device_pages()
    v = P.evaluate(P.TileConfig(32, 32, 16, 2, 128, "mma"), dev)
    assert (v.accum_per_thread, v.regs_per_thread, v.regs_per_block, v.blocks_by_regs) == (8, 8, 1024, 64)
    v = P.evaluate(P.TileConfig(48, 24, 16, 2, 128, "simt"), dev)      # 1152 / 128 = 9 accumulators
    assert (v.accum_per_thread, v.regs_per_thread) == (9, 16)


def test_conv_sweep_pins():
    """The convolution's sweep, where each candidate computes
    K = taps * ceil(C / BK) * BK (the kernel pads a tap's channels to whole
    K steps):
    * K's closed forms (C = 3 and 96 over the gfx950 K steps);
    * with C a multiple of 64 every K step gives K = taps * C, and the plan's
      choice is the GEMM plan's (a 64-wide step);
    * the rank key's time term worked by hand for C = 3 and C = 96 at each K
      step, and the K step it makes the plan take."""
    assert [P.conv_k(3, 9, bk) for bk in (16, 32, 64)] == [144, 288, 576]
    assert [P.conv_k(96, 9, bk) for bk in (16, 32, 64)] == [864, 864, 1152]
    g = P.device_gfx950()
    ins = [s for s, _ in g.instr_shapes]
    for co, px, c, taps in [(256, 6272, 256, 9), (128, 3000, 64, 1), (96, 20000, 128, 25)]:
        conv = P.sweep_conv(co, px, c, taps)[0].config
        gemm = P.sweep(co, px, taps * c, g, ins)[0].config
        assert conv == gemm and conv.block_k == 64
    # First layer, 64 output channels over 8 x 112 x 112 pixels, C = 3, 3x3:
    # a 128x128 tile, 2 stages, 256 threads (mfma32 for every K step): grid
    # 1 x 784 tiles -> W = 4 on the busiest CU (784 / 256), all resident
    # (u = 4: 2 blocks by LDS at BK = 64 ... at most 4 useful), 256 panel rows.
    g = P.replace(P.device_gfx950(), step_cost_k=22, tile_cost_k=0)
    res = {v.config: v for v in P.sweep_conv(64, 8 * 112 * 112, 3, 9, dev=g)}
    keys = {bk: P.rank_key(res[P.TileConfig(128, 128, bk, 2, 256, "mfma32")], g)[0] for bk in (16, 32, 64)}
    assert keys == {16: 4 * 256 * 9 * (16 + 22), 32: 4 * 256 * 9 * (32 + 22), 64: 4 * 256 * 9 * (64 + 22)}
    assert keys == {16: 350208, 32: 497664, 64: 792576}
    # C = 96 (8 x 56 x 56 pixels, 128 output channels): BK = 16 and 32 both
    # pad nothing (K = 864) but 16 takes 54 steps against 27; BK = 64 pads
    # to 1152 in 18 steps.  Same tile: W = ceil(196 / 256) = 1.
    res = {v.config: v for v in P.sweep_conv(128, 8 * 56 * 56, 96, 9, dev=g)}
    keys = {bk: P.rank_key(res[P.TileConfig(128, 128, bk, 2, 256, "mfma32")], g)[0] for bk in (16, 32, 64)}
    assert keys == {16: 256 * 54 * 38, 32: 256 * 27 * 54, 64: 256 * 18 * 86}
    assert min(keys, key=keys.get) == 32
    # a round cost of f adds R * (BM + BN) * f to each (here R = 1 round of 256 panel rows)
    gf = P.replace(g, tile_cost_k=600)
    resf = {v.config: v for v in P.sweep_conv(128, 8 * 56 * 56, 96, 9, dev=gf)}
    assert {bk: P.rank_key(resf[P.TileConfig(128, 128, bk, 2, 256, "mfma32")], gf)[0] for bk in (16, 32, 64)} == \
        {bk: k + 256 * 600 for bk, k in keys.items()}


def test_conv_plan_without_step_cost_never_pads_more():
    """With the step cost set to zero, a candidate's K loop costs its padded
    K alone, and the time term is W * (BM + BN) * K(BK) with W independent of
    BK: the plan's K step is one of those that pad least for its tile shape
    (no BK with a smaller padded K is feasible for the same BM, BN,
    threads and instruction), whatever the channel count."""
    g0 = P.replace(P.device_gfx950(), step_cost_k=0, tile_cost_k=0)
    for c in (1, 3, 8, 20, 48, 72, 96, 100, 160, 200, 256, 333):
        best = P.sweep_conv(128, 8 * 28 * 28, c, 9, dev=g0)[0]
        b = best.config
        same_shape = [v for v in P.sweep_conv(128, 8 * 28 * 28, c, 9, dev=g0)
                      if (v.config.block_m, v.config.block_n, v.config.threads, v.config.instr)
                      == (b.block_m, b.block_n, b.threads, b.instr)]
        assert P.conv_k(c, 9, b.block_k) == min(P.conv_k(c, 9, v.config.block_k) for v in same_shape), c


def test_split_ranges_and_total_closed_forms():
    """split_ranges: each range ceil(K / S) rounded up to whole K steps, the
    last the rest; splitk_total: T_S + 8 S b M N c / (eb cores) + launch."""
    assert P.split_ranges(1000, 3, 64) == 3          # 334 -> 384 per range: 384, 384, 232
    assert P.split_ranges(200, 4, 64) == 4           # 50 -> 64: 64, 64, 64, 8
    assert P.split_ranges(100, 8, 64) == 2           # 13 -> 64: 64, 36 -- fewer ranges than asked
    assert P.split_ranges(4096, 16, 64) == 16 and P.split_ranges(4096, 12, 64) == 11   # 342 -> 384: 10 full + 256
    assert P.split_ranges(0, 8, 64) == 1 and P.split_ranges(5000, 1, 16) == 1
    g = P.device_gfx950()
    assert (g.split_byte_cost, g.launch_cost_k) == (6, 67000)
    assert P.splitk_total(1000, 1, 1, 512, 512, 2, g) == 1000
    assert P.splitk_total(1000, 4, 1, 512, 512, 2, g) == 1000 + 8 * 4 * 512 * 512 * 6 // (2 * 256) + 67000
    assert P.splitk_total(1000, 4, 1, 512, 512, 2, g) == 1000 + 98304 + 67000
    assert P.splitk_total(7, 3, 2, 100, 24, 2, g) == 7 + P.Fraction(8 * 3 * 2 * 100 * 24 * 6, 512) + 67000


def test_splitk_plan_extremes_and_structure():
    """With the split free of cost the plan takes the split that minimises the
    busiest CU's time; with a prohibitive cost it never splits; one 64x64
    tile over a long K (64 x 64 x 16384) shows both, worked by hand."""
    free = P.replace(P.device_gfx950(), split_byte_cost=0, launch_cost_k=0, tile_cost_k=0)
    # one tile per split: W = 1, 128 panel rows, ceil(16384 / S / 64) steps of 64 + 22: least at S = 16
    S, v = P.splitk_plan(64, 64, 16384, dev=free)
    assert S == 16 and (v.config.block_m, v.config.block_n, v.config.block_k) == (64, 64, 64)
    assert P.busiest_core_time(v, free) == 1 * 128 * 16 * 86
    costly = P.replace(P.device_gfx950(), split_byte_cost=10 ** 6)
    assert P.splitk_plan(64, 64, 16384, dev=costly)[0] == 1
    # the launch cost alone: a split whose time saving is below it is not taken
    launch_only = P.replace(free, launch_cost_k=10 ** 9)
    assert P.splitk_plan(64, 64, 16384, dev=launch_only)[0] == 1
    # a problem that fills the machine with one wave of tiles gains nothing from a split
    assert P.splitk_plan(4096, 4096, 4096)[0] == 1
    # C a multiple of 64: the convolution's split plan is the GEMM's for K = taps * C
    for co, px, c, taps in [(64, 4096, 128, 9), (128, 1000, 64, 1)]:
        Sc, vc = P.conv_splitk_plan(co, px, c, taps)
        Sg, vg = P.splitk_plan(co, px, taps * c)
        assert (Sc, vc.config) == (Sg, vg.config)
    # a fixed split count plans only that count
    S, v = P.splitk_plan(512, 512, 8192, splits=6)
    c = v.config
    assert S == 6 and v.grid == 6 * (512 // c.block_m) * (512 // c.block_n) and v.k_loop == -(-8192 // 6)
