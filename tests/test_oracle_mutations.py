"""The oracle's pins catch plausible mistakes: each test plants one mistake in
a copy of an oracle function (on the CPU) and checks that the pin it targets
then fails.  The real oracle is never modified."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import htile as H
from oracle import intensity as I
from oracle import planner as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        return [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]


def readme_sweep_pin(planner_mod) -> bool:
    gold = _lines("readme_sweep_topk8.txt")
    res = planner_mod.sweep(4096, 4096, 4096, planner_mod.device_pages(), ["wgmma"])
    summ = planner_mod.sweep_summary(res)
    rows = planner_mod.sweep_rows(res, 8)
    want = [l.split()[1:] for l in gold if l.startswith("row ")]
    ok = all(rows[i].split() == w for i, w in enumerate(want))
    ok &= summ["feasible"] == 459 and summ["tied"] == 8 and summ["best_fill_pct"] == "94%"
    return ok


def readme_diagnose_pin(planner_mod) -> bool:
    gold = _lines("readme_diagnose_overbudget.txt")
    v = planner_mod.diagnose(planner_mod.TileConfig(256, 256, 64, 4, 256, "wgmma"), planner_mod.device_pages(),
                             4096, 4096)
    got = planner_mod.diagnose_lines(v)
    return [l.split() for l in got[:3]] == [g.split() for g in gold[:3]] and \
        [f.split() for f in got if f.startswith("FAIL")] == [g.split() for g in gold if g.startswith("FAIL")]


def halo_pin(hw_tile) -> bool:
    lines = _lines("tiling_halo_example.txt")
    tiles = [list(map(int, l.split()[1:])) for l in lines if l.startswith("tile ")]
    ok = True
    for want in tiles:
        t = hw_tile(9, 3, 2, 1, 1, want[0], want[1])
        ok &= (t.in_start, t.in_end, t.in_span, t.pt, t.pb) == tuple(want[2:7]) and t.halo == 1
    return ok


def granule_pin(planner_mod) -> bool:
    """tile_decision.py page, C2: registers are handed out 256 per warp of 32,
    i.e. 8 per thread: 8 accumulators per thread stay 8 registers."""
    v = planner_mod.evaluate(planner_mod.TileConfig(32, 32, 16, 2, 128, "mma"), planner_mod.device_pages())
    return v.accum_per_thread == 8 and v.regs_per_thread == 8 and v.blocks_by_regs == 65536 // (8 * 128)


def window_pin(hw_tile) -> bool:
    """Brute force: the padded slice reproduces every output row's window."""
    for Hh in range(1, 10):
        for kh, sh, pt, d in ((3, 2, 1, 1), (3, 1, 2, 1), (2, 3, 0, 1), (3, 1, 1, 2)):
            if pt >= H.window_rows(kh, d):
                continue
            OHt = H.out_size(Hh, kh, sh, pt, pt, d)
            for toh in range(1, OHt + 1):
                for o0 in range(0, OHt, toh):
                    t = hw_tile(Hh, kh, sh, pt, d, o0, min(o0 + toh, OHt))
                    rows_in = min(t.in_end, Hh) - t.in_start
                    if (t.pt + rows_in + t.pb - H.window_rows(kh, d)) // sh + 1 != t.o1 - t.o0:
                        return False
                    if t.in_start - t.pt != t.o0 * sh - pt:
                        return False
    return True


def test_real_oracle_passes_every_pin():
    assert readme_sweep_pin(P) and readme_diagnose_pin(P) and halo_pin(H.hw_tile)
    assert granule_pin(P) and window_pin(H.hw_tile)


def test_dropped_c_write_term_in_c0_is_caught(monkeypatch):
    monkeypatch.setattr(P, "dram_traffic", lambda m, n, k, cfg, elem_bytes=2, batch=1:
                        batch * elem_bytes * m * n * k * (Fraction(1, cfg.block_n) + Fraction(1, cfg.block_m)))
    assert not readme_sweep_pin(P)


def test_wrong_register_granule_is_caught(monkeypatch):
    real = P.device_pages
    monkeypatch.setattr(P, "device_pages", lambda sm_count=132, smem_kb=228:
                        P.replace(real(sm_count, smem_kb), reg_granule_per_lane=16))
    assert not granule_pin(P)


def test_missing_per_block_reserve_is_caught(monkeypatch):
    real = P.device_pages
    monkeypatch.setattr(P, "device_pages", lambda sm_count=132, smem_kb=228:
                        P.replace(real(sm_count, smem_kb), onchip_per_block_max=smem_kb * 1024))
    assert not readme_diagnose_pin(P)


def test_smem_counting_one_operand_is_caught(monkeypatch):
    real_eval = P.evaluate

    def wrong(cfg, dev, elem_bytes=2, accum_bytes=4):
        v = real_eval(cfg, dev, elem_bytes, accum_bytes)
        v.smem_per_stage = cfg.block_m * cfg.block_k * elem_bytes
        v.smem_total = v.smem_per_stage * cfg.stages
        return v
    monkeypatch.setattr(P, "evaluate", wrong)
    assert not readme_diagnose_pin(P)


@pytest.mark.parametrize("mistake", ["in_end_no_plus_one", "halo_sign", "pt_no_clamp", "pb_uses_in_start"])
def test_htile_mistakes_are_caught(mistake):
    def hw_tile(Hh, kh, sh, pt, d, o0, o1):
        t = H.hw_tile(Hh, kh, sh, pt, d, o0, o1)
        if mistake == "in_end_no_plus_one":
            e = t.in_end - 1
            return H.HSlice(t.o0, t.o1, t.in_start, e, e - t.in_start, t.pt, max(0, e - Hh), t.halo)
        if mistake == "halo_sign":
            return H.HSlice(t.o0, t.o1, t.in_start, t.in_end, t.in_span, t.pt, t.pb, sh - H.window_rows(kh, d))
        if mistake == "pt_no_clamp":
            return H.HSlice(t.o0, t.o1, t.in_start, t.in_end, t.in_span, pt - o0 * sh, t.pb, t.halo)
        return H.HSlice(t.o0, t.o1, t.in_start, t.in_end, t.in_span, t.pt, max(0, t.in_start - Hh), t.halo)
    assert not (halo_pin(hw_tile) and window_pin(hw_tile))


def test_naive_intensity_with_one_operand_is_caught():
    wrong = Fraction(I.flops_per_element(4096), 4096 * 2)  # counts only the row of A
    assert wrong != Fraction(1, 2)
    wrong_tiled = Fraction(128 * 128 * 2 * 4096, 128 * 4096 * 2)  # counts only the A panel
    assert wrong_tiled != 64


def test_transposed_operand_in_gemm_is_caught():
    """The numpy cross-check of the GEMM oracle fails for a transposed B."""
    from oracle import gemm_conv as G
    rng = np.random.default_rng(3)
    A = rng.integers(-2, 3, (13, 17)).astype(np.float64)
    B = rng.integers(-2, 3, (17, 13)).astype(np.float64)
    C, _ = G.gemm(A, B)
    # a transposed use of the operands is a different product of these
    # non-symmetric inputs, so the cross-check would flag it
    assert not np.array_equal(C, B.T @ A.T)
    assert np.array_equal(C, A @ B)


def test_conv_padding_on_wrong_side_is_caught():
    """Brute force with the pad applied only at the bottom differs from the
    oracle's symmetric padding on the first output row."""
    from oracle import gemm_conv as G
    rng = np.random.default_rng(4)
    x = rng.integers(-2, 3, (1, 2, 7, 6)).astype(np.float64)
    w = rng.integers(-2, 3, (3, 2, 3, 3)).astype(np.float64)
    y, _ = G.conv2d(x, w, (1, 1), (1, 1), (1, 1))
    xp = np.pad(x, ((0, 0), (0, 0), (0, 2), (1, 1)))   # both H pad rows at the bottom
    wrong = np.zeros_like(y)
    for co in range(3):
        for oh in range(y.shape[2]):
            for ow in range(y.shape[3]):
                wrong[0, co, oh, ow] = np.sum(xp[0, :, oh:oh + 3, ow:ow + 3] * w[co])
    assert not np.array_equal(wrong, y)


def _fails(fn) -> bool:
    try:
        fn()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("mistake", ["rounds_as_tiles", "no_step_cost", "k_not_in_whole_steps", "panel_one_side"])
def test_time_term_mistakes_are_caught(monkeypatch, mistake):
    """The hand-worked closed forms of the gfx950 time term catch a round cost
    charged per tile instead of per round, a dropped step cost, a K loop not
    cut into whole steps, and a panel counting one operand only."""
    import test_oracle_planner as T

    def wrong(v, dev, k_loop=None):
        c = v.config
        k = v.k_loop if k_loop is None else k_loop
        w = -(-v.grid // dev.cores)
        if w == 0:
            return 0
        u = min(v.blocks_per_core, w)
        rounds = -(-w // u)
        steps = -(-k // c.block_k)
        panel = c.block_m + c.block_n
        step_cost = dev.step_cost_k
        if mistake == "rounds_as_tiles":
            rounds = w
        elif mistake == "no_step_cost":
            step_cost = 0
        elif mistake == "k_not_in_whole_steps":
            return w * panel * k + rounds * panel * dev.tile_cost_k
        elif mistake == "panel_one_side":
            panel = c.block_m
        return w * panel * steps * (c.block_k + step_cost) + rounds * panel * dev.tile_cost_k
    monkeypatch.setattr(P, "busiest_core_time", wrong)
    assert _fails(T.test_gfx950_busiest_core_time_closed_forms)


@pytest.mark.parametrize("mistake", ["partials_counted_for_two_ranges", "total_without_launch", "ranges_floor"])
def test_split_mistakes_are_caught(monkeypatch, mistake):
    """The split pins catch partial-sum traffic that stops growing past two
    ranges, a dropped reduction launch, and ranges cut by floor instead of by
    whole K steps."""
    import test_oracle_planner as T
    real_total, real_ranges = P.splitk_total, P.split_ranges
    if mistake == "partials_counted_for_two_ranges":
        monkeypatch.setattr(P, "splitk_total", lambda t, s, b, m, n, eb, dev: real_total(t, min(s, 2), b, m, n, eb, dev)
                            if s > 1 else real_total(t, s, b, m, n, eb, dev))
    elif mistake == "total_without_launch":
        monkeypatch.setattr(P, "splitk_total", lambda t, s, b, m, n, eb, dev:
                            real_total(t, s, b, m, n, eb, P.replace(dev, launch_cost_k=0)))
    else:
        monkeypatch.setattr(P, "split_ranges", lambda k, s, bk: max(1, k // (-(-k // s)) if s > 1 and k else 1))
    assert _fails(T.test_split_ranges_and_total_closed_forms)
