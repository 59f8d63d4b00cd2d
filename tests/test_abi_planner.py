"""C ABI checks that need no GPU: the library loads and exports every entry
point declared in include/tss.h; the C++ planner agrees bit for bit with the
oracle; the H-tile formulas agree; argument errors are reported before any
device work."""
import ctypes
import itertools
import os
import re
from fractions import Fraction

import numpy as np
import pytest

from oracle import htile as OH
from oracle import planner as OP
import tile_size_selection_amd as tss
from tile_size_selection_amd import _capi as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "tss.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"^(?:int32_t|int64_t|const char \*)\s*(tss_\w+)\(", hdr, flags=re.M))
    assert declared == set(C.EXPORTS)
    L = C.lib()
    for name in declared:
        assert hasattr(L, name), name


def _oracle_dev(dev_c, name):
    if name == "gfx950":
        return OP.device_gfx950()
    sm, kb = name
    return OP.device_pages(sm, kb)


def _same(v_c: dict, v_o: OP.Verdict, name_map=None):
    c = v_c["config"]
    o = v_o.config
    assert (c.bm, c.bn, c.bk, c.stages, c.threads, c.instr) == \
        (o.block_m, o.block_n, o.block_k, o.stages, o.threads, o.instr)
    assert v_c["smem_per_stage"] == v_o.smem_per_stage and v_c["smem_total"] == v_o.smem_total
    assert v_c["accum_per_thread"] == v_o.accum_per_thread and v_c["regs_per_thread"] == v_o.regs_per_thread
    assert v_c["regs_per_block"] == v_o.regs_per_block
    assert (v_c["blocks_by_regs"], v_c["blocks_by_smem"], v_c["blocks_by_threads"], v_c["blocks_per_core"]) == \
        (v_o.blocks_by_regs, v_o.blocks_by_smem, v_o.blocks_by_threads, v_o.blocks_per_core)
    assert v_c["failures"] == v_o.failures
    assert v_c["binding"] == v_o.binding
    if not v_o.failures:
        assert (v_c["grid"], v_c["waves"], v_c["fill"]) == (v_o.grid, v_o.waves, v_o.fill)
        assert v_c["warnings"] == v_o.warnings
        assert v_c["traffic"] == v_o.traffic
        assert v_c["traffic_rounded"] == OP.round_half_even(v_o.traffic)


DEVICES = [("gfx950", None), ((132, 228), None), ((108, 164), None)]


def _cdev(name):
    return tss.device_gfx950() if name == "gfx950" else tss.device_pages(*name)


@pytest.mark.parametrize("name", ["gfx950", (132, 228), (108, 164)])
def test_planner_sweep_bit_exact(name):
    cd, od = _cdev(name), _oracle_dev(None, name)
    shapes = [(1, 4096, 4096, 4096), (1, 256, 256, 256), (4, 3000, 5000, 2048), (1, 8192, 8192, 8192),
              (1, 256, 6272, 2304), (1, 100, 37, 24)]
    instr_sets = [None] if name == "gfx950" else ["wgmma", "mma", "simt"]
    for (b, M, N, K), ins in itertools.product(shapes, instr_sets):
        instrs = [s for s, _ in od.instr_shapes] if ins is None else [ins]
        ores = OP.sweep(M, N, K, od, instrs, batch=b)
        best, lst, n = tss.tile_plan(M, N, K, batch=b, dev=cd, instr=ins, cap=len(ores) + 5)
        assert n == len(ores)
        assert len(lst) == len(ores)
        for vc, vo in zip(lst, ores):
            _same(vc, vo)
        if ores:
            _same(best, ores[0])


def _tc(c: OP.TileConfig) -> tss.TileConfig:
    return tss.TileConfig(c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_plan_with_measured_usage_bit_exact(seed):
    """tss_tile_plan_usage against the oracle's sweep with the same table:
    imagined compiled kernels with registers above and below the model's
    estimate, some spilling, some missing."""
    g = OP.device_gfx950()
    instrs = [s for s, _ in g.instr_shapes]
    rng = np.random.default_rng(seed)
    feas = [c for c in OP.candidates(g, 1 << 20, instrs) if OP.evaluate(c, g).feasible]
    usage_o = {}
    for c in feas:
        if rng.random() < 0.1:
            continue                                              # no kernel
        usage_o[c] = (int(rng.integers(1, 257)), int(rng.integers(1, 600)) if rng.random() < 0.1 else 0)
    usage_c = {_tc(c): u for c, u in usage_o.items()}
    for (b, M, N, K) in [(1, 4096, 4096, 4096), (1, 256, 6272, 2304), (4, 3000, 5000, 2048), (1, 100, 37, 24)]:
        ores = OP.sweep(M, N, K, g, instrs, batch=b, regs=usage_o)
        best, lst, n = tss.tile_plan_usage(M, N, K, usage_c, batch=b, cap=len(ores) + 5)
        assert n == len(ores) and len(lst) == len(ores)
        for vc, vo in zip(lst, ores):
            _same(vc, vo)
        _same(best, ores[0])
        assert all(u[1] == 0 for c, u in usage_o.items() if c in {v.config for v in ores})


def test_measured_usage_closed_forms():
    """Occupancy from measured registers, worked by hand: per SIMD 512 /
    registers (rounded up to 8) waves, at most 8; a block's waves spread over
    the 4 SIMDs.  A spilling kernel fails C2; feeding the model's own
    estimate back changes nothing."""
    g = OP.device_gfx950()
    big = OP.TileConfig(256, 256, 64, 2, 512, "mfma16")
    v = OP.evaluate(big, g)                                # 128 accumulators + 32 = 160 -> 3 waves/SIMD, 12 per CU
    assert (v.regs_per_thread, v.blocks_by_regs) == (160, 1)
    v = OP.evaluate(big, g, regs_measured=250)             # 256 -> 2 waves/SIMD, 8 per CU: one 8-wave block
    assert (v.regs_per_thread, v.blocks_by_regs, v.blocks_per_core) == (256, 1, 1)
    small = OP.TileConfig(64, 64, 32, 2, 256, "mfma16")
    v = OP.evaluate(small, g)                              # 16 + 32 = 48 -> 8 waves/SIMD, 32 per CU: 8 blocks
    assert (v.regs_per_thread, v.blocks_by_regs) == (48, 8)
    v = OP.evaluate(small, g, regs_measured=97)            # 104 -> 4 waves/SIMD, 16 per CU: 4 blocks of 4 waves
    assert (v.regs_per_thread, v.blocks_by_regs, v.blocks_per_core) == (104, 4, 4)
    assert v.accum_per_thread == 16 and not v.failures
    wide = OP.TileConfig(256, 256, 64, 2, 256, "mfma16")   # 256 accumulators: the model's C2 lets it through
    assert OP.evaluate(wide, g).feasible
    v = OP.evaluate(wide, g, regs_measured=512, spill_bytes=144)
    assert v.failures == ["C2"] and "spills 144 bytes" in v.messages[0]
    instrs = [s for s, _ in g.instr_shapes]
    for (b, M, N, K) in [(1, 4096, 4096, 4096), (1, 256, 6272, 2304)]:
        plain = OP.sweep(M, N, K, g, instrs, batch=b)
        fed = OP.sweep(M, N, K, g, instrs, batch=b, regs={x.config: (x.regs_per_thread, 0) for x in plain})
        assert [x.config for x in fed] == [x.config for x in plain]
        assert [x.blocks_per_core for x in fed] == [x.blocks_per_core for x in plain]
        best_c, lst_c, n_c = tss.tile_plan_usage(M, N, K, {_tc(x.config): (x.regs_per_thread, 0) for x in plain},
                                                 batch=b, cap=len(plain))
        best_p, lst_p, n_p = tss.tile_plan(M, N, K, batch=b, cap=len(plain))
        assert n_c == n_p and [x["config"] for x in lst_c] == [x["config"] for x in lst_p]
    L = C.lib()
    t = (C.MeasuredUsage * 1)()
    t[0].cfg = _tc(big).c()
    for r, sc in ((0, 0), (-1, 0), (160, -1)):
        t[0].regs_per_lane, t[0].scratch_bytes = r, sc
        assert L.tss_tile_plan_usage(1, 64, 64, 64, 2, t, 1, None, None, 0, None) == C.TSS_E_ARG
    assert L.tss_tile_plan_usage(1, 64, 64, 64, 2, None, 1, None, None, 0, None) == C.TSS_E_ARG
    assert L.tss_tile_plan_usage(1, 64, 64, 64, 2, None, 0, None, None, 0, None) == C.TSS_E_INFEASIBLE


def test_planner_pages_printout_through_c():
    """The README page's printed sweep figures, reproduced by the C++ planner."""
    best, lst, n = tss.tile_plan(4096, 4096, 4096, dev=tss.device_pages(), instr="wgmma", cap=8)
    assert n == 459
    assert [(v["config"].bm, v["config"].bn, v["config"].bk, v["config"].stages, v["config"].threads)
            for v in lst[:2]] == [(256, 256, 16, 2, 512), (256, 256, 16, 3, 512)]
    assert all(f"{float(v['traffic']) / 1e6:.1f}" == "1107.3" for v in lst)
    assert all((v["regs_per_thread"], v["blocks_per_core"], v["waves"], f"{float(v['fill']) * 100:.0f}%",
                v["binding"]) == (128, 1, 2, "94%", "regs") for v in lst)


def test_evaluate_random_configs_bit_exact():
    rng = np.random.default_rng(7)
    for _ in range(3000):
        name = DEVICES[rng.integers(0, 3)][0]
        cd, od = _cdev(name), _oracle_dev(None, name)
        instrs = [s for s, _ in od.instr_shapes]
        ins = instrs[rng.integers(0, len(instrs))]
        cfg = OP.TileConfig(int(rng.choice([8, 16, 24, 32, 48, 64, 96, 128, 192, 256, 512])),
                            int(rng.choice([8, 16, 32, 40, 64, 128, 256, 512])),
                            int(rng.choice([8, 16, 32, 48, 64, 128])), int(rng.integers(1, 6)),
                            int(rng.choice([32, 64, 96, 100, 128, 192, 256, 512, 1024, 2048])), ins)
        b, M, N, K = int(rng.integers(1, 5)), int(rng.integers(0, 20000)), int(rng.integers(0, 20000)), \
            int(rng.integers(0, 20000))
        eb = int(rng.choice([1, 2, 4]))
        vo = OP.evaluate(cfg, od, elem_bytes=eb)
        OP.finish_parallelism(vo, M, N, od, b)
        vo.traffic = OP.dram_traffic(M, N, K, cfg, eb, b)
        vc = tss.evaluate(tss.TileConfig(cfg.block_m, cfg.block_n, cfg.block_k, cfg.stages, cfg.threads, ins),
                          M, N, K, batch=b, elem_bytes=eb, dev=cd)
        # compare C4/C0 even for infeasible configs
        assert (vc["grid"], vc["waves"], vc["fill"], vc["warnings"]) == (vo.grid, vo.waves, vo.fill, vo.warnings)
        assert vc["traffic"] == vo.traffic
        _same(vc, vo)


def test_hw_tile_matches_oracle():
    for H, kh, sh, pt, d in itertools.product((1, 5, 9, 56), (1, 3, 5), (1, 2, 3), (0, 1, 2), (1, 2)):
        OHt = OH.out_size(H, kh, sh, pt, pt, d)
        if OHt <= 0:
            continue
        for toh in (1, 2, 3, 8):
            for t in OH.tile_table(H, kh, sh, pt, d, OHt, toh):
                c = tss.hw_tile(H, kh, sh, pt, d, t.o0, t.o1)
                assert (c["in_start"], c["in_end"], c["in_span"], c["pt"], c["pb"], c["halo"]) == \
                    (t.in_start, t.in_end, t.in_span, t.pt, t.pb, t.halo)


def test_hw_tile_worked_example():
    a = tss.hw_tile(9, 3, 2, 1, 1, 0, 2)
    b = tss.hw_tile(9, 3, 2, 1, 1, 2, 4)
    assert (a["in_start"], a["in_end"], a["in_span"], a["pt"], a["pb"]) == (0, 4, 4, 1, 0)
    assert (b["in_start"], b["in_end"], b["in_span"], b["pt"], b["pb"]) == (3, 8, 5, 0, 0)
    assert a["halo"] == b["halo"] == 1


def test_argument_errors_before_device_work():
    L = C.lib()
    cfg = C.TileConfig(256, 256, 64, 2, 256, C.INSTR["mfma32"])
    g = lambda *a: L.tss_gemm(*a)
    assert g(64, 64, 64, 7, 16, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_DTYPE
    assert g(64, 64, 64, C.TSS_F16, 16, 16, 16, 1, C.TSS_BF16, None, None) == C.TSS_E_DTYPE
    assert g(64, 64, 60, C.TSS_F16, 16, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_ALIGN   # K % 8
    assert g(64, 36, 64, C.TSS_F16, 16, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_ALIGN   # N % 8
    assert g(64, 64, 64, C.TSS_F16, 24, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_ALIGN   # A misaligned
    assert g(64, 64, 64, C.TSS_F16, None, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_ARG
    assert g(-1, 64, 64, C.TSS_F16, 16, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_ARG
    assert g(64, 64, 64, C.TSS_F16, 16, 16, 16, 0, C.TSS_F32, None, None) == C.TSS_E_ARG
    assert g(0, 64, 64, C.TSS_F16, None, None, None, 1, C.TSS_F32, None, None) == C.TSS_OK  # empty: no-op
    assert g(1 << 17, 1 << 14, 1 << 14, C.TSS_F16, 16, 16, 16, 1, C.TSS_F32, None, None) == C.TSS_E_ARG  # >2 GiB
    bad = C.TileConfig(256, 256, 64, 3, 256, C.INSTR["mfma32"])       # 192 KiB of LDS: C1
    assert g(64, 64, 64, C.TSS_F16, 16, 16, 16, 1, C.TSS_F32, ctypes.byref(bad), None) == C.TSS_E_INFEASIBLE
    nv = C.TileConfig(128, 128, 32, 2, 256, C.INSTR["wgmma"])
    assert g(64, 64, 64, C.TSS_F16, 16, 16, 16, 1, C.TSS_F32, ctypes.byref(nv), None) == C.TSS_E_ARG
    cv = lambda *a: L.tss_conv2d(*a)
    wsz = L.tss_conv2d_workspace_size
    # channel-last input at offset 0, reordered weights at the next 256-byte boundary; channels rounded up
    # to 64 (the largest K step a tile can take)
    assert wsz(8, 256, 56, 56, 256, 3, 3) == 8 * 56 * 56 * 256 * 2 + 256 * 9 * 256 * 2
    assert wsz(2, 3, 5, 5, 4, 3, 3) == 2 * 5 * 5 * 64 * 2 + 4 * 9 * 64 * 2     # 6400 B: already aligned
    assert wsz(1, 8, 1, 1, 4, 1, 1) == 256 + 4 * 64 * 2                         # xc 64*2 = 128 B -> 256
    assert wsz(1, 72, 1, 3, 8, 1, 1) == 3 * 128 * 2 + 8 * 128 * 2              # C 72 -> 128 channels
    assert wsz(0, 3, 5, 5, 4, 3, 3) == C.TSS_E_ARG
    assert wsz(1, 1 << 31, 5, 5, 4, 3, 3) == C.TSS_E_ARG
    base = [8, 256, 56, 56, 256, 3, 3, 2, 2, 1, 1, 1, 1]
    ws = wsz(*base[:7])
    ok_ptrs = [16, 16, 16, 256, ws]
    assert cv(*base, 0, C.TSS_F16, C.TSS_F32, *ok_ptrs, None, None) == C.TSS_E_ARG          # tile_oh 0
    assert cv(*base, 29, C.TSS_F16, C.TSS_F32, *ok_ptrs, None, None) == C.TSS_E_ARG         # tile_oh > OH
    assert cv(*base, 8, C.TSS_F32, C.TSS_F32, *ok_ptrs, None, None) == C.TSS_E_DTYPE
    assert cv(*base, 8, C.TSS_F16, C.TSS_F32, 16, 24, 16, 256, ws, None, None) == C.TSS_E_ALIGN
    assert cv(*base, 8, C.TSS_F16, C.TSS_F32, 16, 16, 16, None, ws, None, None) == C.TSS_E_ARG   # no workspace
    assert cv(*base, 8, C.TSS_F16, C.TSS_F32, 16, 16, 16, 256, ws - 1, None, None) == C.TSS_E_ARG  # too small
    assert cv(*base, 8, C.TSS_F16, C.TSS_F32, 16, 16, 16, 264, ws, None, None) == C.TSS_E_ALIGN  # misaligned
    assert cv(*[8, 256, 1, 56, 256, 3, 3, 2, 2, 0, 1, 1, 1], 1, C.TSS_F16, C.TSS_F32, *ok_ptrs, None,
              None) == C.TSS_E_ARG                                                           # window > input
    cvt = lambda *a: L.tss_conv2d_tiled(*a)
    for tn, toh, tow in [(0, 8, 8), (9, 8, 8), (8, 0, 8), (8, 29, 8), (8, 8, 0), (8, 8, 29)]:
        assert cvt(*base, tn, toh, tow, C.TSS_F16, C.TSS_F32, *ok_ptrs, None, None) == C.TSS_E_ARG, (tn, toh, tow)
    assert cvt(*base, 8, 8, 8, C.TSS_F16, C.TSS_F32, 16, 16, 16, 256, ws - 1, None, None) == C.TSS_E_ARG
    lp = L.tss_lds_probe
    assert lp(1, 1, 10, 1, None, None) == C.TSS_E_ARG                 # no output buffer
    assert lp(99, 1, 10, 1, 64, None) == C.TSS_E_ARG                  # unknown pattern
    assert lp(2, 6, 10, 1, 64, None) == C.TSS_E_ARG                   # 16-byte reads at a 24-byte stride
    assert lp(3, 3, 10, 1, 64, None) == C.TSS_E_ARG                   # 8-byte reads at a 12-byte stride
    assert lp(1, 1, 0, 1, 64, None) == C.TSS_E_ARG and lp(1, 1, 10, 0, 64, None) == C.TSS_E_ARG
    assert L.tss_evaluate(ctypes.byref(cfg), None, 0, 1, 1, 1, 2, ctypes.byref(C.Verdict())) == C.TSS_E_ARG
    assert L.tss_hw_tile(9, 3, 2, 1, 1, 2, 2, ctypes.byref(C.HwSlice())) == C.TSS_E_ARG
    assert L.tss_tile_plan(1, 64, 64, 64, 2, None, 99, None, None, 0, None) == C.TSS_E_ARG
    assert L.tss_status_string(-4).decode() == "tile configuration infeasible"


def test_every_feasible_gfx950_config_has_a_kernel():
    g = OP.device_gfx950()
    n = 0
    for c in OP.candidates(g, 1 << 20, ["mfma32", "mfma16"]):
        ok = OP.evaluate(c, g).feasible
        for dt in ("f16", "bf16"):
            for op in ("gemm", "conv"):
                assert tss.kernel_available(tss.TileConfig(c.block_m, c.block_n, c.block_k, c.stages, c.threads,
                                                           c.instr), dt, op) == ok
        n += ok
    assert n == 292


def test_default_config_is_planner_best():
    for (b, M, N, K) in [(1, 4096, 4096, 4096), (4, 3000, 5000, 2048), (1, 256, 256, 256), (1, 8192, 8192, 8192)]:
        best, _, _ = tss.tile_plan(M, N, K, batch=b)
        assert tss.default_config(M, N, K, batch=b) == best["config"]


def test_default_config_cache_under_concurrent_callers():
    """tss_gemm_default_config from 8 threads at once (ctypes drops the GIL
    around the call) over more distinct shapes than the plan cache holds, so
    that it is cleared while other threads read and fill it: every answer is
    still the uncached planner's best."""
    import threading
    rng = np.random.default_rng(5)
    shapes = sorted({(int(b), int(m), int(n) * 8, int(k) * 8)
                     for b, m, n, k in zip(rng.integers(1, 5, 6000), rng.integers(1, 9000, 6000),
                                           rng.integers(1, 1200, 6000), rng.integers(1, 1200, 6000))})
    assert len(shapes) > 4096
    want = {s: tss.tile_plan(s[1], s[2], s[3], batch=s[0])[0]["config"] for s in shapes}
    bad = []

    def worker(part):
        for s in part:
            got = tss.default_config(s[1], s[2], s[3], batch=s[0])
            if got != want[s]:
                bad.append((s, got, want[s]))

    threads = [threading.Thread(target=worker, args=(shapes[i::8],)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]


@pytest.mark.parametrize("seed", [4, 5])
def test_conv_plan_bit_exact(seed):
    """tss_conv_plan against the oracle's sweep_conv, every verdict in rank
    order (each with its candidate's own padded K), on random convolutions and
    on the conv workload."""
    rng = np.random.default_rng(seed)
    probs = [(256, 6272, 256, 9), (64, 8 * 112 * 112, 3, 9)]
    probs += [(int(rng.integers(1, 600)), int(rng.integers(1, 20000)), int(rng.integers(1, 300)),
               int(rng.choice([1, 4, 9, 25, 49]))) for _ in range(6)]
    for co, px, c, taps in probs:
        ores = OP.sweep_conv(co, px, c, taps)
        best, lst, n = tss.conv_plan(co, px, c, taps, cap=len(ores) + 5)
        assert n == len(ores) == len(lst)
        for vc, vo in zip(lst, ores):
            _same(vc, vo)
        _same(best, ores[0])


def test_conv_default_config_is_the_conv_plan():
    from tile_size_selection_amd.inputs import WORKLOADS
    cw = WORKLOADS[5]
    cfg = tss.conv2d_default_config(cw.N, cw.C, cw.H, cw.W, cw.Co, cw.kh, cw.kw, cw.stride, cw.pad, cw.dil)
    assert cfg == tss.conv_plan(cw.Co, cw.N * 28 * 28, cw.C, cw.kh * cw.kw)[0]["config"]
    assert cfg == tss.TileConfig(128, 64, 64, 4, 512, "mfma16")
    with pytest.raises(tss.TssError):
        tss.conv_plan(64, 100, 0, 9)


def _with_costs(step, tile, target=4):
    d = tss.device_gfx950()
    d.step_cost_k, d.tile_cost_k, d.target_waves_per_simd = step, tile, target
    return d, OP.replace(OP.device_gfx950(), step_cost_k=step, tile_cost_k=tile, target_waves_per_simd=target)


@pytest.mark.parametrize("step,tile,target", [(0, 0, 0), (22, 0, 4), (10, 300, 2), (40, 2000, 8), (22, 900, 0)])
def test_ranking_cost_parameters_bit_exact(step, tile, target):
    """The gfx950 ranking's cost parameters and waves target come from the
    device record on both sides: with any values, the C++ plans equal the
    oracle's, GEMM and convolution, every verdict in rank order."""
    cd, od = _with_costs(step, tile, target)
    ins = [s for s, _ in od.instr_shapes]
    for (b, M, N, K) in [(1, 4096, 4096, 4096), (1, 4096, 4096, 72), (1, 2048, 8192, 136), (4, 3000, 5000, 2048),
                         (1, 256, 256, 256), (1, 8192, 1024, 8192)]:
        ores = OP.sweep(M, N, K, od, ins, batch=b)
        best, lst, n = tss.tile_plan(M, N, K, batch=b, dev=cd, cap=len(ores) + 5)
        assert n == len(ores) == len(lst)
        for vc, vo in zip(lst, ores):
            _same(vc, vo)
    for co, px, c, taps in [(256, 6272, 256, 9), (64, 8 * 112 * 112, 3, 9), (128, 8 * 56 * 56, 96, 9)]:
        ores = OP.sweep_conv(co, px, c, taps, dev=od)
        best, lst, n = tss.conv_plan(co, px, c, taps, cap=len(ores) + 5, dev=cd)
        assert n == len(ores) == len(lst)
        for vc, vo in zip(lst, ores):
            _same(vc, vo)


def test_planner_at_the_edge_of_its_size_bounds():
    """batch * M * N up to 2^62 and K up to 2^40 are planned exactly (C0's
    numerator near 2^115, the time term near 2^105): the plans equal the
    oracle's, whose integers are unbounded; one past a bound is an argument
    error, as is a device with a negative cost parameter."""
    g = OP.device_gfx950()
    ins = [s for s, _ in g.instr_shapes]
    for (b, M, N, K) in [(1, 1 << 31, 1 << 31, 1 << 40), (1 << 20, 1 << 21, 1 << 21, 1 << 40),
                         (3, (1 << 30) + 7, (1 << 30) + 1, (1 << 40) - 3)]:
        ores = OP.sweep(M, N, K, g, ins, batch=b)
        best, lst, n = tss.tile_plan(M, N, K, batch=b, cap=len(ores))
        assert n == len(ores)
        for vc, vo in zip(lst, ores):
            c, o = vc["config"], vo.config
            assert (c.bm, c.bn, c.bk, c.stages, c.threads, c.instr) == \
                (o.block_m, o.block_n, o.block_k, o.stages, o.threads, o.instr)
            assert (vc["grid"], vc["waves"], vc["fill"], vc["traffic"]) == (vo.grid, vo.waves, vo.fill, vo.traffic)
            r = OP.round_half_even(vo.traffic)
            assert vc["traffic_rounded"] == min(r, (1 << 64) - 1)
    # conv plan at the edge: K = 512 taps * 2^30 channels = 2^39
    ores = OP.sweep_conv(1 << 31, 1 << 31, 1 << 30, 512)
    best, lst, n = tss.conv_plan(1 << 31, 1 << 31, 1 << 30, 512, cap=len(ores))
    assert n == len(ores) and [v["config"] for v in lst] == [_tc(v.config) for v in ores]
    L = C.lib()
    v = C.Verdict()
    for args in [(1, 1 << 31, (1 << 31) + 1, 64), (1 << 20, 1 << 21, (1 << 21) + 1, 64), (1, 8, 8, (1 << 40) + 1),
                 ((1 << 20) + 1, 1, 1, 1), (1, (1 << 40) + 1, 1, 1)]:
        assert L.tss_tile_plan(*args, 2, None, 0, ctypes.byref(v), None, 0, None) == C.TSS_E_ARG, args
    cfg = tss.TileConfig(256, 256, 64, 2, 512, "mfma16").c()
    assert L.tss_evaluate(ctypes.byref(cfg), None, 1, 1 << 31, (1 << 31) + 1, 64, 2, ctypes.byref(v)) == C.TSS_E_ARG
    assert L.tss_conv_plan(1 << 31, (1 << 31) + 1, 64, 9, 2, None, ctypes.byref(v), None, 0, None) == C.TSS_E_ARG
    d = tss.device_gfx950()
    d.step_cost_k = -1
    assert L.tss_tile_plan(1, 64, 64, 64, 2, ctypes.byref(d), 0, ctypes.byref(v), None, 0, None) == C.TSS_E_ARG
    d = tss.device_gfx950()
    d.target_waves_per_simd = -1
    assert L.tss_tile_plan(1, 64, 64, 64, 2, ctypes.byref(d), 0, ctypes.byref(v), None, 0, None) == C.TSS_E_ARG
    pages = tss.device_pages()
    assert L.tss_conv_plan(64, 64, 64, 9, 2, ctypes.byref(pages), ctypes.byref(v), None, 0, None) == C.TSS_E_ARG


@pytest.mark.parametrize("costs", [None, (22, 0, 6, 67000), (0, 300, 2, 10000), (22, 600, 0, 0)])
def test_splitk_plan_bit_exact(costs):
    """tss_splitk_plan / tss_conv_splitk_plan against the oracle's
    splitk_plan / conv_splitk_plan: the same split count and tile, with the
    default and other cost parameters, for a free and a fixed split count."""
    cd, od = tss.device_gfx950(), OP.device_gfx950()
    if costs:
        cd.step_cost_k, cd.tile_cost_k, cd.split_byte_cost, cd.launch_cost_k = costs
        od = OP.replace(od, step_cost_k=costs[0], tile_cost_k=costs[1], split_byte_cost=costs[2],
                        launch_cost_k=costs[3])
    for (b, M, N, K) in [(1, 256, 256, 256), (1, 512, 512, 8192), (1, 1024, 1024, 8192), (1, 128, 128, 16384),
                         (2, 300, 328, 1000), (1, 4096, 4096, 4096), (1, 64, 64, 8)]:
        for fixed in (0, 3):
            S_o, v_o = OP.splitk_plan(M, N, K, dev=od, batch=b, splits=fixed)
            S_c, v_c = tss.splitk_plan(M, N, K, batch=b, dev=cd, splits=fixed)
            assert S_c == S_o, (b, M, N, K, fixed)
            _same(v_c, v_o)
    for co, px, c, taps in [(256, 6272, 256, 9), (64, 200, 3, 9), (32, 64, 100, 9), (16, 96, 512, 25)]:
        for fixed in (0, 2):
            S_o, v_o = OP.conv_splitk_plan(co, px, c, taps, dev=od, splits=fixed)
            S_c, v_c = tss.conv_splitk_plan(co, px, c, taps, dev=cd, splits=fixed)
            assert S_c == S_o, (co, px, c, taps, fixed)
            _same(v_c, v_o)
