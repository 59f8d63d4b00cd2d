"""The compiled kernels as the HIP runtime reads them from their code
objects: the runtime's occupancy calculator agrees with the planner's
per-SIMD occupancy rule once that rule is given the kernel's real registers
and LDS; exactly the tiles with 256 accumulators per lane spill; the
measured plan is the usage-table plan and leaves the spilling kernels out."""
import pytest

from oracle import planner as OP
import tile_size_selection_amd as tss

pytestmark = pytest.mark.gpu


def _configs():
    g = OP.device_gfx950()
    for c in OP.candidates(g, 1 << 20, [s for s, _ in g.instr_shapes]):
        v = OP.evaluate(c, g)
        if v.feasible:
            yield tss.TileConfig(c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr), v.accum_per_thread


def test_every_kernel_usage():
    n, off, spill = 0, [], []
    for cfg, acc in _configs():
        for dt in ("f16", "bf16"):
            for op in ("gemm", "conv"):
                u = tss.kernel_usage(cfg, dt, op)
                n += 1
                assert u["max_threads"] >= cfg.threads, (cfg, dt, op, u)
                assert u["lds_bytes"] >= (cfg.bm + cfg.bn) * cfg.bk * 2 * cfg.stages, (cfg, dt, op, u)
                regs = -(-u["regs_per_lane"] // 8) * 8
                waves_per_simd = min(8, 512 // regs)
                want = min(4 * waves_per_simd // (cfg.threads // 64), 163840 // u["lds_bytes"], 2048 // cfg.threads)
                if want != u["blocks_per_cu"]:
                    off.append((cfg, dt, op, u, want))
                if u["scratch_bytes"]:
                    spill.append((cfg, dt, op, acc, u["regs_per_lane"], u["scratch_bytes"]))
    print(f"{n} kernels; occupancy rule vs runtime calculator: {len(off)} differ; {len(spill)} spill", flush=True)
    for o in off[:10]:
        print("  occupancy", o, flush=True)
    assert n == 1168
    assert not off
    # spilling: every kernel with 256 accumulators per lane (37 configurations x 2 dtypes x 2 operations), no other
    assert len(spill) == 148 and all(acc == 256 for _, _, _, acc, _, _ in spill), spill[:5]


def test_measured_plan_is_the_usage_table_plan():
    for (b, M, N, K), dt, op in [((1, 4096, 4096, 4096), "f16", "gemm"), ((4, 3000, 5000, 2048), "f16", "gemm"),
                                 ((1, 8192, 8192, 8192), "bf16", "gemm"), ((1, 256, 6272, 2304), "f16", "conv"),
                                 ((1, 256, 256, 256), "f16", "gemm")]:
        best_m, lst_m, n_m = tss.tile_plan_measured(M, N, K, batch=b, dtype=dt, op=op, cap=400)
        usage = {}
        for cfg, _ in _configs():
            u = tss.kernel_usage(cfg, dt, op)
            usage[cfg] = (u["regs_per_lane"], u["scratch_bytes"])
        best_u, lst_u, n_u = tss.tile_plan_usage(M, N, K, usage, batch=b, cap=400)
        assert n_m == n_u == 292 - 37
        assert [v["config"] for v in lst_m] == [v["config"] for v in lst_u]
        assert [v["blocks_per_core"] for v in lst_m] == [v["blocks_per_core"] for v in lst_u]
        assert all(usage[v["config"]][1] == 0 for v in lst_m)
        plain, _, _ = tss.tile_plan(M, N, K, batch=b)
        assert usage[plain["config"]][1] == 0          # the model's choice is never a spilling kernel here
        print(f"{op} {b}x{M}x{N}x{K} {dt}: measured plan {best_m['config']} "
              f"(regs {best_m['regs_per_thread']}, blocks/CU {best_m['blocks_per_core']}); "
              f"model plan {plain['config']} (regs {plain['regs_per_thread']}, "
              f"blocks/CU {plain['blocks_per_core']})", flush=True)


def test_measured_plan_equals_the_oracle_with_the_kernels_table():
    """tss_tile_plan_measured (C++, table read from the code objects through
    the HIP runtime) against the oracle's sweep given the same table: the
    same candidates in the same order, with the same occupancy, grid and C0."""
    g = OP.device_gfx950()
    ins = [s for s, _ in g.instr_shapes]
    for (b, M, N, K), dt, op in [((1, 4096, 4096, 4096), "f16", "gemm"), ((1, 256, 6272, 2304), "f16", "conv"),
                                 ((4, 3000, 5000, 2048), "bf16", "gemm"), ((1, 4096, 4096, 72), "f16", "gemm")]:
        regs = {}
        for cfg, _ in _configs():
            u = tss.kernel_usage(cfg, dt, op)
            regs[OP.TileConfig(cfg.bm, cfg.bn, cfg.bk, cfg.stages, cfg.threads, cfg.instr)] = \
                (u["regs_per_lane"], u["scratch_bytes"])
        ores = OP.sweep(M, N, K, g, ins, batch=b, regs=regs)
        best, lst, n = tss.tile_plan_measured(M, N, K, batch=b, dtype=dt, op=op, cap=len(ores) + 5)
        assert n == len(ores) == len(lst)
        for vc, vo in zip(lst, ores):
            c, o = vc["config"], vo.config
            assert (c.bm, c.bn, c.bk, c.stages, c.threads, c.instr) == \
                (o.block_m, o.block_n, o.block_k, o.stages, o.threads, o.instr)
            assert (vc["regs_per_thread"], vc["blocks_per_core"], vc["grid"], vc["waves"], vc["fill"],
                    vc["traffic"]) == (vo.regs_per_thread, vo.blocks_per_core, vo.grid, vo.waves, vo.fill,
                                       vo.traffic)
        print(f"{op} {dt} {b}x{M}x{N}x{K}: measured plan {best['config']} equals the oracle's", flush=True)
