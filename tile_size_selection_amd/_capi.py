"""ctypes declarations of the C ABI in include/tss.h (argument marshalling only).

The library is loaded from this package directory; if it has not been built
the import fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtss.so")

TSS_OK, TSS_E_ARG, TSS_E_DTYPE, TSS_E_ALIGN, TSS_E_INFEASIBLE, TSS_E_HIP, TSS_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
TSS_E_SCRATCH = -7
TSS_SCRATCH_BYTES = 64 << 20
TSS_F16, TSS_BF16, TSS_F32 = 1, 2, 3
LDS_PATTERN = {"b32": 1, "b128": 2, "tr_b64": 3, "gemm_a": 4, "gemm_a_plain": 5, "gemm_b": 6, "gemm_b_plain": 7}
INSTR = {"mfma32": 1, "mfma16": 2, "mma": 16, "wgmma": 17, "simt": 18}
INSTR_NAME = {v: k for k, v in INSTR.items()}
FAIL_BITS = ["C3_M", "C3_N", "C3_K", "C3_THREADS", "C3_MAXTHREADS", "C3_WAVEGRID", "C3_LOAD", "C1", "C2", "OCC0"]
WARN_BITS = ["tail", "idle"]
BINDING = {0: "", 1: "regs", 2: "smem", 3: "threads"}

i32, i64, u32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64


class Device(ctypes.Structure):
    _fields_ = [(n, i32) for n in (
        "cores", "onchip_per_core", "onchip_per_block_max", "max_threads_per_core", "max_threads_per_block",
        "max_blocks_per_core", "lane_count", "reg_granule_per_lane", "acc_regs_max", "reg_overhead", "reg_model",
        "regs_per_core", "simds_per_core", "regs_per_lane_per_simd", "max_waves_per_simd", "wave_grid_rule",
        "load_bytes_per_lane", "ranking", "step_cost_k", "tile_cost_k", "split_byte_cost", "launch_cost_k",
        "target_waves_per_simd")]


class TileConfig(ctypes.Structure):
    _fields_ = [(n, i32) for n in ("bm", "bn", "bk", "stages", "threads", "instr")]


class Verdict(ctypes.Structure):
    _fields_ = ([("cfg", TileConfig)]
                + [(n, i64) for n in ("smem_per_stage", "smem_total", "accum_per_thread", "regs_per_thread",
                                      "regs_per_block", "blocks_by_regs", "blocks_by_smem", "blocks_by_threads",
                                      "blocks_per_core", "grid", "waves", "fill_num", "fill_den")]
                + [(n, u64) for n in ("traffic_num_hi", "traffic_num_lo", "traffic_den", "traffic_rounded")]
                + [("failures", u32), ("warnings", u32), ("binding", i32), ("pad_", i32)])


class MeasuredUsage(ctypes.Structure):
    _fields_ = [("cfg", TileConfig), ("regs_per_lane", i32), ("scratch_bytes", i32)]


class KernelUsage(ctypes.Structure):
    _fields_ = [(n, i32) for n in ("regs_per_lane", "lds_bytes", "scratch_bytes", "max_threads", "blocks_per_cu",
                                   "pad_")]


class HwSlice(ctypes.Structure):
    _fields_ = [(n, i64) for n in ("o0", "o1", "in_start", "in_end", "in_span", "pt", "pb", "halo")]


EXPORTS = ["tss_device_gfx950", "tss_device_pages", "tss_device_query", "tss_evaluate", "tss_tile_plan", "tss_conv_plan",
           "tss_tile_plan_usage", "tss_hw_tile", "tss_gemm", "tss_conv2d", "tss_conv2d_tiled",
           "tss_conv2d_workspace_size", "tss_kernel_available", "tss_kernel_usage_query", "tss_tile_plan_measured",
           "tss_lds_probe", "tss_gemm_default_config", "tss_status_string", "tss_instr_shape", "tss_gemm_splitk",
           "tss_gemm_splitk_workspace_size", "tss_conv2d_splitk", "tss_conv2d_splitk_workspace_size",
           "tss_conv2d_nhwc", "tss_conv2d_nhwc_workspace_size", "tss_gemm_autotune",
           "tss_splitk_plan", "tss_conv_splitk_plan", "tss_conv2d_splitk_noalloc"]

_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tile_size_selection_amd.build`"
                          " (the HIP library is required; there is no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    L.tss_device_gfx950.argtypes = [P(Device)]
    L.tss_device_pages.argtypes = [i32, i32, P(Device)]
    L.tss_device_query.argtypes = [i32, P(Device)]
    L.tss_evaluate.argtypes = [P(TileConfig), P(Device), i64, i64, i64, i64, i32, P(Verdict)]
    L.tss_tile_plan.argtypes = [i64, i64, i64, i64, i32, P(Device), i32, P(Verdict), P(Verdict), i32, P(i32)]
    L.tss_conv_plan.argtypes = [i64, i64, i64, i64, i32, P(Device), P(Verdict), P(Verdict), i32, P(i32)]
    L.tss_tile_plan_usage.argtypes = [i64, i64, i64, i64, i32, P(MeasuredUsage), i32, P(Verdict), P(Verdict), i32,
                                      P(i32)]
    L.tss_hw_tile.argtypes = [i64, i64, i64, i64, i64, i64, i64, P(HwSlice)]
    L.tss_gemm.argtypes = [i64, i64, i64, i32, vp, vp, vp, i64, i32, P(TileConfig), vp]
    L.tss_conv2d.argtypes = [i64] * 14 + [i32, i32, vp, vp, vp, vp, i64, P(TileConfig), vp]
    L.tss_conv2d_tiled.argtypes = [i64] * 16 + [i32, i32, vp, vp, vp, vp, i64, P(TileConfig), vp]
    L.tss_conv2d_workspace_size.argtypes = [i64] * 7
    L.tss_kernel_available.argtypes = [P(TileConfig), i32, i32]
    L.tss_kernel_usage_query.argtypes = [P(TileConfig), i32, i32, P(KernelUsage)]
    L.tss_tile_plan_measured.argtypes = [i64, i64, i64, i64, i32, i32, P(Verdict), P(Verdict), i32, P(i32)]
    L.tss_lds_probe.argtypes = [i32, i32, i32, i32, vp, vp]
    L.tss_gemm_default_config.argtypes = [i64, i64, i64, i64, i32, P(TileConfig)]
    L.tss_instr_shape.argtypes = [i32, P(i32)]
    L.tss_gemm_splitk.argtypes = [i64, i64, i64, i32, vp, vp, vp, i64, i32, P(TileConfig), i32, vp, i64, vp]
    L.tss_gemm_splitk_workspace_size.argtypes = [i64, i64, i64, i32]
    L.tss_conv2d_splitk.argtypes = [i64] * 16 + [i32, i32, vp, vp, vp, i32, vp, i64, P(TileConfig), vp]
    L.tss_conv2d_splitk_workspace_size.argtypes = [i64] * 13 + [i32]
    L.tss_conv2d_nhwc.argtypes = [i64] * 16 + [i32, i32, vp, vp, vp, i32, vp, i64, P(TileConfig), vp]
    L.tss_conv2d_nhwc_workspace_size.argtypes = [i64] * 13 + [i32]
    L.tss_gemm_autotune.argtypes = [i64, i64, i64, i32, vp, vp, vp, i64, i32, i32, i32, vp, P(TileConfig),
                                     P(ctypes.c_float)]
    L.tss_conv2d_splitk_noalloc.argtypes = [i64] * 16 + [i32, i32, vp, vp, vp, i32, P(TileConfig), vp]
    L.tss_splitk_plan.argtypes = [i64, i64, i64, i64, i32, P(Device), P(Verdict), P(i32)]
    L.tss_conv_splitk_plan.argtypes = [i64, i64, i64, i64, i32, P(Device), P(Verdict), P(i32)]
    L.tss_status_string.argtypes = [i32]
    L.tss_status_string.restype = ctypes.c_char_p
    for n in EXPORTS:
        if n != "tss_status_string":
            getattr(L, n).restype = i32
    L.tss_conv2d_workspace_size.restype = i64
    L.tss_gemm_splitk_workspace_size.restype = i64
    L.tss_conv2d_splitk_workspace_size.restype = i64
    L.tss_conv2d_nhwc_workspace_size.restype = i64
    _lib = L
    return L


class TssError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().tss_status_string(status).decode()} (status {status})")


def check(status: int, where: str) -> None:
    if status != TSS_OK:
        raise TssError(status, where)
