"""tss -- tile-size-selected fp16/bf16 GEMM and implicit-GEMM convolution for
MI355X (gfx950), with the tile planner that picks their tiles.

The work is done by libtss.so (include/tss.h); this package only marshals
arguments.  Importing the package loads nothing; the first call loads the
library and fails loudly if it has not been built.
"""
from .api import (TileConfig, autotune_gemm, conv2d, conv2d_noalloc, conv2d_default_config, conv2d_workspace_size, conv_plan, default_config,
                  device_gfx950, device_pages, device_query, evaluate, gemm, gemm_splitk_workspace_size, hw_tile,
                  kernel_available, kernel_usage, lds_probe, splitk_plan, conv_splitk_plan, tile_plan, tile_plan_measured,
                  tile_plan_usage, verdict_dict)
from ._capi import TssError

__all__ = ["TileConfig", "autotune_gemm", "conv2d", "conv2d_noalloc", "conv2d_default_config", "conv2d_workspace_size", "conv_plan", "default_config",
           "device_gfx950", "device_pages", "device_query", "evaluate", "gemm", "gemm_splitk_workspace_size",
           "hw_tile", "kernel_available",
           "kernel_usage", "lds_probe", "splitk_plan", "conv_splitk_plan", "tile_plan", "tile_plan_measured", "tile_plan_usage", "verdict_dict",
           "TssError"]
