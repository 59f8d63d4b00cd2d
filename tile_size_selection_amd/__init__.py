"""tss -- tile-size-selected fp16/bf16 GEMM and implicit-GEMM convolution for
MI355X (gfx950), with the tile planner that picks their tiles."""
