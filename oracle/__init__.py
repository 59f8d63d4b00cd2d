"""CPU oracle for the tiled GEMM / conv path and its tile-size planner.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library may import, call,
link or execute anything in this package.  Only the test suite, the smoke check
of the graft entry point and the CPU-baseline leg of the benchmark use it.

Every function here is written to be slow and obviously correct, straight from
the three source pages:

* "tile_decision.py" (tilelang tutorial, chapter 28, section 4: the tile-size
  decision procedure) -- constraints C0..C4 and the shortlist sweep;
* "04-tile-size-decision/README.md" (the same example's README) -- the
  constraint list, the commands and their printed expected output;
* "Tiling（分块）" (nlpx.cn) -- arithmetic intensity, the H/W tiling
  formulas with their worked example, multi-level GEMM tiling and the
  shared-memory / register examples of its constraint analysis.

Modules:
  planner     C0..C4 constraint evaluation and the sweep, on any device model
  htile       H-dimension tile slices, pads and halo for a convolution
  intensity   arithmetic-intensity arithmetic
  gemm_conv   fp64 triple-loop GEMM and direct / H-tiled convolution (plain C
              compiled with gcc, loaded with ctypes)
"""
