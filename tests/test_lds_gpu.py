"""The LDS bank table (tss_lds_probe), the measured counterpart of the Tiling
page's bank-conflict table: an odd word stride is as fast as the contiguous
read, power-of-two strides conflict more as they grow, and the GEMM kernel's
XOR swizzle makes its fragment reads conflict-free where the same reads
without it conflict."""
import pytest

import tile_size_selection_amd as tss

pytestmark = pytest.mark.gpu

IT = 2000


def _c(pattern, stride=0):
    # the best of three launches: the table is about bank conflicts, not about noise
    return min(tss.lds_probe(pattern, stride, iters=IT) for _ in range(3))


def test_strided_reads():
    tss.lds_probe("b32", 1, iters=50)  # warm-up
    base = _c("b32", 1)
    by_stride = {s: _c("b32", s) for s in (2, 4, 8, 16, 32, 64)}
    print("ds_read_b32 cycles/instr:", round(base, 2), {s: round(v, 2) for s, v in by_stride.items()}, flush=True)
    assert _c("b32", 65) < 1.2 * base                      # odd stride: every lane in its own bank
    assert by_stride[2] > 1.2 * base                       # stride 2: lanes share banks
    seq = [base] + [by_stride[s] for s in (2, 4, 8, 16, 32)]
    assert all(b >= 0.95 * a for a, b in zip(seq, seq[1:]))  # never cheaper as the stride doubles
    assert by_stride[32] > 8 * base and by_stride[64] > 8 * base
    b128 = _c("b128", 4)
    assert _c("b128", 64) > 4 * b128


def test_gemm_fragment_reads_conflict_free_with_swizzle():
    tss.lds_probe("b128", 4, iters=50)  # warm-up
    b128, tr = _c("b128", 4), _c("tr_b64", 2)
    a, a_plain = _c("gemm_a"), _c("gemm_a_plain")
    b, b_plain = _c("gemm_b"), _c("gemm_b_plain")
    print(f"A fragment {a:.2f} (no swizzle {a_plain:.2f}, contiguous b128 {b128:.2f}); "
          f"B fragment {b:.2f} (no swizzle {b_plain:.2f}, contiguous tr {tr:.2f})", flush=True)
    # a two-way conflict costs about 1.5x (the stride-2 row of the table); the
    # swizzled reads stay below that, and the same reads without the swizzle
    # (3-4x) cost more than twice as much
    assert a < 1.4 * b128 and b < 1.4 * tr
    assert a_plain > 2 * a and b_plain > 2 * b
