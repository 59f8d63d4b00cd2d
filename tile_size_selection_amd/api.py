"""Python front end of libtss: argument marshalling only.  Every step of the
GEMM / convolution runs in the HIP kernels; torch supplies device memory and
the stream."""
from __future__ import annotations

import ctypes
import functools
from dataclasses import dataclass
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple, Union

from . import _capi as C

try:
    import torch
except ImportError:  # the planner needs no torch
    torch = None


@dataclass(frozen=True)
class TileConfig:
    bm: int
    bn: int
    bk: int
    stages: int
    threads: int
    instr: str = "mfma32"

    def c(self) -> C.TileConfig:
        if self.instr not in C.INSTR:
            raise ValueError(f"unknown instruction shape {self.instr!r}")
        return C.TileConfig(self.bm, self.bn, self.bk, self.stages, self.threads, C.INSTR[self.instr])

    @staticmethod
    def from_c(c: C.TileConfig) -> "TileConfig":
        return TileConfig(c.bm, c.bn, c.bk, c.stages, c.threads, C.INSTR_NAME.get(c.instr, str(c.instr)))


def device_gfx950() -> C.Device:
    d = C.Device()
    C.check(C.lib().tss_device_gfx950(ctypes.byref(d)), "tss_device_gfx950")
    return d


def device_pages(sm_count: int = 132, smem_kb: int = 228) -> C.Device:
    d = C.Device()
    C.check(C.lib().tss_device_pages(sm_count, smem_kb, ctypes.byref(d)), "tss_device_pages")
    return d


def device_query(hip_device: int = 0) -> C.Device:
    d = C.Device()
    C.check(C.lib().tss_device_query(hip_device, ctypes.byref(d)), "tss_device_query")
    return d


def verdict_dict(v: C.Verdict) -> dict:
    num = (v.traffic_num_hi << 64) | v.traffic_num_lo
    return {
        "config": TileConfig.from_c(v.cfg),
        "smem_per_stage": v.smem_per_stage, "smem_total": v.smem_total,
        "accum_per_thread": v.accum_per_thread, "regs_per_thread": v.regs_per_thread,
        "regs_per_block": v.regs_per_block, "blocks_by_regs": v.blocks_by_regs,
        "blocks_by_smem": v.blocks_by_smem, "blocks_by_threads": v.blocks_by_threads,
        "blocks_per_core": v.blocks_per_core, "grid": v.grid, "waves": v.waves,
        "fill": Fraction(v.fill_num, v.fill_den) if v.fill_den else Fraction(0),
        "traffic": Fraction(num, v.traffic_den) if v.traffic_den else Fraction(0),
        "traffic_rounded": v.traffic_rounded,
        "failures": [n for i, n in enumerate(C.FAIL_BITS) if v.failures >> i & 1],
        "warnings": [n for i, n in enumerate(C.WARN_BITS) if v.warnings >> i & 1],
        "binding": C.BINDING.get(v.binding, "?"),
    }


def evaluate(cfg: TileConfig, M: int, N: int, K: int, batch: int = 1, elem_bytes: int = 2,
             dev: Optional[C.Device] = None) -> dict:
    v = C.Verdict()
    C.check(C.lib().tss_evaluate(ctypes.byref(cfg.c()), ctypes.byref(dev) if dev is not None else None,
                                 batch, M, N, K, elem_bytes, ctypes.byref(v)), "tss_evaluate")
    return verdict_dict(v)


def tile_plan(M: int, N: int, K: int, batch: int = 1, elem_bytes: int = 2, dev: Optional[C.Device] = None,
              instr: Optional[str] = None, cap: int = 0) -> Tuple[Optional[dict], List[dict], int]:
    """(best verdict or None, the first `cap` ranked verdicts, number feasible)."""
    best = C.Verdict()
    lst = (C.Verdict * max(cap, 1))()
    n = C.i32(0)
    st = C.lib().tss_tile_plan(batch, M, N, K, elem_bytes, ctypes.byref(dev) if dev is not None else None,
                               C.INSTR[instr] if instr else 0, ctypes.byref(best), lst if cap else None, cap,
                               ctypes.byref(n))
    if st == C.TSS_E_INFEASIBLE:
        return None, [], 0
    C.check(st, "tss_tile_plan")
    return verdict_dict(best), [verdict_dict(lst[i]) for i in range(min(cap, n.value))], n.value


def conv_plan(Cout: int, pixels: int, channels: int, taps: int, elem_bytes: int = 2,
              cap: int = 0, dev: Optional[C.Device] = None) -> Tuple[Optional[dict], List[dict], int]:
    """tss_conv_plan: the gfx950 plan of a convolution's implicit GEMM (M =
    Cout, N = output pixels), each candidate with the K its kernel computes,
    taps * ceil(channels / BK) * BK.  dev: a gfx950-ranked device (its cost
    parameters), None = the gfx950 model.  (best or None, first `cap`
    ranked, n feasible)."""
    best = C.Verdict()
    lst = (C.Verdict * max(cap, 1))()
    n = C.i32(0)
    st = C.lib().tss_conv_plan(Cout, pixels, channels, taps, elem_bytes, ctypes.byref(dev) if dev is not None else None,
                               ctypes.byref(best), lst if cap else None, cap, ctypes.byref(n))
    return _plan_result(st, best, lst, cap, n, "tss_conv_plan")


def splitk_plan(M: int, N: int, K: int, batch: int = 1, elem_bytes: int = 2, dev: Optional[C.Device] = None,
                splits: int = 0) -> Tuple[int, dict]:
    """tss_splitk_plan: (split count, verdict of the tile for the split
    problem); splits > 0 plans the tile for that count only."""
    v, S = C.Verdict(), C.i32(splits)
    C.check(C.lib().tss_splitk_plan(batch, M, N, K, elem_bytes, ctypes.byref(dev) if dev is not None else None,
                                    ctypes.byref(v), ctypes.byref(S)), "tss_splitk_plan")
    return S.value, verdict_dict(v)


def conv_splitk_plan(Cout: int, pixels: int, channels: int, taps: int, elem_bytes: int = 2,
                     dev: Optional[C.Device] = None, splits: int = 0) -> Tuple[int, dict]:
    """tss_conv_splitk_plan: as splitk_plan for a convolution's implicit GEMM."""
    v, S = C.Verdict(), C.i32(splits)
    C.check(C.lib().tss_conv_splitk_plan(Cout, pixels, channels, taps, elem_bytes,
                                         ctypes.byref(dev) if dev is not None else None, ctypes.byref(v),
                                         ctypes.byref(S)), "tss_conv_splitk_plan")
    return S.value, verdict_dict(v)


@functools.lru_cache(maxsize=4096)
def _planned_splits(conv: bool, a: int, b: int, c: int, d: int) -> int:
    """The split-K plan's count for sizing a workspace, cached per problem as
    the library caches its own plan (planning evaluates every candidate at
    every count, far longer than a launch).  conv: (Cout, pixels, C, taps);
    else (batch, M, N, K)."""
    if conv:
        return conv_splitk_plan(a, b, c, d)[0]
    return splitk_plan(b, c, d, batch=a)[0]


def conv2d_default_config(N: int, channels: int, H: int, W: int, Cout: int, kh: int, kw: int,
                          stride: Union[int, Sequence[int]] = 1, padding: Union[int, Sequence[int]] = 0,
                          dilation: Union[int, Sequence[int]] = 1) -> TileConfig:
    """The tile conv2d launches when no cfg is given: tss_conv_plan over the
    whole problem's output pixels."""
    pair = lambda v: (v, v) if isinstance(v, int) else tuple(v)
    (sh, sw), (ph, pw), (dh, dw) = pair(stride), pair(padding), pair(dilation)
    OH = (H + 2 * ph - (kh - 1) * dh - 1) // sh + 1
    OW = (W + 2 * pw - (kw - 1) * dw - 1) // sw + 1
    best, _, _ = conv_plan(Cout, N * OH * OW, channels, kh * kw)
    if best is None:
        raise RuntimeError("no feasible tile for this convolution")
    return best["config"]


def _plan_result(st, best, lst, cap, n, where):
    if st == C.TSS_E_INFEASIBLE:
        return None, [], 0
    C.check(st, where)
    return verdict_dict(best), [verdict_dict(lst[i]) for i in range(min(cap, n.value))], n.value


def tile_plan_usage(M: int, N: int, K: int, usage: dict, batch: int = 1, elem_bytes: int = 2,
                    cap: int = 0) -> Tuple[Optional[dict], List[dict], int]:
    """tss_tile_plan_usage: the gfx950 plan with each candidate's occupancy
    taken from its compiled kernel's registers per lane, and kernels that
    spill failing C2; usage = {TileConfig: (registers per lane, scratch bytes
    per lane)}."""
    table = (C.MeasuredUsage * max(len(usage), 1))()
    for i, (cfg, (r, sc)) in enumerate(usage.items()):
        table[i].cfg = cfg.c()
        table[i].regs_per_lane = int(r)
        table[i].scratch_bytes = int(sc)
    best, lst, n = C.Verdict(), (C.Verdict * max(cap, 1))(), C.i32(0)
    st = C.lib().tss_tile_plan_usage(batch, M, N, K, elem_bytes, table if usage else None, len(usage),
                                     ctypes.byref(best), lst if cap else None, cap, ctypes.byref(n))
    return _plan_result(st, best, lst, cap, n, "tss_tile_plan_usage")


def kernel_usage(cfg: TileConfig, dtype: str = "f16", op: str = "gemm") -> dict:
    """tss_kernel_usage_query: what the compiled kernel uses (needs a GPU)."""
    u = C.KernelUsage()
    C.check(C.lib().tss_kernel_usage_query(ctypes.byref(cfg.c()), _DT[dtype], 0 if op == "gemm" else 1,
                                           ctypes.byref(u)), "tss_kernel_usage_query")
    return {f: getattr(u, f) for f, _ in C.KernelUsage._fields_ if f != "pad_"}


def tile_plan_measured(M: int, N: int, K: int, batch: int = 1, dtype: str = "f16", op: str = "gemm",
                       cap: int = 0) -> Tuple[Optional[dict], List[dict], int]:
    """tss_tile_plan_measured: tile_plan_usage with every compiled kernel's
    usage read from its code object (needs a GPU)."""
    best, lst, n = C.Verdict(), (C.Verdict * max(cap, 1))(), C.i32(0)
    st = C.lib().tss_tile_plan_measured(batch, M, N, K, _DT[dtype], 0 if op == "gemm" else 1, ctypes.byref(best),
                                        lst if cap else None, cap, ctypes.byref(n))
    return _plan_result(st, best, lst, cap, n, "tss_tile_plan_measured")


def lds_probe(pattern: str, stride_words: int = 1, iters: int = 2000, blocks: int = 256, stream=None) -> float:
    """tss_lds_probe: shader-clock cycles per LDS read instruction of one wave
    (median over every wave of the launch) for an access pattern; see
    LDS_PATTERN in _capi for the names.  Needs a GPU."""
    if torch is None:
        raise RuntimeError("lds_probe needs torch for its device buffer")
    cycles = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    C.check(C.lib().tss_lds_probe(C.LDS_PATTERN[pattern], stride_words, iters, blocks, cycles.data_ptr(),
                                  _stream_ptr(stream)), "tss_lds_probe")
    torch.cuda.synchronize()
    c = cycles.cpu()
    if bool((c <= 0).any()):
        raise RuntimeError("lds_probe: a wave reported no cycles")
    return float(c.double().median()) / (iters * 8)


def hw_tile(H: int, kh: int, sh: int, pt: int, d: int, o0: int, o1: int) -> dict:
    s = C.HwSlice()
    C.check(C.lib().tss_hw_tile(H, kh, sh, pt, d, o0, o1, ctypes.byref(s)), "tss_hw_tile")
    return {f: getattr(s, f) for f, _ in C.HwSlice._fields_}


def kernel_available(cfg: TileConfig, dtype: str = "f16", op: str = "gemm") -> bool:
    return bool(C.lib().tss_kernel_available(ctypes.byref(cfg.c()), _DT[dtype], 0 if op == "gemm" else 1))


def default_config(M: int, N: int, K: int, batch: int = 1, dtype: str = "f16") -> TileConfig:
    c = C.TileConfig()
    C.check(C.lib().tss_gemm_default_config(batch, M, N, K, _DT[dtype], ctypes.byref(c)), "tss_gemm_default_config")
    return TileConfig.from_c(c)


_DT = {"f16": C.TSS_F16, "bf16": C.TSS_BF16, "f32": C.TSS_F32}


def _dt_of(t) -> str:
    names = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
    if t.dtype not in names:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return names[t.dtype]


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _same_device(*tensors):
    """Every tensor a device tensor on one GPU; returns that device.  (A host
    or other-device pointer handed to a kernel would fault.)"""
    dev = tensors[0].device
    for t in tensors:
        if not t.is_cuda or t.device != dev:
            raise ValueError("every tensor must be on the same GPU")
    return dev


def _check_gemm_operands(A, B):
    """(batch, M, N, K, dtype) of row-major device operands A [b,] M x K and
    B [b,] K x N, or ValueError."""
    if A.dim() not in (2, 3) or B.dim() != A.dim():
        raise ValueError("A and B must both be 2-D or both 3-D")
    if A.dtype != B.dtype:
        raise ValueError("A and B must share a dtype")
    if not (A.is_cuda and B.is_cuda and A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous device tensors")
    batched = A.dim() == 3
    bt = A.shape[0] if batched else 1
    M, K = A.shape[-2], A.shape[-1]
    K2, N = B.shape[-2], B.shape[-1]
    if K != K2 or (batched and B.shape[0] != bt):
        raise ValueError(f"shape mismatch {tuple(A.shape)} x {tuple(B.shape)}")
    return bt, M, N, K, _dt_of(A)


def _gemm_out(out, bt: int, M: int, N: int, od: str, A):
    """The caller's output tensor (checked) or a new one, [b,] M x N of od."""
    shape = (bt, M, N) if A.dim() == 3 else (M, N)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[od]
    if out is None:
        return torch.empty(shape, dtype=tdt, device=A.device)
    if tuple(out.shape) != shape or out.dtype != tdt or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    return out


def gemm(A, B, out_dtype: Optional[str] = None, cfg: Optional[TileConfig] = None, out=None, stream=None,
         splits: int = 1, workspace=None):
    """C = A @ B for row-major fp16/bf16 device tensors, A [b,] M x K and
    B [b,] K x N; fp32 accumulation; out_dtype 'f32' or the input dtype
    (default: the input dtype).  splits > 1: split K into at most that many
    ranges (tss_gemm_splitk), 0: as many as the split-K plan says, with
    `workspace` (a device tensor of at least gemm_splitk_workspace_size
    bytes; allocated here when not given)."""
    bt, M, N, K, dt = _check_gemm_operands(A, B)
    od = out_dtype or dt
    out = _gemm_out(out, bt, M, N, od, A)
    if splits == 1:
        with torch.cuda.device(_same_device(A, B, out)):
            st = C.lib().tss_gemm(M, N, K, _DT[dt], A.data_ptr(), B.data_ptr(), out.data_ptr(), bt, _DT[od],
                                  ctypes.byref(cfg.c()) if cfg else None, _stream_ptr(stream))
        C.check(st, "tss_gemm")
        return out
    # splits == 0: the library plans the count; the workspace is sized for it
    need = gemm_splitk_workspace_size(bt, M, N, splits or _planned_splits(False, bt, M, N, K))
    workspace = _workspace(workspace, need, A.device)
    with torch.cuda.device(_same_device(A, B, out, workspace)):
        st = C.lib().tss_gemm_splitk(M, N, K, _DT[dt], A.data_ptr(), B.data_ptr(), out.data_ptr(), bt, _DT[od],
                                     ctypes.byref(cfg.c()) if cfg else None, splits, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    C.check(st, "tss_gemm_splitk")
    return out


def gemm_splitk_workspace_size(batch: int, M: int, N: int, splits: int) -> int:
    n = C.lib().tss_gemm_splitk_workspace_size(batch, M, N, splits)
    if n < 0:
        C.check(int(n), "tss_gemm_splitk_workspace_size")
    return int(n)


def autotune_gemm(A, B, out_dtype: Optional[str] = None, topk: int = 64, iters: int = 10, out=None,
                  stream=None) -> Tuple[TileConfig, float]:
    """tss_gemm_autotune: time the planner's first `topk` candidates on these
    operands (blocking) and return (the fastest tile, its microseconds per
    launch); pass the tile to gemm(..., cfg=...)."""
    bt, M, N, K, dt = _check_gemm_operands(A, B)
    od = out_dtype or dt
    out = _gemm_out(out, bt, M, N, od, A)
    best = C.TileConfig()
    us = ctypes.c_float(0.0)
    with torch.cuda.device(_same_device(A, B, out)):
        st = C.lib().tss_gemm_autotune(M, N, K, _DT[dt], A.data_ptr(), B.data_ptr(), out.data_ptr(), bt, _DT[od],
                                       topk, iters, _stream_ptr(stream), ctypes.byref(best), ctypes.byref(us))
    C.check(st, "tss_gemm_autotune")
    return TileConfig.from_c(best), float(us.value)


def _workspace(workspace, need: int, device):
    """The caller's workspace (checked), or a new one from torch's caching
    allocator (device memory; the launches that use it are on one stream)."""
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not (workspace.is_cuda and workspace.is_contiguous() and workspace.numel() * workspace.element_size() >= need):
        raise ValueError(f"workspace must be a contiguous device tensor of at least {need} bytes")
    return workspace


def conv2d_noalloc(x, w, stride: Union[int, Sequence[int]] = 1, padding: Union[int, Sequence[int]] = 0,
                   dilation: Union[int, Sequence[int]] = 1, tile_oh: Optional[int] = None,
                   out_dtype: Optional[str] = None, cfg: Optional[TileConfig] = None, out=None, stream=None,
                   tile_ow: Optional[int] = None, tile_n: Optional[int] = None, splits: int = 1):
    """conv2d through tss_conv2d_splitk_noalloc: the workspace is the
    library's static device array (no allocation by the library; `out` must
    be given, so nothing is allocated here either).  Calls on one GPU share
    the array and must not overlap."""
    pair = lambda v: (v, v) if isinstance(v, int) else tuple(v)
    (sh, sw), (ph, pw), (dh, dw) = pair(stride), pair(padding), pair(dilation)
    if x.dim() != 4 or w.dim() != 4 or x.dtype != w.dtype:
        raise ValueError("x must be NCHW and w OIHW, same dtype")
    if out is None:
        raise ValueError("out must be given")
    N, Ci, H, W = x.shape
    Co, _, kh, kw = w.shape
    OH = (H + 2 * ph - (kh - 1) * dh - 1) // sh + 1
    OW = (W + 2 * pw - (kw - 1) * dw - 1) // sw + 1
    dt = _dt_of(x)
    od = _dt_of(out)
    if out_dtype is not None and out_dtype != od:
        raise ValueError("out_dtype and out disagree")
    if tuple(out.shape) != (N, Co, OH, OW) or not (x.is_contiguous() and w.is_contiguous() and out.is_contiguous()):
        raise ValueError("x, w, out must be contiguous, out of shape (N, Cout, OH, OW)")
    with torch.cuda.device(_same_device(x, w, out)):
        st = C.lib().tss_conv2d_splitk_noalloc(N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, tile_n or N,
                                               tile_oh or OH, tile_ow or OW, _DT[dt], _DT[od], x.data_ptr(),
                                               w.data_ptr(), out.data_ptr(), splits,
                                               ctypes.byref(cfg.c()) if cfg else None, _stream_ptr(stream))
    C.check(st, "tss_conv2d_splitk_noalloc")
    return out


def conv2d_workspace_size(N: int, Ci: int, H: int, W: int, Cout: int, kh: int, kw: int) -> int:
    """Bytes of device workspace tss_conv2d needs for these sizes (Ci input
    channels)."""
    n = C.lib().tss_conv2d_workspace_size(N, Ci, H, W, Cout, kh, kw)
    if n < 0:
        C.check(int(n), "tss_conv2d_workspace_size")
    return int(n)


def conv2d(x, w, stride: Union[int, Sequence[int]] = 1, padding: Union[int, Sequence[int]] = 0,
           dilation: Union[int, Sequence[int]] = 1, tile_oh: Optional[int] = None, out_dtype: Optional[str] = None,
           cfg: Optional[TileConfig] = None, out=None, stream=None, workspace=None, tile_ow: Optional[int] = None,
           tile_n: Optional[int] = None, splits: int = 1, layout: Optional[str] = None):
    """Convolution as an implicit GEMM over tiles of tile_n images x tile_oh
    output rows x tile_ow output columns (defaults: the whole batch, height
    and width).  x is (N, C, H, W), w (Cout, C, kh, kw), the result
    (N, Cout, OH, OW), in one of two memory layouts:
      layout "nchw": contiguous x, w and result (tss_conv2d_tiled; the
        operands are first rewritten into channel-last copies in
        `workspace`, an optional device tensor of at least
        conv2d_workspace_size(...) bytes, allocated here when not given;
        with twice that, consecutive calls alternate between two sets of the
        operand copies, which runs the layout pass faster);
      layout "nhwc": x, w and the result in torch's channels_last format
        (stored [N][H][W][C], [Cout][kh][kw][C], [N][OH][OW][Cout]), read and
        written in place (tss_conv2d_nhwc; C a multiple of 8; the workspace
        holds only split-K partial outputs).
    layout None: "nhwc" when x and w are channels_last and not both also
    plain contiguous (a tensor with H = W = 1 or C = 1 is both).
    splits > 1: the K loop cut into at most that many ranges (the workspace
    then also holds their partial outputs); 0: the split-K plan's count."""
    pair = lambda v: (v, v) if isinstance(v, int) else tuple(v)
    (sh, sw), (ph, pw), (dh, dw) = pair(stride), pair(padding), pair(dilation)
    if x.dim() != 4 or w.dim() != 4 or x.dtype != w.dtype:
        raise ValueError("x must be (N, C, H, W) and w (Cout, C, kh, kw), same dtype")
    cl = torch.channels_last
    if layout is None:
        both_cl = x.is_contiguous(memory_format=cl) and w.is_contiguous(memory_format=cl)
        layout = "nhwc" if both_cl and not (x.is_contiguous() and w.is_contiguous()) else "nchw"
    if layout not in ("nchw", "nhwc"):
        raise ValueError("layout must be 'nchw' or 'nhwc'")
    nhwc = layout == "nhwc"
    fmt = cl if nhwc else torch.contiguous_format
    if not (x.is_cuda and w.is_cuda and x.is_contiguous(memory_format=fmt) and w.is_contiguous(memory_format=fmt)):
        raise ValueError("x and w must be device tensors, contiguous in the " +
                         ("channels_last" if nhwc else "NCHW") + " memory format")
    N, Ci, H, W = x.shape
    Co, Ci2, kh, kw = w.shape
    if Ci != Ci2:
        raise ValueError("channel mismatch")
    OH = (H + 2 * ph - (kh - 1) * dh - 1) // sh + 1
    OW = (W + 2 * pw - (kw - 1) * dw - 1) // sw + 1
    dt = _dt_of(x)
    od = out_dtype or dt
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[od]
    shape = (N, Co, OH, OW)
    if out is None:
        out = torch.empty(shape, dtype=tdt, device=x.device, memory_format=fmt)
    elif tuple(out.shape) != shape or out.dtype != tdt or not out.is_contiguous(memory_format=fmt):
        raise ValueError("out has the wrong shape, dtype or layout")
    if nhwc:
        n_splits = splits or _planned_splits(True, Co, N * OH * OW, Ci, kh * kw)
        ws_bytes = C.lib().tss_conv2d_nhwc_workspace_size(N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, n_splits)
        if ws_bytes < 0:
            C.check(int(ws_bytes), "tss_conv2d_nhwc_workspace_size")
        workspace = _workspace(workspace, ws_bytes, x.device) if ws_bytes else workspace
        with torch.cuda.device(_same_device(x, w, out, *(() if workspace is None else (workspace,)))):
            st = C.lib().tss_conv2d_nhwc(
                N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, tile_n or N, tile_oh or OH, tile_ow or OW, _DT[dt],
                _DT[od], x.data_ptr(), w.data_ptr(), out.data_ptr(), splits,
                workspace.data_ptr() if workspace is not None else None,
                workspace.numel() * workspace.element_size() if workspace is not None else 0,
                ctypes.byref(cfg.c()) if cfg else None, _stream_ptr(stream))
        C.check(st, "tss_conv2d_nhwc")
        return out
    if splits == 1:
        ws_bytes = conv2d_workspace_size(N, Ci, H, W, Co, kh, kw)
    else:
        n_splits = splits or _planned_splits(True, Co, N * OH * OW, Ci, kh * kw)
        ws_bytes = C.lib().tss_conv2d_splitk_workspace_size(N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw,
                                                            n_splits)
        if ws_bytes < 0:
            C.check(int(ws_bytes), "tss_conv2d_splitk_workspace_size")
    # torch's caching allocator when none is given: device memory only, no
    # host copy; the convolution's launches fill and read it on one stream.
    # Allocated here, it has room for a second set of the operand copies, so
    # that consecutive calls alternate between the two (tss_conv2d).
    if workspace is None:
        ws_bytes += (conv2d_workspace_size(N, Ci, H, W, Co, kh, kw) + 255) // 256 * 256
    workspace = _workspace(workspace, ws_bytes, x.device)
    with torch.cuda.device(_same_device(x, w, out, workspace)):
        args = (N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, tile_n or N, tile_oh or OH, tile_ow or OW, _DT[dt],
                _DT[od], x.data_ptr(), w.data_ptr(), out.data_ptr())
        tail = (workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                ctypes.byref(cfg.c()) if cfg else None, _stream_ptr(stream))
        if splits == 1:
            st = C.lib().tss_conv2d_tiled(*args, *tail)
        else:
            st = C.lib().tss_conv2d_splitk(*args, splits, *tail)
    C.check(st, "tss_conv2d_tiled" if splits == 1 else "tss_conv2d_splitk")
    return out
