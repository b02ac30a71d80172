"""Python binding of the tkg C ABI (``include/tkg.h``): tiled dense GEMM on
AMD MI355X (gfx950).

Argument marshalling only: every step of the product runs in the HIP
kernels of ``libtkg.so``. torch supplies device memory and the current
stream. Names match the C entry points: ``gemm_bf16``, ``gemm_fp8``,
``gemm_fp4_blockscaled``, ``tkg_gemm_ex`` and ``tkg_status_string``.

Operand layouts: ``A`` is M x K row-major; ``B`` is passed column-major,
i.e. as an N x K row-major tensor ``Bt``; the result is an M x N row-major
bf16 tensor. There is no CPU fallback: importing works without a GPU (the
library loads), but every product needs the HIP device.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "gemm_bf16", "gemm_fp8", "gemm_fp4_blockscaled", "tkg_gemm_ex",
    "tkg_status_string", "lds_fragment_offsets", "lds_fragment_rows",
    "lds_row_bytes", "lib",
    "TkgError", "DTYPE_BF16", "DTYPE_FP8", "DTYPE_FP4_BLOCKSCALED",
    "DTYPE_MXFP4", "DTYPE_MXFP8", "gemm_mxfp4", "gemm_mxfp8",
    "STATUS", "LIB_PATH", "tkg_attention_fwd", "attn_lds_offsets",
    "num_variants", "variant_info", "launch_masked", "gemm_splitk", "device_info",
    "splitk_workspace_size", "splitk_count", "gemm_splitk_noalloc",
    "NOALLOC_SCRATCH_BYTES", "plan_launch", "tile_order",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtkg.so")

DTYPE_BF16, DTYPE_FP8, DTYPE_FP4_BLOCKSCALED = 0, 1, 2
DTYPE_MXFP4, DTYPE_MXFP8 = 3, 4
STATUS = {"TKG_OK": 0, "TKG_ERR_NULL": -1, "TKG_ERR_SHAPE": -2,
          "TKG_ERR_ALIGN": -3, "TKG_ERR_LAUNCH": -4, "TKG_ERR_DEVICE": -5,
          "TKG_ERR_WORKSPACE": -6, "TKG_ERR_VALUE": -7}


class TkgError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = int(status)
        super().__init__("%s%s" % (what + ": " if what else "",
                                   tkg_status_string(status)))


class TkgOpts(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("xcd_remap", ctypes.c_int32), ("variant", ctypes.c_int32)]


class LaunchPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "variant", "tile", "tiles", "grid", "group_m", "xcd_remap", "units",
        "tail_variant", "tail_units", "tail_grid")]


class VariantDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "stage_kbytes", "slots", "waves", "load_waves", "mfma_block", "tile",
        "per_cu", "swizzle", "schedule")]


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (same soname as ROCm's). Loading torch
    # first makes libtkg bind to that one, so the library and torch share
    # one runtime (devices, streams, memory) in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libtkg.so is not built (%s); run `python "
            "tiled_dense_gemm_amd/_build.py`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    L.gemm_bf16.argtypes = [i64, i64, i64, vp, vp, vp, vp]
    L.gemm_bf16.restype = i32
    L.gemm_fp8.argtypes = [i64, i64, i64, vp, f32, vp, f32, vp, vp]
    L.gemm_fp8.restype = i32
    L.gemm_fp4_blockscaled.argtypes = [i64, i64, i64, vp, vp, f32, vp, vp,
                                       f32, vp, vp]
    L.gemm_fp4_blockscaled.restype = i32
    for name in ("gemm_mxfp4", "gemm_mxfp8"):
        getattr(L, name).argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        getattr(L, name).restype = i32
    L.tkg_gemm_ex.argtypes = [i32, i64, i64, i64, vp, vp, f32, vp, vp, f32,
                              vp, vp, ctypes.POINTER(TkgOpts)]
    L.tkg_gemm_ex.restype = i32
    L.tkg_status_string.argtypes = [i32]
    L.tkg_status_string.restype = ctypes.c_char_p
    L.tkg_lds_fragment_offsets.argtypes = [i32, i32, i32, i32,
                                           ctypes.POINTER(ctypes.c_uint32)]
    L.tkg_lds_fragment_offsets.restype = i32
    L.tkg_lds_row_bytes.argtypes = [i32]
    L.tkg_lds_row_bytes.restype = i32
    L.tkg_lds_fragment_rows.argtypes = [i32]
    L.tkg_lds_fragment_rows.restype = i32
    L.tkg_lds_finish_offsets.argtypes = [i32, i32, i32, i32,
                                         ctypes.POINTER(ctypes.c_uint32)]
    L.tkg_lds_finish_offsets.restype = i32
    L.tkg_gemm_splitk.argtypes = [i32, i64, i64, i64, vp, f32, vp, f32, vp, vp,
                                  ctypes.c_size_t, i32, vp]
    L.tkg_gemm_splitk.restype = i32
    L.tkg_gemm_splitk_noalloc.argtypes = [i32, i64, i64, i64, vp, f32, vp, f32, vp, i32, vp]
    L.tkg_gemm_splitk_noalloc.restype = i32
    L.tkg_gemm_splitk_workspace_size.argtypes = [i32, i64, i64, i64, i32]
    L.tkg_gemm_splitk_workspace_size.restype = i64
    L.tkg_gemm_splitk_count.argtypes = [i32, i64, i64, i64, i32]
    L.tkg_gemm_splitk_count.restype = i32
    L.tkg_attention_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                    i64, i64, f32, i32, vp]
    L.tkg_attention_fwd.restype = i32
    L.tkg_attn_lds_offsets.argtypes = [i32, i32, i32, i32, i32, i32,
                                       ctypes.POINTER(ctypes.c_uint32)]
    L.tkg_attn_lds_offsets.restype = i32
    L.tkg_variant_info.argtypes = [i32, i32, ctypes.POINTER(VariantDesc)]
    L.tkg_variant_info.restype = i32
    L.tkg_launch_masked.argtypes = [i32, i64, i64, i64, i32]
    L.tkg_launch_masked.restype = i32
    L.tkg_tile_order.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                 ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.tkg_tile_order.restype = i32
    L.tkg_plan_launch.argtypes = [i32, i64, i64, i64, ctypes.POINTER(TkgOpts), i32,
                                  ctypes.POINTER(LaunchPlan)]
    L.tkg_plan_launch.restype = i32
    L.tkg_device_info.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.tkg_device_info.restype = i32
    return L


lib = _load()


def attn_lds_offsets(d: int, kind: int, i0=0, i1=0, i2=0, i3=0):
    """The 64 per-lane LDS (or copy source) offsets of the attention
    kernel's ring (``tkg_attn_lds_offsets``); no GPU work."""
    out = (ctypes.c_uint32 * 64)()
    st = lib.tkg_attn_lds_offsets(d, kind, i0, i1, i2, i3, out)
    if st != 0:
        raise TkgError(st, "tkg_attn_lds_offsets")
    return list(out)


def tkg_status_string(status: int) -> str:
    return lib.tkg_status_string(int(status)).decode()


SCHEDULES = {0: "interleaved", 1: "early B release", 2: "ping-pong", 3: "early reads"}


def num_variants(dtype: int) -> int:
    """Kernel configurations of a dtype (``tkg_variant_info``)."""
    r = lib.tkg_variant_info(int(dtype), 0, None)
    if r < 0:
        raise TkgError(r, "tkg_variant_info")
    return r


def variant_info(dtype: int, variant: int) -> dict:
    """The configuration behind ``variant`` of a dtype (see tkg.h)."""
    d = VariantDesc()
    r = lib.tkg_variant_info(int(dtype), int(variant), ctypes.byref(d))
    if r < 0:
        raise TkgError(r, "tkg_variant_info")
    out = {n: getattr(d, n) for n, _ in VariantDesc._fields_}
    out["schedule_name"] = SCHEDULES.get(d.schedule, "?")
    return out


def launch_masked(dtype: int, M: int, N: int, K: int, variant: int = 0) -> bool:
    """Whether the launch runs the masked kernel instance (every load
    bounds-checked per lane; ``tkg_launch_masked``). No GPU work."""
    r = lib.tkg_launch_masked(int(dtype), int(M), int(N), int(K), int(variant))
    if r < 0:
        raise TkgError(r, "tkg_launch_masked")
    return bool(r)


def plan_launch(dtype: int, M: int, N: int, K: int, cus: int = 256, grid: int = 0,
                group_m: int = 0, xcd_remap: int = 1, variant: int = 0) -> dict:
    """The launch ``tkg_gemm_ex`` makes with these options on a device of
    ``cus`` compute units (``tkg_plan_launch``): configuration, tile edge,
    tile count, grid and tile order. No GPU work."""
    o = TkgOpts(int(grid), int(group_m), int(xcd_remap), int(variant))
    p = LaunchPlan()
    r = lib.tkg_plan_launch(int(dtype), int(M), int(N), int(K), ctypes.byref(o), int(cus),
                            ctypes.byref(p))
    if r < 0:
        raise TkgError(r, "tkg_plan_launch")
    return {n: getattr(p, n) for n, _ in LaunchPlan._fields_}


def device_info() -> dict:
    """The current device's compute units and peak shader clock
    (``tkg_device_info``): {"cus": int, "peak_clock_mhz": float}."""
    cus, clk = ctypes.c_int32(), ctypes.c_int32()
    r = lib.tkg_device_info(ctypes.byref(cus), ctypes.byref(clk))
    if r < 0:
        raise TkgError(r, "tkg_device_info")
    return {"cus": cus.value, "peak_clock_mhz": clk.value / 1000.0}


def tile_order(t: int, grid: int, xcd_remap: int, tiles_m: int, tiles_n: int,
               group_m: int, quad_base: int = -1):
    """(tile row, tile column) of work item t in the kernels' persistent
    order (``tkg_tile_order``; quad_base >= 0: a tail-launch quadrant). No
    GPU work."""
    pm, pn = ctypes.c_int32(), ctypes.c_int32()
    r = lib.tkg_tile_order(int(t), int(grid), int(xcd_remap), int(tiles_m), int(tiles_n),
                           int(group_m), int(quad_base), ctypes.byref(pm), ctypes.byref(pn))
    if r < 0:
        raise TkgError(r, "tkg_tile_order")
    return pm.value, pn.value


def lds_row_bytes(dtype: int) -> int:
    r = lib.tkg_lds_row_bytes(int(dtype))
    if r < 0:
        raise TkgError(r, "tkg_lds_row_bytes")
    return r


def lds_fragment_rows(dtype: int) -> int:
    r = lib.tkg_lds_fragment_rows(int(dtype))
    if r < 0:
        raise TkgError(r, "tkg_lds_fragment_rows")
    return r


def lds_fragment_offsets(dtype: int, step: int, part: int, frag: int):
    """The 64 per-lane LDS byte offsets of one fragment read (see tkg.h)."""
    buf = (ctypes.c_uint32 * 64)()
    r = lib.tkg_lds_fragment_offsets(int(dtype), int(step), int(part),
                                     int(frag), buf)
    if r < 0:
        raise TkgError(r, "tkg_lds_fragment_offsets")
    return list(buf)


def lds_finish_offsets(mi: int, rj: int, kind: int, index: int):
    """The 64 per-lane LDS byte offsets of one access of the finish's
    staging strip (see tkg.h); kind 0 = write, 1 = read."""
    buf = (ctypes.c_uint32 * 64)()
    r = lib.tkg_lds_finish_offsets(int(mi), int(rj), int(kind), int(index), buf)
    if r < 0:
        raise TkgError(r, "tkg_lds_finish_offsets")
    return list(buf)


def lds_finish_count(mi: int, rj: int, kind: int) -> int:
    """Writes (kind 0) or reads (kind 1) per round of the finish strip."""
    buf = (ctypes.c_uint32 * 64)()
    r = lib.tkg_lds_finish_offsets(int(mi), int(rj), int(kind), 0, buf)
    if r < 0:
        raise TkgError(r, "tkg_lds_finish_offsets")
    return r


# ------------------------------------------------------------ torch layer

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_mat(x, name, rows, cols, dtypes, device):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s"
                        % (name, x.dtype, dtypes))
    if x.dim() != 2 or tuple(x.shape) != (rows, cols):
        raise ValueError("%s has shape %s, expected (%d, %d)"
                         % (name, tuple(x.shape), rows, cols))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.device.type != "cuda" or (device is not None and x.device != device):
        raise ValueError("%s must be on the GPU (%s)" % (name, device))


def _out(out, M, N, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    _check_mat(out, "out", M, N, (torch.bfloat16,), device)
    return out


def _raise(st, what):
    if st != 0:
        raise TkgError(st, what)


def gemm_bf16(A, Bt, out=None, stream=None):
    """out (M x N bf16) = A (M x K bf16) @ B, with B given as Bt (N x K)."""
    torch = _torch()
    M, K = A.shape
    N = Bt.shape[0]
    dt = (torch.bfloat16, torch.int16, torch.uint16)
    _check_mat(A, "A", M, K, dt, None)
    _check_mat(Bt, "Bt", N, K, dt, A.device)
    out = _out(out, M, N, A.device)
    with torch.cuda.device(A.device):
        st = lib.gemm_bf16(M, N, K, A.data_ptr(), Bt.data_ptr(),
                           out.data_ptr(), _stream_ptr(stream))
    _raise(st, "gemm_bf16")
    return out


def _fp8_types():
    torch = _torch()
    return tuple(t for t in (torch.uint8, getattr(torch, "float8_e4m3fn", None))
                 if t is not None)


def gemm_fp8(A, scale_a, Bt, scale_b, out=None, stream=None):
    """out = (scale_a * A) @ (scale_b * B); A: M x K e4m3, Bt: N x K e4m3
    (uint8 or float8_e4m3fn tensors), fp32 scales."""
    torch = _torch()
    M, K = A.shape
    N = Bt.shape[0]
    _check_mat(A, "A", M, K, _fp8_types(), None)
    _check_mat(Bt, "Bt", N, K, _fp8_types(), A.device)
    out = _out(out, M, N, A.device)
    with torch.cuda.device(A.device):
        st = lib.gemm_fp8(M, N, K, A.data_ptr(), float(scale_a),
                          Bt.data_ptr(), float(scale_b), out.data_ptr(),
                          _stream_ptr(stream))
    _raise(st, "gemm_fp8")
    return out


def gemm_splitk(A, Bt, scale_a=1.0, scale_b=1.0, splits=0, workspace=None,
                out=None, stream=None):
    """Split-K product (see tkg.h tkg_gemm_splitk): bf16 A, Bt (scales
    ignored) or e4m3 A, Bt with fp32 scales. `workspace` (a device tensor of
    at least splitk_workspace_size(...) bytes) is allocated here through
    torch when not given."""
    torch = _torch()
    M, K = A.shape
    N = Bt.shape[0]
    if A.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
        _check_mat(A, "A", M, K, (torch.bfloat16,), None)
        _check_mat(Bt, "Bt", N, K, (torch.bfloat16,), A.device)
    else:
        dtype = DTYPE_FP8
        _check_mat(A, "A", M, K, _fp8_types(), None)
        _check_mat(Bt, "Bt", N, K, _fp8_types(), A.device)
    out = _out(out, M, N, A.device)
    need = splitk_workspace_size(dtype, M, N, K, splits)
    own = workspace is None and need > 0
    if own:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(A.device):
        st = lib.tkg_gemm_splitk(dtype, M, N, K, A.data_ptr(), float(scale_a),
                                 Bt.data_ptr(), float(scale_b), out.data_ptr(),
                                 ws_ptr, ws_bytes, int(splits), _stream_ptr(stream))
    if own and stream is not None:
        # the kernels use the block on `stream`: keep the caching allocator
        # from handing it out again before that stream is past them
        workspace.record_stream(stream)
    _raise(st, "tkg_gemm_splitk")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # TKG_NOALLOC_SCRATCH_BYTES in tkg.h


def gemm_splitk_noalloc(A, Bt, out, scale_a=1.0, scale_b=1.0, splits=0, stream=None):
    """Split-K product without allocation (tkg_gemm_splitk_noalloc): the
    partial sums use the library's device scratch, and the caller passes
    the result tensor `out` (M x N bf16)."""
    torch = _torch()
    M, K = A.shape
    N = Bt.shape[0]
    if A.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
        _check_mat(A, "A", M, K, (torch.bfloat16,), None)
        _check_mat(Bt, "Bt", N, K, (torch.bfloat16,), A.device)
    else:
        dtype = DTYPE_FP8
        _check_mat(A, "A", M, K, _fp8_types(), None)
        _check_mat(Bt, "Bt", N, K, _fp8_types(), A.device)
    _check_mat(out, "out", M, N, (torch.bfloat16,), A.device)
    with torch.cuda.device(A.device):
        st = lib.tkg_gemm_splitk_noalloc(dtype, M, N, K, A.data_ptr(), float(scale_a),
                                         Bt.data_ptr(), float(scale_b), out.data_ptr(),
                                         int(splits), _stream_ptr(stream))
    _raise(st, "tkg_gemm_splitk_noalloc")
    return out


def splitk_workspace_size(dtype, M, N, K, splits=0) -> int:
    r = lib.tkg_gemm_splitk_workspace_size(int(dtype), int(M), int(N), int(K), int(splits))
    if r < 0:
        raise TkgError(r, "tkg_gemm_splitk_workspace_size")
    return r


def splitk_count(dtype, M, N, K, splits=0) -> int:
    r = lib.tkg_gemm_splitk_count(int(dtype), int(M), int(N), int(K), int(splits))
    if r < 0:
        raise TkgError(r, "tkg_gemm_splitk_count")
    return r


def gemm_fp4_blockscaled(A, A_scales, a_scale, Bt, B_scales, b_scale,
                         out=None, stream=None):
    """Block-scaled 4-bit product. A: M x K/2 packed e2m1 (uint8),
    A_scales: M x K/16 e4m3 (uint8), a_scale: fp32; Bt, B_scales, b_scale
    likewise for B in column-major order (N rows)."""
    torch = _torch()
    M, Kh = A.shape
    K = 2 * Kh
    N = Bt.shape[0]
    u8 = (torch.uint8,)
    _check_mat(A, "A", M, Kh, u8, None)
    _check_mat(Bt, "Bt", N, Kh, u8, A.device)
    _check_mat(A_scales, "A_scales", M, K // 16, _fp8_types(), A.device)
    _check_mat(B_scales, "B_scales", N, K // 16, _fp8_types(), A.device)
    out = _out(out, M, N, A.device)
    with torch.cuda.device(A.device):
        st = lib.gemm_fp4_blockscaled(
            M, N, K, A.data_ptr(), A_scales.data_ptr(), float(a_scale),
            Bt.data_ptr(), B_scales.data_ptr(), float(b_scale),
            out.data_ptr(), _stream_ptr(stream))
    _raise(st, "gemm_fp4_blockscaled")
    return out


def _gemm_mx(name, elem_per_byte, A, A_scales, Bt, B_scales, out, stream):
    torch = _torch()
    M, Kb = A.shape
    K = Kb * elem_per_byte
    N = Bt.shape[0]
    u8 = (torch.uint8,)
    vt = u8 if elem_per_byte == 2 else _fp8_types()
    _check_mat(A, "A", M, Kb, vt, None)
    _check_mat(Bt, "Bt", N, Kb, vt, A.device)
    _check_mat(A_scales, "A_scales", M, K // 32, u8, A.device)
    _check_mat(B_scales, "B_scales", N, K // 32, u8, A.device)
    out = _out(out, M, N, A.device)
    with torch.cuda.device(A.device):
        st = getattr(lib, name)(M, N, K, A.data_ptr(), A_scales.data_ptr(),
                                Bt.data_ptr(), B_scales.data_ptr(),
                                out.data_ptr(), _stream_ptr(stream))
    _raise(st, name)
    return out


def gemm_mxfp4(A, A_scales, Bt, B_scales, out=None, stream=None):
    """MXFP4 product. A: M x K/2 packed e2m1 (uint8), A_scales: M x K/32
    E8M0 (uint8); Bt, B_scales likewise for B in column-major order."""
    return _gemm_mx("gemm_mxfp4", 2, A, A_scales, Bt, B_scales, out, stream)


def gemm_mxfp8(A, A_scales, Bt, B_scales, out=None, stream=None):
    """MXFP8 product. A: M x K e4m3 (uint8 or float8_e4m3fn), A_scales:
    M x K/32 E8M0 (uint8); Bt, B_scales likewise for B (N rows)."""
    return _gemm_mx("gemm_mxfp8", 1, A, A_scales, Bt, B_scales, out, stream)


def tkg_gemm_ex(dtype, M, N, K, A, A_scales, a_scale, Bt, B_scales, b_scale,
                out, stream=None, grid=0, group_m=0, xcd_remap=1, variant=0):
    """Raw entry point with launch options (see tkg.h). Tensors or None for
    unused operands; returns the tkg status instead of raising."""
    torch = _torch()
    ptr = lambda t: None if t is None else t.data_ptr()
    o = TkgOpts(int(grid), int(group_m), int(xcd_remap), int(variant))
    with torch.cuda.device(out.device):
        return lib.tkg_gemm_ex(int(dtype), int(M), int(N), int(K), ptr(A),
                               ptr(A_scales), float(a_scale), ptr(Bt),
                               ptr(B_scales), float(b_scale), ptr(out),
                               _stream_ptr(stream), ctypes.byref(o))


def _check_4d(x, name, shape, device):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("%s has dtype %s, expected bfloat16" % (name, x.dtype))
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.device.type != "cuda" or (device is not None and x.device != device):
        raise ValueError("%s must be on the GPU (%s)" % (name, device))


def tkg_attention_fwd(Q, K, V, causal=False, scale=None, out=None, lse=None,
                      stream=None):
    """Softmax attention forward (``tkg_attention_fwd``): Q [B, Hq, Nq, D],
    K and V [B, Hkv, Nk, D] bf16 on the GPU; returns O [B, Hq, Nq, D] bf16.
    ``lse``: None (not stored), True (allocate and return (O, lse)) or an
    fp32 [B, Hq, Nq] tensor to fill (then (O, lse) is returned).
    ``scale`` defaults to 1/sqrt(D)."""
    import math
    torch = _torch()
    if Q.dim() != 4 or K.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, D]")
    B, Hq, Nq, D = Q.shape
    Hkv, Nk = K.shape[1], K.shape[2]
    _check_4d(Q, "Q", (B, Hq, Nq, D), None)
    _check_4d(K, "K", (B, Hkv, Nk, D), Q.device)
    _check_4d(V, "V", (B, Hkv, Nk, D), Q.device)
    if out is None:
        out = torch.empty((B, Hq, Nq, D), dtype=torch.bfloat16, device=Q.device)
    else:
        _check_4d(out, "out", (B, Hq, Nq, D), Q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=Q.device)
    if want_lse:
        if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq)
                or not lse.is_contiguous() or lse.device != Q.device):
            raise ValueError("lse must be a contiguous fp32 [B, Hq, Nq] GPU tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D) if D > 0 else 1.0
    with torch.cuda.device(Q.device):
        st = lib.tkg_attention_fwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                   out.data_ptr(), lse.data_ptr() if want_lse else None,
                                   B, Hq, Hkv, Nq, Nk, D, float(scale),
                                   1 if causal else 0, _stream_ptr(stream))
    _raise(st, "tkg_attention_fwd")
    return (out, lse) if want_lse else out
