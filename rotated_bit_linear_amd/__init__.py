"""Thin Python binding of libconvrot.so (the gfx950 rotated W8A8 NVFP4 linear layer).

Argument marshalling only: torch tensors provide device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing it is built, and if it cannot be loaded or the
device is not gfx950 the calls raise.

The C entry points are exposed under their own names (``cr_quant_act`` ...), taking
tensors in place of pointers; ``linear_nvfp4`` allocates the output and the workspace
and runs the whole layer.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

from . import build as _build

CR_ABI_VERSION = 3
CR_BF16, CR_FP16, CR_FP32, CR_I32 = 0, 1, 2, 3
CR_FLAG_NONE, CR_FLAG_FORCE_TWO_PASS, CR_FLAG_BLOCK_TRANSPOSED = 0, 1, 2
CR_MAX_K_PAD = 133120
NOALLOC_SCRATCH_BYTES = 64 << 20
DEFAULT_MAX_TILE_BYTES = 128 << 20
STATUS = {0: "CR_OK", 1: "CR_ERR_INVALID_ARG", 2: "CR_ERR_UNSUPPORTED_DTYPE", 3: "CR_ERR_MISALIGNED",
          4: "CR_ERR_TOO_LARGE", 5: "CR_ERR_NO_DEVICE", 6: "CR_ERR_LAUNCH"}

_TORCH_TO_CR = {torch.bfloat16: CR_BF16, torch.float16: CR_FP16, torch.float32: CR_FP32,
                torch.int32: CR_I32}
_CR_TO_TORCH = {v: k for k, v in _TORCH_TO_CR.items()}

LIB_PATH = _build.LIB
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "convrot.h")


class CrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """The loaded library (built in-tree first if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            _build.build()
        L = C.CDLL(LIB_PATH)
        i64, u32, vp, sz = C.c_int64, C.c_uint32, C.c_void_p, C.c_size_t
        sig = {
            "cr_abi_version": (C.c_int, []),
            "cr_status_string": (C.c_char_p, [C.c_int]),
            "cr_padded_k": (i64, [i64]),
            "cr_prep_weight_nvfp4": (C.c_int, [vp, i64, vp, i64, vp, i64, i64, vp, i64, vp, u32, vp]),
            "cr_quant_act": (C.c_int, [vp, C.c_int, i64, i64, i64, vp, i64, vp, u32, vp]),
            "cr_quant_act_swiglu": (C.c_int, [vp, C.c_int, i64, i64, i64, vp, i64, vp, u32, vp]),
            "cr_swiglu": (C.c_int, [vp, C.c_int, i64, i64, i64, vp, i64, vp]),
            "cr_gemm_s8_rowscale": (C.c_int, [vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, C.c_int, i64, vp]),
            "cr_gemm_s8_rowscale_bias": (C.c_int, [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, vp, C.c_int, i64,
                                                   vp]),
            "cr_quant_act_ex": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, vp, i64, vp, u32, vp]),
            "cr_linear_nvfp4_workspace_bytes": (sz, [i64, i64, i64, sz]),
            "cr_linear_nvfp4_plan": (C.c_int, [i64, i64, i64, sz, C.POINTER(i64), C.POINTER(i64)]),
            "cr_linear_nvfp4": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64, vp, i64,
                                          vp, C.c_int, i64, vp, sz, sz, u32, vp, vp]),
            "cr_linear_nvfp4_ex": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, vp, i64, vp, i64, vp,
                                             i64, vp, vp, C.c_int, i64, vp, sz, sz, u32, vp, vp]),
            "cr_linear_nvfp4_noalloc": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, vp, i64, vp, i64, vp,
                                                  i64, vp, vp, C.c_int, i64, sz, u32, vp]),
            "cr_weight_amax_nvfp4": (C.c_int, [vp, i64, vp, i64, vp, i64, i64, vp, u32, vp]),
            "cr_quant_weight_w4": (C.c_int, [vp, C.c_int, i64, i64, i64, vp, i64, vp, u32, vp]),
            "cr_gemm_s8s4_rowscale": (C.c_int, [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, vp, C.c_int, i64, vp]),
            "cr_linear_w4a8_workspace_bytes": (sz, [i64, i64]),
            "cr_linear_w4a8": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64, vp, vp, C.c_int,
                                         i64, vp, sz, u32, vp]),
            "cr_quant_act_w4": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, u32, vp]),
            "cr_gemm_s4s4_rowscale": (C.c_int, [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, vp, C.c_int, i64, vp]),
            "cr_linear_w4a4_workspace_bytes": (sz, [i64, i64]),
            "cr_linear_w4a4": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64, vp, vp, C.c_int,
                                         i64, vp, sz, u32, vp]),
            "cr_quant_weight_w4_e2m3": (C.c_int, [vp, C.c_int, i64, i64, i64, vp, i64, vp, u32, vp]),
            "cr_repack_w4_e2m3": (C.c_int, [vp, i64, i64, i64, vp, i64, vp]),
            "cr_quant_act_w4_e2m3": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, u32, vp]),
            "cr_gemm_e2m3_rowscale": (C.c_int, [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, vp, C.c_int, i64, vp]),
            "cr_linear_w4a4_e2m3_workspace_bytes": (sz, [i64, i64]),
            "cr_linear_w4a4_e2m3": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64, vp, vp,
                                              C.c_int, i64, vp, sz, u32, vp]),
            "cr_gemm_nvfp4_fused": (C.c_int, [vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, i64, i64, i64, vp,
                                              C.c_int, i64, u32, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        v = L.cr_abi_version()
        if v != CR_ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH}: ABI version {v}, binding expects {CR_ABI_VERSION}")
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/convrot.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cr_\w+)\s*\(", src)))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise CrError(fn, status)


def _rows_ld(t: torch.Tensor):
    assert t.dim() == 2 and t.stride(1) == 1, "expected a row-major 2-D tensor (unit column stride)"
    return t.shape[0], t.stride(0)


def padded_k(k: int) -> int:
    return int(lib().cr_padded_k(k))


# ------------------------------------------------------------------- entry points ----

def cr_prep_weight_nvfp4(w_fp4, w_sf, global_scale, K, w_s8, w_scale, flags=0, stream=None):
    n, ld_fp4 = _rows_ld(w_fp4)
    _, ld_sf = _rows_ld(w_sf)
    _, ld_s8 = _rows_ld(w_s8)
    _check("cr_prep_weight_nvfp4", lib().cr_prep_weight_nvfp4(
        _ptr(w_fp4), ld_fp4, _ptr(w_sf), ld_sf, _ptr(global_scale), n, K, _ptr(w_s8), ld_s8,
        _ptr(w_scale), flags, _stream(stream)))


def cr_quant_act(x, K, x_s8, x_scale, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    _, ld_s8 = _rows_ld(x_s8)
    _check("cr_quant_act", lib().cr_quant_act(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, M, K, _ptr(x_s8), ld_s8, _ptr(x_scale), flags,
        _stream(stream)))


def cr_quant_act_swiglu(h, F, x_s8, x_scale, flags=0, stream=None):
    M, ld_h = _rows_ld(h)
    _, ld_s8 = _rows_ld(x_s8)
    _check("cr_quant_act_swiglu", lib().cr_quant_act_swiglu(
        _ptr(h), _TORCH_TO_CR[h.dtype], ld_h, M, F, _ptr(x_s8), ld_s8, _ptr(x_scale), flags,
        _stream(stream)))


def cr_quant_act_ex(x, K, swiglu, pre_scale, x_s8, x_scale, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    _, ld_s8 = _rows_ld(x_s8)
    _check("cr_quant_act_ex", lib().cr_quant_act_ex(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(pre_scale), _ptr(x_s8), ld_s8,
        _ptr(x_scale), flags, _stream(stream)))


def cr_swiglu(h, F, out, stream=None):
    M, ld_h = _rows_ld(h)
    _, ld_out = _rows_ld(out)
    _check("cr_swiglu", lib().cr_swiglu(_ptr(h), _TORCH_TO_CR[h.dtype], ld_h, M, F, _ptr(out), ld_out,
                                        _stream(stream)))


def cr_gemm_s8_rowscale(a_s8, a_scale, b_s8, b_scale, c, stream=None, M=None, N=None):
    Ma, lda = _rows_ld(a_s8)
    Nb, ldb = _rows_ld(b_s8)
    _, ldc = _rows_ld(c)
    M = Ma if M is None else M
    N = Nb if N is None else N
    K_pad = a_s8.shape[1]
    _check("cr_gemm_s8_rowscale", lib().cr_gemm_s8_rowscale(
        _ptr(a_s8), lda, _ptr(a_scale), _ptr(b_s8), ldb, _ptr(b_scale), M, N, K_pad, _ptr(c),
        _TORCH_TO_CR[c.dtype], ldc, _stream(stream)))


def cr_linear_nvfp4_workspace_bytes(M, N, K, max_tile_bytes=0) -> int:
    return int(lib().cr_linear_nvfp4_workspace_bytes(M, N, K, max_tile_bytes))


def cr_gemm_s8_rowscale_bias(a_s8, a_scale, b_s8, b_scale, bias, c, stream=None):
    M, lda = _rows_ld(a_s8)
    N, ldb = _rows_ld(b_s8)
    _, ldc = _rows_ld(c)
    _check("cr_gemm_s8_rowscale_bias", lib().cr_gemm_s8_rowscale_bias(
        _ptr(a_s8), lda, _ptr(a_scale), _ptr(b_s8), ldb, _ptr(b_scale), _ptr(bias), M, N, a_s8.shape[1],
        _ptr(c), _TORCH_TO_CR[c.dtype], ldc, _stream(stream)))


def cr_linear_nvfp4_plan(M, N, K, max_tile_bytes=0) -> tuple[int, int]:
    """(rows per weight chunk, number of chunks) that cr_linear_nvfp4 uses on this device."""
    r, n = C.c_int64(0), C.c_int64(0)
    _check("cr_linear_nvfp4_plan", lib().cr_linear_nvfp4_plan(M, N, K, max_tile_bytes,
                                                              C.byref(r), C.byref(n)))
    return int(r.value), int(n.value)


def cr_linear_nvfp4(x, K, swiglu, w_fp4, w_sf, global_scale, out, workspace, max_tile_bytes=0,
                    flags=0, stream=None, aux_stream=None, pre_scale=None, bias=None):
    """cr_linear_nvfp4, or cr_linear_nvfp4_ex when a pre-scale or a bias is given."""
    M, ld_x = _rows_ld(x)
    N, ld_fp4 = _rows_ld(w_fp4)
    _, ld_sf = _rows_ld(w_sf)
    _, ldc = _rows_ld(out)
    aux = None if aux_stream is None else _stream(aux_stream)
    ws = (_ptr(workspace), workspace.numel() * workspace.element_size(), max_tile_bytes, flags,
          _stream(stream), aux)
    if pre_scale is None and bias is None:
        _check("cr_linear_nvfp4", lib().cr_linear_nvfp4(
            _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(w_fp4), ld_fp4,
            _ptr(w_sf), ld_sf, _ptr(global_scale), N, _ptr(out), _TORCH_TO_CR[out.dtype], ldc, *ws))
    else:
        _check("cr_linear_nvfp4_ex", lib().cr_linear_nvfp4_ex(
            _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(pre_scale), _ptr(w_fp4), ld_fp4,
            _ptr(w_sf), ld_sf, _ptr(global_scale), N, _ptr(bias), _ptr(out), _TORCH_TO_CR[out.dtype], ldc, *ws))


def cr_linear_nvfp4_noalloc(x, K, swiglu, w_fp4, w_sf, global_scale, out, max_tile_bytes=0, flags=0,
                            stream=None, pre_scale=None, bias=None):
    """The layer with the library's own device scratch as its workspace (nothing allocated)."""
    M, ld_x = _rows_ld(x)
    N, ld_fp4 = _rows_ld(w_fp4)
    _, ld_sf = _rows_ld(w_sf)
    _, ldc = _rows_ld(out)
    _check("cr_linear_nvfp4_noalloc", lib().cr_linear_nvfp4_noalloc(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(pre_scale), _ptr(w_fp4), ld_fp4,
        _ptr(w_sf), ld_sf, _ptr(global_scale), N, _ptr(bias), _ptr(out), _TORCH_TO_CR[out.dtype], ldc,
        max_tile_bytes, flags, _stream(stream)))


def cr_weight_amax_nvfp4(w_fp4, w_sf, global_scale, K, w_amax, flags=0, stream=None):
    n, ld_fp4 = _rows_ld(w_fp4)
    _, ld_sf = _rows_ld(w_sf)
    _check("cr_weight_amax_nvfp4", lib().cr_weight_amax_nvfp4(
        _ptr(w_fp4), ld_fp4, _ptr(w_sf), ld_sf, _ptr(global_scale), n, K, _ptr(w_amax), flags, _stream(stream)))


def cr_gemm_nvfp4_fused(a_s8, a_scale, w_fp4, w_sf, global_scale, w_amax, K, c, bias=None, flags=0,
                        stream=None):
    M, lda = _rows_ld(a_s8)
    N, ld_fp4 = _rows_ld(w_fp4)
    _, ld_sf = _rows_ld(w_sf)
    _, ldc = _rows_ld(c)
    _check("cr_gemm_nvfp4_fused", lib().cr_gemm_nvfp4_fused(
        _ptr(a_s8), lda, _ptr(a_scale), _ptr(w_fp4), ld_fp4, _ptr(w_sf), ld_sf, _ptr(global_scale),
        _ptr(w_amax), _ptr(bias), M, N, K, _ptr(c), _TORCH_TO_CR[c.dtype], ldc, flags, _stream(stream)))


def cr_quant_weight_w4(w, K, w_s4, w_scale, flags=0, stream=None):
    N, ld_w = _rows_ld(w)
    _, ld_s4 = _rows_ld(w_s4)
    _check("cr_quant_weight_w4", lib().cr_quant_weight_w4(
        _ptr(w), _TORCH_TO_CR[w.dtype], ld_w, N, K, _ptr(w_s4), ld_s4, _ptr(w_scale), flags, _stream(stream)))


def cr_gemm_s8s4_rowscale(a_s8, a_scale, b_s4, b_scale, c, bias=None, stream=None):
    M, lda = _rows_ld(a_s8)
    N, ldb = _rows_ld(b_s4)
    _, ldc = _rows_ld(c)
    _check("cr_gemm_s8s4_rowscale", lib().cr_gemm_s8s4_rowscale(
        _ptr(a_s8), lda, _ptr(a_scale), _ptr(b_s4), ldb, _ptr(b_scale), _ptr(bias), M, N, a_s8.shape[1],
        _ptr(c), _TORCH_TO_CR[c.dtype], ldc, _stream(stream)))


def cr_linear_w4a8_workspace_bytes(M, K) -> int:
    return int(lib().cr_linear_w4a8_workspace_bytes(M, K))


def cr_linear_w4a8(x, K, swiglu, w_s4, w_scale, out, workspace, bias=None, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    N, ld_s4 = _rows_ld(w_s4)
    _, ldc = _rows_ld(out)
    _check("cr_linear_w4a8", lib().cr_linear_w4a8(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(w_s4), ld_s4, _ptr(w_scale), N,
        _ptr(bias), _ptr(out), _TORCH_TO_CR[out.dtype], ldc, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), flags, _stream(stream)))


def cr_quant_act_w4(x, K, swiglu, x_s4, x_scale, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    _, ld_s4 = _rows_ld(x_s4)
    _check("cr_quant_act_w4", lib().cr_quant_act_w4(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(x_s4), ld_s4, _ptr(x_scale), flags,
        _stream(stream)))


def cr_gemm_s4s4_rowscale(a_s4, a_scale, b_s4, b_scale, c, bias=None, K_pad=None, stream=None):
    M, lda = _rows_ld(a_s4)
    N, ldb = _rows_ld(b_s4)
    _, ldc = _rows_ld(c)
    kp = 2 * a_s4.shape[1] if K_pad is None else K_pad
    _check("cr_gemm_s4s4_rowscale", lib().cr_gemm_s4s4_rowscale(
        _ptr(a_s4), lda, _ptr(a_scale), _ptr(b_s4), ldb, _ptr(b_scale), _ptr(bias), M, N, kp,
        _ptr(c), _TORCH_TO_CR[c.dtype], ldc, _stream(stream)))


def cr_linear_w4a4_workspace_bytes(M, K) -> int:
    return int(lib().cr_linear_w4a4_workspace_bytes(M, K))


def cr_linear_w4a4(x, K, swiglu, w_s4, w_scale, out, workspace, bias=None, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    N, ld_s4 = _rows_ld(w_s4)
    _, ldc = _rows_ld(out)
    _check("cr_linear_w4a4", lib().cr_linear_w4a4(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(w_s4), ld_s4, _ptr(w_scale), N,
        _ptr(bias), _ptr(out), _TORCH_TO_CR[out.dtype], ldc, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), flags, _stream(stream)))


def cr_quant_weight_w4_e2m3(w, K, w_f6, w_scale, flags=0, stream=None):
    N, ld_w = _rows_ld(w)
    _, ld_f6 = _rows_ld(w_f6)
    _check("cr_quant_weight_w4_e2m3", lib().cr_quant_weight_w4_e2m3(
        _ptr(w), _TORCH_TO_CR[w.dtype], ld_w, N, K, _ptr(w_f6), ld_f6, _ptr(w_scale), flags, _stream(stream)))


def cr_repack_w4_e2m3(w_s4, w_f6, K_pad=None, stream=None):
    N, ld_s4 = _rows_ld(w_s4)
    _, ld_f6 = _rows_ld(w_f6)
    kp = 2 * w_s4.shape[1] if K_pad is None else K_pad
    _check("cr_repack_w4_e2m3", lib().cr_repack_w4_e2m3(_ptr(w_s4), ld_s4, N, kp, _ptr(w_f6), ld_f6,
                                                          _stream(stream)))


def cr_quant_act_w4_e2m3(x, K, swiglu, x_f6, x_scale, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    _, ld_f6 = _rows_ld(x_f6)
    _check("cr_quant_act_w4_e2m3", lib().cr_quant_act_w4_e2m3(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(x_f6), ld_f6, _ptr(x_scale), flags,
        _stream(stream)))


def cr_gemm_e2m3_rowscale(a_f6, a_scale, b_f6, b_scale, c, bias=None, K_pad=None, stream=None):
    """E2M3-field operands are [quads, >= 3 K_pad] uint8 (four code rows per tensor row); M and N
    are the output's extents."""
    _, lda = _rows_ld(a_f6)
    _, ldb = _rows_ld(b_f6)
    M, ldc = _rows_ld(c)
    N = c.shape[1]
    kp = a_f6.shape[1] // 3 if K_pad is None else K_pad
    _check("cr_gemm_e2m3_rowscale", lib().cr_gemm_e2m3_rowscale(
        _ptr(a_f6), lda, _ptr(a_scale), _ptr(b_f6), ldb, _ptr(b_scale), _ptr(bias), M, N, kp,
        _ptr(c), _TORCH_TO_CR[c.dtype], ldc, _stream(stream)))


def cr_linear_w4a4_e2m3_workspace_bytes(M, K) -> int:
    return int(lib().cr_linear_w4a4_e2m3_workspace_bytes(M, K))


def cr_linear_w4a4_e2m3(x, K, swiglu, w_f6, w_scale, out, workspace, bias=None, flags=0, stream=None):
    M, ld_x = _rows_ld(x)
    _, ld_f6 = _rows_ld(w_f6)
    _, ldc = _rows_ld(out)
    N = out.shape[1]
    _check("cr_linear_w4a4_e2m3", lib().cr_linear_w4a4_e2m3(
        _ptr(x), _TORCH_TO_CR[x.dtype], ld_x, int(bool(swiglu)), M, K, _ptr(w_f6), ld_f6, _ptr(w_scale), N,
        _ptr(bias), _ptr(out), _TORCH_TO_CR[out.dtype], ldc, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), flags, _stream(stream)))


# ---------------------------------------------------------------- conveniences ----

def quant_act(x: torch.Tensor, K: int | None = None, swiglu: bool = False, flags: int = 0,
              pre_scale: torch.Tensor | None = None):
    """(x_s8 [M, K_pad] int8, x_scale [M] fp32) of X [M, K] or of SwiGLU(H [M, 2K]), with an
    optional [K] channel pre-scale."""
    if K is None:
        K = x.shape[1] // 2 if swiglu else x.shape[1]
    kp = padded_k(K)
    q = torch.empty(x.shape[0], kp, dtype=torch.int8, device=x.device)
    s = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    if pre_scale is not None:
        cr_quant_act_ex(x, K, swiglu, pre_scale, q, s, flags)
    else:
        (cr_quant_act_swiglu if swiglu else cr_quant_act)(x, K, q, s, flags)
    return q, s


def prep_weight_nvfp4(w_fp4: torch.Tensor, w_sf: torch.Tensor, global_scale: torch.Tensor, K: int,
                      flags: int = 0):
    kp = padded_k(K)
    q = torch.empty(w_fp4.shape[0], kp, dtype=torch.int8, device=w_fp4.device)
    s = torch.empty(w_fp4.shape[0], dtype=torch.float32, device=w_fp4.device)
    cr_prep_weight_nvfp4(w_fp4, w_sf, global_scale, K, q, s, flags)
    return q, s


def gemm_s8_rowscale(a_s8, a_scale, b_s8, b_scale, out_dtype=torch.bfloat16, bias=None):
    c = torch.empty(a_s8.shape[0], b_s8.shape[0], dtype=out_dtype, device=a_s8.device)
    if bias is not None:
        cr_gemm_s8_rowscale_bias(a_s8, a_scale, b_s8, b_scale, bias, c)
    else:
        cr_gemm_s8_rowscale(a_s8, a_scale, b_s8, b_scale, c)
    return c


def linear_nvfp4(x, w_fp4, w_sf, global_scale, K, out_dtype=torch.bfloat16, swiglu=False, out=None,
                 max_tile_bytes=0, flags=0, aux_stream=None, workspace=None, pre_scale=None, bias=None):
    """y = x W^T (+ b) through the rotated S8 route (SwiGLU(x) W^T when swiglu); pre_scale
    multiplies the input channels before the rotation."""
    M, N = x.shape[0], w_fp4.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    need = cr_linear_nvfp4_workspace_bytes(M, N, K, max_tile_bytes)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    cr_linear_nvfp4(x, K, swiglu, w_fp4, w_sf, global_scale, out, workspace, max_tile_bytes, flags,
                    aux_stream=aux_stream, pre_scale=pre_scale, bias=bias)
    return out


def weight_amax_nvfp4(w_fp4: torch.Tensor, w_sf: torch.Tensor, global_scale: torch.Tensor, K: int,
                      flags: int = 0) -> torch.Tensor:
    """[N] fp32 row maxima of the rotated weight (input of gemm_nvfp4_fused)."""
    a = torch.empty(w_fp4.shape[0], dtype=torch.float32, device=w_fp4.device)
    cr_weight_amax_nvfp4(w_fp4, w_sf, global_scale, K, a, flags)
    return a


def gemm_nvfp4_fused(a_s8, a_scale, w_fp4, w_sf, global_scale, w_amax, K, out_dtype=torch.bfloat16,
                     bias=None, flags=0):
    c = torch.empty(a_s8.shape[0], w_fp4.shape[0], dtype=out_dtype, device=a_s8.device)
    cr_gemm_nvfp4_fused(a_s8, a_scale, w_fp4, w_sf, global_scale, w_amax, K, c, bias, flags)
    return c


def quant_weight_w4(w: torch.Tensor, K: int | None = None, flags: int = 0):
    """(packed 4-bit codes [N, K_pad / 2] uint8, scales [N] fp32) of a dense weight [N, K]."""
    if K is None:
        K = w.shape[1]
    kp = padded_k(K)
    q = torch.empty(w.shape[0], kp // 2, dtype=torch.uint8, device=w.device)
    s = torch.empty(w.shape[0], dtype=torch.float32, device=w.device)
    cr_quant_weight_w4(w, K, q, s, flags)
    return q, s


def linear_w4a8(x, w_s4, w_scale, K, out_dtype=torch.bfloat16, swiglu=False, bias=None, flags=0, out=None):
    """y = x W^T (+ b) through the W4A8 route against a prepared 4-bit weight."""
    M, N = x.shape[0], w_s4.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    ws = torch.empty(max(1, cr_linear_w4a8_workspace_bytes(M, K)), dtype=torch.uint8, device=x.device)
    cr_linear_w4a8(x, K, swiglu, w_s4, w_scale, out, ws, bias=bias, flags=flags)
    return out


def quant_act_w4(x: torch.Tensor, K: int | None = None, swiglu: bool = False, flags: int = 0):
    """(packed 4-bit codes [M, K_pad / 2] uint8, scales [M] fp32) of X [M, K] or of
    SwiGLU(H [M, 2K])."""
    if K is None:
        K = x.shape[1] // 2 if swiglu else x.shape[1]
    kp = padded_k(K)
    q = torch.empty(x.shape[0], kp // 2, dtype=torch.uint8, device=x.device)
    s = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    cr_quant_act_w4(x, K, swiglu, q, s, flags)
    return q, s


def linear_w4a4(x, w_s4, w_scale, K, out_dtype=torch.bfloat16, swiglu=False, bias=None, flags=0, out=None):
    """y = x W^T (+ b) through the W4A4 route against a prepared 4-bit weight."""
    M, N = x.shape[0], w_s4.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    ws = torch.empty(max(1, cr_linear_w4a4_workspace_bytes(M, K)), dtype=torch.uint8, device=x.device)
    cr_linear_w4a4(x, K, swiglu, w_s4, w_scale, out, ws, bias=bias, flags=flags)
    return out


def quant_weight_w4_e2m3(w: torch.Tensor, K: int | None = None, flags: int = 0):
    """(4-bit codes as E2M3 fields in quads of rows [ceil(N / 4), 3 K_pad] uint8, scales [N]
    fp32) of a dense weight; unused rows of the last quad are zero."""
    if K is None:
        K = w.shape[1]
    kp = padded_k(K)
    q = torch.zeros((w.shape[0] + 3) // 4, 3 * kp, dtype=torch.uint8, device=w.device)
    s = torch.empty(w.shape[0], dtype=torch.float32, device=w.device)
    cr_quant_weight_w4_e2m3(w, K, q, s, flags)
    return q, s


def quant_act_w4_e2m3(x: torch.Tensor, K: int | None = None, swiglu: bool = False, flags: int = 0):
    """(4-bit codes as E2M3 fields in quads of rows [ceil(M / 4), 3 K_pad] uint8, scales [M]
    fp32) of X or SwiGLU(H); unused rows of the last quad are zero."""
    if K is None:
        K = x.shape[1] // 2 if swiglu else x.shape[1]
    kp = padded_k(K)
    q = torch.zeros((x.shape[0] + 3) // 4, 3 * kp, dtype=torch.uint8, device=x.device)
    s = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    cr_quant_act_w4_e2m3(x, K, swiglu, q, s, flags)
    return q, s


def linear_w4a4_e2m3(x, w_f6, w_scale, K, out_dtype=torch.bfloat16, swiglu=False, bias=None, flags=0, out=None):
    """y = x W^T (+ b) through the W4A4 route on the 6-bit matrix cores."""
    M, N = x.shape[0], w_scale.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    ws = torch.empty(max(1, cr_linear_w4a4_e2m3_workspace_bytes(M, K)), dtype=torch.uint8, device=x.device)
    cr_linear_w4a4_e2m3(x, K, swiglu, w_f6, w_scale, out, ws, bias=bias, flags=flags)
    return out


def repack_w4_e2m3(w_s4: torch.Tensor, K_pad: int | None = None):
    """The E2M3 form [ceil(N / 4), 3 K_pad] uint8 of nibble-form 4-bit rows [N, K_pad / 2] (the
    row scales are unchanged); unused rows of the last quad are zero."""
    kp = 2 * w_s4.shape[1] if K_pad is None else K_pad
    out = torch.zeros((w_s4.shape[0] + 3) // 4, 3 * kp, dtype=torch.uint8, device=w_s4.device)
    cr_repack_w4_e2m3(w_s4, out, K_pad=kp)
    return out
