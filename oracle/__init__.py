"""Python access to the plain CPU oracle (oracle/oracle.c) through ctypes.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the GPU library or its binding.  Every function takes and
returns host numpy arrays; bf16/fp16 data travels as uint16 bit patterns.

Each function follows one step of the method, in the pages' order (see oracle.c for the
citations and the readings taken where the pages are silent).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

DT_BF16, DT_FP16, DT_FP32, DT_I32 = 0, 1, 2, 3

_lib = None


def lib():
    """The loaded oracle library (built with gcc on first use if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        i64, f32, u8, vp = C.c_int64, C.c_float, C.c_uint8, C.c_void_p
        sig = {
            "or_num_threads": (C.c_int, []),
            "or_padded_k": (i64, [i64]),
            "or_e2m1": (f32, [u8]),
            "or_e4m3": (f32, [u8]),
            "or_exp": (f32, [f32]),
            "or_sigmoid": (f32, [f32]),
            "or_swiglu": (f32, [f32, f32]),
            "or_nvfp4_decode": (None, [vp, i64, vp, i64, f32, i64, i64, vp, i64]),
            "or_fwht256": (None, [vp]),
            "or_convrot256": (None, [vp, i64, i64, i64]),
            "or_row_quant": (None, [vp, i64, i64, i64, vp, i64, vp]),
            "or_act_load": (None, [vp, C.c_int, i64, i64, i64, vp, i64]),
            "or_act_load_swiglu": (None, [vp, C.c_int, i64, i64, i64, vp, i64]),
            "or_quant_act": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp]),
            "or_quant_act_ex": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, vp, i64, vp]),
            "or_act_prescale": (None, [vp, i64, i64, i64, vp]),
            "or_prep_weight_nvfp4": (C.c_int, [vp, i64, vp, i64, f32, i64, i64, vp, i64, vp]),
            "or_weight_amax_nvfp4": (C.c_int, [vp, i64, vp, i64, f32, i64, i64, vp]),
            "or_gemm_s8": (None, [vp, i64, vp, i64, i64, i64, i64, vp, i64]),
            "or_epilogue": (None, [vp, i64, vp, vp, i64, i64, C.c_int, vp, i64]),
            "or_epilogue_ex": (None, [vp, i64, vp, vp, vp, i64, i64, C.c_int, vp, i64]),
            "or_linear_nvfp4": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64,
                                          f32, i64, vp, C.c_int, i64]),
            "or_linear_nvfp4_ex": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, vp, i64, vp, i64,
                                             f32, i64, vp, vp, C.c_int, i64]),
            "or_row_quant_s4": (None, [vp, i64, i64, i64, vp, i64, vp]),
            "or_pack_s4": (None, [vp, i64, i64, i64, vp, i64]),
            "or_unpack_s4": (None, [vp, i64, i64, i64, vp, i64]),
            "or_quant_weight_w4": (C.c_int, [vp, C.c_int, i64, i64, i64, vp, i64, vp]),
            "or_gemm_s8s4": (C.c_int, [vp, i64, vp, i64, i64, i64, i64, vp, i64]),
            "or_linear_w4a8": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64, vp, vp,
                                         C.c_int, i64]),
            "or_e2m3": (C.c_float, [C.c_uint8]),
            "or_pack_e2m3": (C.c_int, [vp, i64, i64, i64, vp, i64]),
            "or_unpack_e2m3": (C.c_int, [vp, i64, i64, i64, vp, i64]),
            "or_gemm_e2m3": (C.c_int, [vp, i64, vp, i64, i64, i64, i64, vp, i64]),
            "or_quant_act_w4": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp]),
            "or_gemm_s4s4": (C.c_int, [vp, i64, vp, i64, i64, i64, i64, vp, i64]),
            "or_linear_w4a4": (C.c_int, [vp, C.c_int, i64, C.c_int, i64, i64, vp, i64, vp, i64, vp, vp,
                                         C.c_int, i64]),
            "or_exp_array": (None, [vp, vp, i64]),
            "or_sigmoid_array": (None, [vp, vp, i64]),
            "or_swiglu_array": (None, [vp, vp, vp, i64]),
            "or_bf16_to_f32_array": (None, [vp, vp, i64]),
            "or_fp16_to_f32_array": (None, [vp, vp, i64]),
            "or_f32_to_bf16_array": (None, [vp, vp, i64]),
            "or_f32_to_fp16_array": (None, [vp, vp, i64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _elem_dtype(dtype: int):
    return {DT_BF16: np.uint16, DT_FP16: np.uint16, DT_FP32: np.float32}[dtype]


def padded_k(k: int) -> int:
    return int(lib().or_padded_k(k))


def num_threads() -> int:
    return int(lib().or_num_threads())


# ------------------------------------------------------------------ formats ----

def e2m1(code: int) -> float:
    return float(lib().or_e2m1(code))


def e4m3(byte: int) -> float:
    return float(lib().or_e4m3(byte))


def _map(fn_name, x, out_dtype):
    x = np.ascontiguousarray(x)
    y = np.empty(x.shape, dtype=out_dtype)
    getattr(lib(), fn_name)(_p(x), _p(y), x.size)
    return y


def bf16_to_f32(h): return _map("or_bf16_to_f32_array", np.asarray(h, np.uint16), np.float32)
def fp16_to_f32(h): return _map("or_fp16_to_f32_array", np.asarray(h, np.uint16), np.float32)
def f32_to_bf16(x): return _map("or_f32_to_bf16_array", np.asarray(x, np.float32), np.uint16)
def f32_to_fp16(x): return _map("or_f32_to_fp16_array", np.asarray(x, np.float32), np.uint16)
def exp(x): return _map("or_exp_array", np.asarray(x, np.float32), np.float32)
def sigmoid(x): return _map("or_sigmoid_array", np.asarray(x, np.float32), np.float32)


def swiglu(gate, value):
    gate = np.ascontiguousarray(gate, np.float32)
    value = np.ascontiguousarray(value, np.float32)
    assert gate.shape == value.shape
    y = np.empty(gate.shape, np.float32)
    lib().or_swiglu_array(_p(gate), _p(value), _p(y), gate.size)
    return y


# -------------------------------------------------------------------- steps ----

def nvfp4_decode(codes: np.ndarray, sf: np.ndarray, g: float, K: int) -> np.ndarray:
    """[N, ld_codes] u8 codes, [N, ld_sf] u8 E4M3 scales -> fp32 [N, K_pad]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    sf = np.ascontiguousarray(sf, np.uint8)
    n = codes.shape[0]
    kp = padded_k(K)
    w = np.empty((n, kp), np.float32)
    lib().or_nvfp4_decode(_p(codes), codes.shape[1], _p(sf), sf.shape[1], g, n, K, _p(w), kp)
    return w


def fwht256(y: np.ndarray) -> np.ndarray:
    y = np.array(y, np.float32, copy=True).reshape(256)
    lib().or_fwht256(_p(y))
    return y


def convrot256(y: np.ndarray) -> np.ndarray:
    """ConvRot256 of every row (a copy); rows must be a multiple of 256 long."""
    y = np.array(y, np.float32, copy=True, order="C")
    n, kp = y.shape
    assert kp % 256 == 0
    lib().or_convrot256(_p(y), n, kp, kp)
    return y


def row_quant(y: np.ndarray):
    y = np.ascontiguousarray(y, np.float32)
    n, kp = y.shape
    q = np.empty((n, kp), np.int8)
    s = np.empty(n, np.float32)
    lib().or_row_quant(_p(y), n, kp, kp, _p(q), kp, _p(s))
    return q, s


def act_load(x: np.ndarray, dtype: int, K: int, swiglu: bool = False) -> np.ndarray:
    """X[M, >=K] (or H[M, >=2F]) -> fp32 [M, K_pad] (SwiGLU applied when asked)."""
    x = np.ascontiguousarray(x, _elem_dtype(dtype))
    M = x.shape[0]
    kp = padded_k(K)
    out = np.empty((M, kp), np.float32)
    fn = lib().or_act_load_swiglu if swiglu else lib().or_act_load
    fn(_p(x), dtype, x.shape[1], M, K, _p(out), kp)
    return out


def _opt_f32(a, n: int):
    """(array or None, pointer or None) for an optional float32 vector of length n."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, np.float32)
    assert a.shape == (n,)
    return a, _p(a)


def act_prescale(buf: np.ndarray, K: int, c: np.ndarray) -> np.ndarray:
    """The channel pre-scale step on loaded rows [M, K_pad] (a copy)."""
    out = np.array(buf, np.float32, order="C")
    c, cp = _opt_f32(c, K)
    lib().or_act_prescale(_p(out), out.shape[0], K, out.shape[1], cp)
    return out


def quant_act(x: np.ndarray, dtype: int, K: int, swiglu: bool = False, pre_scale=None):
    """Activation preparation -> (x_s8 [M, K_pad] int8, x_scale [M] fp32); pre_scale is an
    optional [K] float32 channel pre-scale applied before the rotation."""
    x = np.ascontiguousarray(x, _elem_dtype(dtype))
    M = x.shape[0]
    kp = padded_k(K)
    q = np.empty((M, kp), np.int8)
    s = np.empty(M, np.float32)
    c, cp = _opt_f32(pre_scale, K)
    rc = lib().or_quant_act_ex(_p(x), dtype, x.shape[1], int(swiglu), M, K, cp, _p(q), kp, _p(s))
    assert rc == 0
    return q, s


def prep_weight_nvfp4(codes: np.ndarray, sf: np.ndarray, g: float, K: int):
    """Weight preparation -> (w_s8 [N, K_pad] int8, w_scale [N] fp32)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    sf = np.ascontiguousarray(sf, np.uint8)
    n = codes.shape[0]
    kp = padded_k(K)
    q = np.empty((n, kp), np.int8)
    s = np.empty(n, np.float32)
    rc = lib().or_prep_weight_nvfp4(_p(codes), codes.shape[1], _p(sf), sf.shape[1], g, n, K,
                                    _p(q), kp, _p(s))
    assert rc == 0
    return q, s


def weight_amax_nvfp4(codes: np.ndarray, sf: np.ndarray, g: float, K: int) -> np.ndarray:
    """Row maxima a[n] = max |ConvRot256(decode(W))[n, :]| -> [N] fp32."""
    codes = np.ascontiguousarray(codes, np.uint8)
    sf = np.ascontiguousarray(sf, np.uint8)
    n = codes.shape[0]
    a = np.empty(n, np.float32)
    rc = lib().or_weight_amax_nvfp4(_p(codes), codes.shape[1], _p(sf), sf.shape[1], g, n, K, _p(a))
    assert rc == 0
    return a

def gemm_s8(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """int32 acc[M, N] = A[M, K_pad] . B[N, K_pad]^T."""
    a = np.ascontiguousarray(a, np.int8)
    b = np.ascontiguousarray(b, np.int8)
    M, kp = a.shape
    N = b.shape[0]
    assert b.shape[1] == kp
    acc = np.empty((M, N), np.int32)
    lib().or_gemm_s8(_p(a), kp, _p(b), kp, M, N, kp, _p(acc), N)
    return acc


def epilogue(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray, out_dtype: int, bias=None) -> np.ndarray:
    """Row-scale dequantization (+ optional [N] float32 bias); bf16/fp16 come back as uint16
    bit patterns."""
    acc = np.ascontiguousarray(acc, np.int32)
    s_x = np.ascontiguousarray(s_x, np.float32)
    s_w = np.ascontiguousarray(s_w, np.float32)
    M, N = acc.shape
    b, bp = _opt_f32(bias, N)
    odt = {DT_BF16: np.uint16, DT_FP16: np.uint16, DT_FP32: np.float32, DT_I32: np.int32}[out_dtype]
    out = np.empty((M, N), odt)
    lib().or_epilogue_ex(_p(acc), N, _p(s_x), _p(s_w), bp, M, N, out_dtype, _p(out), N)
    return out


def linear_nvfp4(x: np.ndarray, x_dtype: int, K: int, swiglu: bool, codes: np.ndarray,
                 sf: np.ndarray, g: float, out_dtype: int, pre_scale=None, bias=None) -> np.ndarray:
    """The whole layer on the rows of x (optional channel pre-scale [K] and bias [N])."""
    x = np.ascontiguousarray(x, _elem_dtype(x_dtype))
    codes = np.ascontiguousarray(codes, np.uint8)
    sf = np.ascontiguousarray(sf, np.uint8)
    M = x.shape[0]
    N = codes.shape[0]
    odt = {DT_BF16: np.uint16, DT_FP16: np.uint16, DT_FP32: np.float32, DT_I32: np.int32}[out_dtype]
    out = np.empty((M, N), odt)
    c, cp = _opt_f32(pre_scale, K)
    b, bp = _opt_f32(bias, N)
    rc = lib().or_linear_nvfp4_ex(_p(x), x_dtype, x.shape[1], int(swiglu), M, K, cp, _p(codes),
                                  codes.shape[1], _p(sf), sf.shape[1], g, N, bp, _p(out), out_dtype, N)
    assert rc == 0
    return out


# ------------------------------------------------------------ W4A8 variant ----

def row_quant_s4(y: np.ndarray):
    """4-bit row quantization -> (codes [n, K_pad] int8 in -7..7, scales [n] fp32)."""
    y = np.ascontiguousarray(y, np.float32)
    n, kp = y.shape
    q = np.empty((n, kp), np.int8)
    s = np.empty(n, np.float32)
    lib().or_row_quant_s4(_p(y), n, kp, kp, _p(q), kp, _p(s))
    return q, s


def pack_s4(q: np.ndarray) -> np.ndarray:
    """codes [n, K_pad] (values -8..7) -> packed [n, K_pad / 2] bytes."""
    q = np.ascontiguousarray(q, np.int8)
    n, kp = q.shape
    assert kp % 64 == 0
    p = np.empty((n, kp // 2), np.uint8)
    lib().or_pack_s4(_p(q), n, kp, kp, _p(p), kp // 2)
    return p


def unpack_s4(p: np.ndarray, K_pad: int) -> np.ndarray:
    p = np.ascontiguousarray(p, np.uint8)
    n = p.shape[0]
    q = np.empty((n, K_pad), np.int8)
    lib().or_unpack_s4(_p(p), n, K_pad, p.shape[1], _p(q), K_pad)
    return q


def quant_weight_w4(w: np.ndarray, dtype: int, K: int):
    """Dense W [N, >=K] -> (packed 4-bit codes [N, K_pad / 2] uint8, scales [N] fp32)."""
    w = np.ascontiguousarray(w, _elem_dtype(dtype))
    n = w.shape[0]
    kp = padded_k(K)
    p = np.empty((n, kp // 2), np.uint8)
    s = np.empty(n, np.float32)
    rc = lib().or_quant_weight_w4(_p(w), dtype, w.shape[1], n, K, _p(p), kp // 2, _p(s))
    assert rc == 0
    return p, s


def gemm_s8s4(a: np.ndarray, b_s4: np.ndarray) -> np.ndarray:
    """int32 acc[M, N] = A[M, K_pad] . unpack(B)[N, K_pad]^T."""
    a = np.ascontiguousarray(a, np.int8)
    b_s4 = np.ascontiguousarray(b_s4, np.uint8)
    M, kp = a.shape
    N = b_s4.shape[0]
    acc = np.empty((M, N), np.int32)
    rc = lib().or_gemm_s8s4(_p(a), kp, _p(b_s4), b_s4.shape[1], M, N, kp, _p(acc), N)
    assert rc == 0
    return acc


def linear_w4a8(x: np.ndarray, x_dtype: int, K: int, swiglu: bool, w_s4: np.ndarray, w_scale: np.ndarray,
                out_dtype: int, bias=None) -> np.ndarray:
    """The W4A8 layer on the rows of x against a prepared 4-bit weight."""
    x = np.ascontiguousarray(x, _elem_dtype(x_dtype))
    w_s4 = np.ascontiguousarray(w_s4, np.uint8)
    w_scale = np.ascontiguousarray(w_scale, np.float32)
    M, N = x.shape[0], w_s4.shape[0]
    odt = {DT_BF16: np.uint16, DT_FP16: np.uint16, DT_FP32: np.float32, DT_I32: np.int32}[out_dtype]
    out = np.empty((M, N), odt)
    b, bp = _opt_f32(bias, N)
    rc = lib().or_linear_w4a8(_p(x), x_dtype, x.shape[1], int(swiglu), M, K, _p(w_s4), w_s4.shape[1],
                              _p(w_scale), N, bp, _p(out), out_dtype, N)
    assert rc == 0
    return out


# ------------------------------------------------------------ W4A4 variant ----

def quant_act_w4(x: np.ndarray, dtype: int, K: int, swiglu: bool = False):
    """X [M, >=K] (or H [M, >=2F]) -> (packed 4-bit codes [M, K_pad / 2] uint8, scales [M] fp32)."""
    x = np.ascontiguousarray(x, _elem_dtype(dtype))
    M = x.shape[0]
    kp = padded_k(K)
    p = np.empty((M, kp // 2), np.uint8)
    s = np.empty(M, np.float32)
    rc = lib().or_quant_act_w4(_p(x), dtype, x.shape[1], int(swiglu), M, K, _p(p), kp // 2, _p(s))
    assert rc == 0
    return p, s


def gemm_s4s4(a_s4: np.ndarray, b_s4: np.ndarray, K_pad: int) -> np.ndarray:
    """int32 acc[M, N] = unpack(A)[M, K_pad] . unpack(B)[N, K_pad]^T."""
    a_s4 = np.ascontiguousarray(a_s4, np.uint8)
    b_s4 = np.ascontiguousarray(b_s4, np.uint8)
    M, N = a_s4.shape[0], b_s4.shape[0]
    acc = np.empty((M, N), np.int32)
    rc = lib().or_gemm_s4s4(_p(a_s4), a_s4.shape[1], _p(b_s4), b_s4.shape[1], M, N, K_pad, _p(acc), N)
    assert rc == 0
    return acc


def linear_w4a4(x: np.ndarray, x_dtype: int, K: int, swiglu: bool, w_s4: np.ndarray, w_scale: np.ndarray,
                out_dtype: int, bias=None) -> np.ndarray:
    """The W4A4 layer on the rows of x against a prepared 4-bit weight."""
    x = np.ascontiguousarray(x, _elem_dtype(x_dtype))
    w_s4 = np.ascontiguousarray(w_s4, np.uint8)
    w_scale = np.ascontiguousarray(w_scale, np.float32)
    M, N = x.shape[0], w_s4.shape[0]
    odt = {DT_BF16: np.uint16, DT_FP16: np.uint16, DT_FP32: np.float32, DT_I32: np.int32}[out_dtype]
    out = np.empty((M, N), odt)
    b, bp = _opt_f32(bias, N)
    rc = lib().or_linear_w4a4(_p(x), x_dtype, x.shape[1], int(swiglu), M, K, _p(w_s4), w_s4.shape[1],
                              _p(w_scale), N, bp, _p(out), out_dtype, N)
    assert rc == 0
    return out


# ------------------------------------------- 4-bit codes in E2M3 fields ----

def e2m3(code: int) -> float:
    return float(lib().or_e2m3(code))


def pack_e2m3(q: np.ndarray) -> np.ndarray:
    """Codes [rows, K_pad] (-7..7, K_pad % 128 == 0) -> E2M3 fields in quads of rows:
    [ceil(rows / 4), 3 K_pad] uint8 (one array row per quad of four code rows)."""
    q = np.ascontiguousarray(q, np.int8)
    n, kp = q.shape
    assert kp % 128 == 0
    p = np.empty(((n + 3) // 4, 3 * kp), np.uint8)
    assert lib().or_pack_e2m3(_p(q), n, kp, kp, _p(p), 3 * kp) == 0
    return p


def unpack_e2m3(p: np.ndarray, K_pad: int, n_rows: int) -> np.ndarray:
    p = np.ascontiguousarray(p, np.uint8)
    assert p.shape[0] == (n_rows + 3) // 4
    q = np.empty((n_rows, K_pad), np.int8)
    assert lib().or_unpack_e2m3(_p(p), n_rows, K_pad, p.shape[1], _p(q), K_pad) == 0
    return q


def gemm_e2m3(a: np.ndarray, b: np.ndarray, K_pad: int, M: int, N: int) -> np.ndarray:
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    acc = np.empty((M, N), np.int32)
    assert lib().or_gemm_e2m3(_p(a), a.shape[1], _p(b), b.shape[1], M, N, K_pad, _p(acc), N) == 0
    return acc
