"""ctypes view of the scalar C oracle (qk_oracle.c).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
only marshals numpy arrays; all arithmetic is in qk_oracle.c.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q8_1, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, Q8_K = 2, 3, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("QK_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.orc_block_elems.restype = i64
        L.orc_block_elems.argtypes = [i32]
        L.orc_block_bytes.restype = i64
        L.orc_block_bytes.argtypes = [i32]
        L.orc_row_bytes.restype = i64
        L.orc_row_bytes.argtypes = [i32, i64]
        L.orc_act_type.restype = i32
        L.orc_act_type.argtypes = [i32]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        for name in ("orc_quantize_q8_0", "orc_quantize_q8_K", "orc_quantize_q4_0",
                     "orc_quantize_q4_1", "orc_quantize_q5_0", "orc_quantize_q8_1"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [p, p, i64]
        L.orc_dequantize.restype = i32
        L.orc_dequantize.argtypes = [i32, p, p, i64]
        L.orc_sums_per_block.restype = i64
        L.orc_sums_per_block.argtypes = [i32]
        L.orc_block_sums.restype = i32
        L.orc_block_sums.argtypes = [i32, p, p, i64, p]
        L.orc_vec_dot.restype = i32
        L.orc_vec_dot.argtypes = [i32, p, p, i64, p, p]
        L.orc_gemv.restype = i32
        L.orc_gemv.argtypes = [i32, p, i64, i64, p, i64, p, p]
        L.orc_gemv_block_sums.restype = i32
        L.orc_gemv_block_sums.argtypes = [i32, p, i64, i64, p, i64, p]
        L.orc_swiglu.restype = i32
        L.orc_swiglu.argtypes = [p, p, i64, p]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle returned {rc}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _u8(x):
    return np.ascontiguousarray(x, dtype=np.uint8)


def block_elems(t):
    return int(lib().orc_block_elems(t))


def block_bytes(t):
    return int(lib().orc_block_bytes(t))


def row_bytes(t, n):
    return int(lib().orc_row_bytes(t, n))


def act_type(t):
    return int(lib().orc_act_type(t))


def f16_to_f32(h):
    return float(lib().orc_f16_to_f32(int(h)))


def f32_to_f16(f):
    return int(lib().orc_f32_to_f16(float(np.float32(f))))


def quantize(t, x):
    """Quantize a float32 array (last axis n) to blocks of type t (Q8_0, Q8_1, Q8_K,
    Q4_0, Q4_1, Q5_0)."""
    x = _f32(x)
    n = x.shape[-1]
    rows = x.reshape(-1, n)
    fn = {Q8_0: lib().orc_quantize_q8_0, Q8_K: lib().orc_quantize_q8_K,
          Q4_0: lib().orc_quantize_q4_0, Q4_1: lib().orc_quantize_q4_1,
          Q5_0: lib().orc_quantize_q5_0, Q8_1: lib().orc_quantize_q8_1}[t]
    rb = row_bytes(t, n)
    if rb == 0:
        raise OracleError(f"n={n} is not whole blocks of type {t}")
    out = np.zeros((rows.shape[0], rb), dtype=np.uint8)
    for i in range(rows.shape[0]):
        _check(fn(_ptr(rows[i]), _ptr(out[i]), n), "quantize")
    return out.reshape(*x.shape[:-1], rb)


def dequantize(t, src, n):
    """Dequantize n elements (whole blocks) of type t to float32."""
    src = _u8(src).reshape(-1)
    out = np.zeros(n, dtype=np.float32)
    _check(lib().orc_dequantize(t, _ptr(src), _ptr(out), n), "dequantize")
    return out


def block_sums(wt, w_row, xq_row, n):
    """Exact int32 sums per weight block of one row: shape [n/block, k]."""
    k = int(lib().orc_sums_per_block(wt))
    nb = n // block_elems(wt)
    out = np.zeros((nb, k), dtype=np.int32)
    _check(lib().orc_block_sums(wt, _ptr(_u8(w_row)), _ptr(_u8(xq_row)), n, _ptr(out)),
           "block_sums")
    return out


def vec_dot(wt, w_row, xq_row, n):
    """(f32 result, tolerance scale in f64) of one weight row against one act row: the
    sum over blocks of the absolute float terms of each block step (|c_b| for the
    one-term formats; |scale term| + |min term| for Q4_K and Q5_K)."""
    y = np.zeros(1, dtype=np.float32)
    l1 = np.zeros(1, dtype=np.float64)
    _check(lib().orc_vec_dot(wt, _ptr(_u8(w_row)), _ptr(_u8(xq_row)), n, _ptr(y), _ptr(l1)),
           "vec_dot")
    return float(y[0]), float(l1[0])


def gemv_block_sums(wt, W, n_out, n_in, xq, ncols=1):
    """block_sums of every (column, row): shape [ncols, n_out, n_in/block, k]."""
    k = int(lib().orc_sums_per_block(wt))
    out = np.zeros((ncols, n_out, n_in // block_elems(wt), k), dtype=np.int32)
    _check(lib().orc_gemv_block_sums(wt, _ptr(_u8(W)), n_out, n_in, _ptr(_u8(xq)), ncols, _ptr(out)),
           "gemv_block_sums")
    return out


def gemv(wt, W, n_out, n_in, xq, ncols=1):
    """y [ncols, n_out] f32 and l1 [ncols, n_out] f64 (the vec_dot tolerance scale per
    output)."""
    y = np.zeros((ncols, n_out), dtype=np.float32)
    l1 = np.zeros((ncols, n_out), dtype=np.float64)
    _check(lib().orc_gemv(wt, _ptr(_u8(W)), n_out, n_in, _ptr(_u8(xq)), ncols, _ptr(y),
                          _ptr(l1)), "gemv")
    return y, l1


def swiglu(g, u):
    """h = silu(g) * u in f64 from f32 g and u of the same shape."""
    g32 = np.ascontiguousarray(g, dtype=np.float32)
    u32 = np.ascontiguousarray(u, dtype=np.float32)
    assert g32.shape == u32.shape
    h = np.zeros(g32.shape, dtype=np.float64)
    _check(lib().orc_swiglu(_ptr(g32), _ptr(u32), g32.size, _ptr(h)), "swiglu")
    return h
