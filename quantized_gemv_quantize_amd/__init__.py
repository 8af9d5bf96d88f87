"""MI355X block-quantized GEMV (ggml Q8_0 / Q4_0 / Q5_0 / Q4_K / Q5_K / Q6_K) - Python binding.

A thin ctypes binding over libqk.so (C ABI in include/qk.h).  Functions carry
the C names and only marshal arguments: torch tensors supply device pointers
and the current stream; every step of the computation runs in the HIP kernels.
There is no fallback: if libqk.so is missing or cannot be loaded, calls raise.
"""
import ctypes
import os

QK_TYPE_Q4_0 = 2
QK_TYPE_Q4_1 = 3
QK_TYPE_Q5_0 = 6
QK_TYPE_Q5_1 = 7
QK_TYPE_Q8_0 = 8
QK_TYPE_Q8_1 = 9
QK_TYPE_Q2_K = 10
QK_TYPE_Q3_K = 11
QK_TYPE_Q4_K = 12
QK_TYPE_Q5_K = 13
QK_TYPE_Q6_K = 14
QK_TYPE_Q8_K = 15
WEIGHT_TYPES = (QK_TYPE_Q8_0, QK_TYPE_Q4_0, QK_TYPE_Q5_0, QK_TYPE_Q4_1, QK_TYPE_Q5_1, QK_TYPE_Q2_K,
                QK_TYPE_Q3_K, QK_TYPE_Q4_K, QK_TYPE_Q5_K, QK_TYPE_Q6_K)
DEQUANT_TYPES = WEIGHT_TYPES
QUANT_ROW_TYPES = (QK_TYPE_Q8_0, QK_TYPE_Q4_0, QK_TYPE_Q4_1, QK_TYPE_Q5_0)
QK_EPI_NONE = 0
QK_EPI_SWIGLU = 1
TYPE_NAMES = {QK_TYPE_Q4_0: "Q4_0", QK_TYPE_Q4_1: "Q4_1", QK_TYPE_Q5_0: "Q5_0", QK_TYPE_Q5_1: "Q5_1",
              QK_TYPE_Q8_0: "Q8_0", QK_TYPE_Q4_K: "Q4_K", QK_TYPE_Q5_K: "Q5_K", QK_TYPE_Q6_K: "Q6_K",
              QK_TYPE_Q8_1: "Q8_1", QK_TYPE_Q2_K: "Q2_K", QK_TYPE_Q3_K: "Q3_K", QK_TYPE_Q8_K: "Q8_K"}

# the in-tree build; QK_LIB_PATH names another build of the same sources (the
# host-sanitizer test runs the host-side checks against one)
DEFAULT_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqk.so")
LIB_PATH = os.environ.get("QK_LIB_PATH") or DEFAULT_LIB_PATH

_lib = None


class QKError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_str(status)})")


def lib():
    """Load libqk.so once.  torch is imported first so that the library binds to
    the HIP runtime torch already mapped (they share the soname)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (HIP runtime must be torch's)
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python quantized_gemv_quantize_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.qk_block_elems.restype = i64
        L.qk_block_elems.argtypes = [i32]
        L.qk_block_bytes.restype = i64
        L.qk_block_bytes.argtypes = [i32]
        L.qk_row_bytes.restype = i64
        L.qk_row_bytes.argtypes = [i32, i64]
        L.qk_act_type.restype = i32
        L.qk_act_type.argtypes = [i32]
        L.qk_status_str.restype = ctypes.c_char_p
        L.qk_status_str.argtypes = [i32]
        L.qk_max_n_in.restype = i64
        L.qk_max_n_in.argtypes = [i32]
        L.qk_quantize_act.restype = i32
        L.qk_quantize_act.argtypes = [i32, p, p, i64, i64, p]
        L.qk_quantize_act_timed.restype = i32
        L.qk_quantize_act_timed.argtypes = [i32, p, p, i64, i64, p, p, p]
        L.qk_quantize_row.restype = i32
        L.qk_quantize_row.argtypes = [i32, p, p, i64, p]
        L.qk_gemv.restype = i32
        L.qk_gemv.argtypes = [i32, p, i64, i64, p, i64, p, p]
        L.qk_gemv_typed.restype = i32
        L.qk_gemv_typed.argtypes = [i32, i32, p, i64, i64, p, i64, p, p]
        L.qk_gemv_timed.restype = i32
        L.qk_gemv_timed.argtypes = [i32, p, i64, i64, p, i64, p, p, p, p]
        L.qk_gemv_block_sums.restype = i32
        L.qk_gemv_block_sums.argtypes = [i32, p, i64, i64, p, i64, p, p]
        L.qk_dequantize_row.restype = i32
        L.qk_dequantize_row.argtypes = [i32, p, p, i64, p]
        L.qk_gemv_pair.restype = i32
        L.qk_gemv_pair.argtypes = [i32, p, p, i64, i64, p, i64, i32, p, p]
        L.qk_gemv_pair_timed.restype = i32
        L.qk_gemv_pair_timed.argtypes = [i32, p, p, i64, i64, p, i64, i32, p, p, p, p]
        L.qk_read_probe.restype = i32
        L.qk_read_probe.argtypes = [p, i64, p, p, p, p]
        L.qk_read_probe_ex.restype = i32
        L.qk_read_probe_ex.argtypes = [p, i64, p, i32, i64, i32, p, p, p]
        _lib = L
    return _lib


def status_str(status):
    return lib().qk_status_str(int(status)).decode()


def qk_block_elems(t):
    return int(lib().qk_block_elems(t))


def qk_block_bytes(t):
    return int(lib().qk_block_bytes(t))


def qk_row_bytes(t, n):
    return int(lib().qk_row_bytes(t, n))


def qk_act_type(t):
    return int(lib().qk_act_type(t))


def qk_max_n_in(t):
    return int(lib().qk_max_n_in(t))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise QKError(rc, what)


def qk_quantize_act(act_type, x, xq=None, stream=None):
    """Quantize x (f32 [ncols, n] or [n], device) into act blocks; returns xq
    (uint8 [ncols, row_bytes])."""
    import torch
    n = x.shape[-1]
    ncols = x.numel() // n if n else 0
    if xq is None:
        xq = torch.empty((ncols, max(qk_row_bytes(act_type, n), 0)), dtype=torch.uint8,
                         device=x.device)
    _check(lib().qk_quantize_act(act_type, _ptr(x), _ptr(xq), n, ncols, _stream(stream)),
           "qk_quantize_act")
    return xq


def qk_quantize_act_timed(act_type, x, xq, ev_start, ev_stop, stream=None):
    """qk_quantize_act whose kernel launch records the torch.cuda.Event(enable_timing=True)
    pair itself (either may be None)."""
    n = x.shape[-1]
    ncols = x.numel() // n if n else 0
    e0 = ctypes.c_void_p(ev_start.cuda_event) if ev_start is not None else None
    e1 = ctypes.c_void_p(ev_stop.cuda_event) if ev_stop is not None else None
    _check(lib().qk_quantize_act_timed(act_type, _ptr(x), _ptr(xq), n, ncols, _stream(stream), e0, e1),
           "qk_quantize_act_timed")
    return xq


def qk_quantize_row(t, x, dst=None, stream=None):
    """Quantize f32 weights x (device, numel a multiple of 32) into GGUF blocks of
    type t; returns dst (uint8 [row_bytes])."""
    import torch
    n = x.numel()
    if dst is None:
        dst = torch.empty((max(qk_row_bytes(t, n), 0),), dtype=torch.uint8, device=x.device)
    _check(lib().qk_quantize_row(t, _ptr(x), _ptr(dst), n, _stream(stream)),
           "qk_quantize_row")
    return dst


def qk_gemv(w_type, W, n_out, n_in, xq, ncols=1, y=None, stream=None):
    """y [ncols, n_out] f32 = W x for quantized W (device uint8) and act blocks xq."""
    import torch
    if y is None:
        y = torch.empty((ncols, n_out), dtype=torch.float32, device=W.device)
    _check(lib().qk_gemv(w_type, _ptr(W), n_out, n_in, _ptr(xq), ncols, _ptr(y),
                         _stream(stream)), "qk_gemv")
    return y


def qk_gemv_typed(w_type, act_type, W, n_out, n_in, xq, ncols=1, y=None, stream=None):
    """qk_gemv with the activation type of xq stated: QKError (QK_E_PAIR) when it is
    not qk_act_type(w_type)."""
    import torch
    if y is None:
        y = torch.empty((ncols, n_out), dtype=torch.float32, device=W.device)
    _check(lib().qk_gemv_typed(w_type, act_type, _ptr(W), n_out, n_in, _ptr(xq), ncols, _ptr(y),
                               _stream(stream)), "qk_gemv_typed")
    return y


def qk_gemv_timed(w_type, W, n_out, n_in, xq, ncols, y, ev_start, ev_stop, stream=None):
    """qk_gemv with torch.cuda.Event(enable_timing=True) pair recorded by the
    kernel launch itself (start of the first / end of the last GEMV kernel)."""
    e0 = ctypes.c_void_p(ev_start.cuda_event) if ev_start is not None else None
    e1 = ctypes.c_void_p(ev_stop.cuda_event) if ev_stop is not None else None
    _check(lib().qk_gemv_timed(w_type, _ptr(W), n_out, n_in, _ptr(xq), ncols, _ptr(y),
                               _stream(stream), e0, e1), "qk_gemv_timed")
    return y


def qk_gemv_block_sums(w_type, W, n_out, n_in, xq, ncols=1, sums=None, stream=None):
    """Per-block int32 sums [ncols, n_out, n_in/block, k] of the GEMV kernels."""
    import torch
    k = 2 if w_type in (QK_TYPE_Q2_K, QK_TYPE_Q4_K, QK_TYPE_Q5_K) else 1
    nb = n_in // qk_block_elems(w_type) if qk_block_elems(w_type) else 0
    if sums is None:
        sums = torch.empty((ncols, n_out, nb, k), dtype=torch.int32, device=W.device)
    _check(lib().qk_gemv_block_sums(w_type, _ptr(W), n_out, n_in, _ptr(xq), ncols, _ptr(sums),
                                    _stream(stream)), "qk_gemv_block_sums")
    return sums


def qk_dequantize_row(t, src, n, dst=None, stream=None):
    """f32 [n] values of n elements (whole blocks) of type t."""
    import torch
    if dst is None:
        dst = torch.empty((n,), dtype=torch.float32, device=src.device)
    _check(lib().qk_dequantize_row(t, _ptr(src), _ptr(dst), n, _stream(stream)),
           "qk_dequantize_row")
    return dst


def qk_gemv_pair(w_type, W1, W2, n_out, n_in, xq, ncols=1, epilogue=QK_EPI_NONE, out=None,
                 stream=None):
    """Gate and up projections in one launch: out [ncols, 2, n_out] (y1, y2), or
    [ncols, n_out] silu(y1) * y2 with epilogue=QK_EPI_SWIGLU."""
    import torch
    if out is None:
        shape = (ncols, n_out) if epilogue == QK_EPI_SWIGLU else (ncols, 2, n_out)
        out = torch.empty(shape, dtype=torch.float32, device=W1.device)
    _check(lib().qk_gemv_pair(w_type, _ptr(W1), _ptr(W2), n_out, n_in, _ptr(xq), ncols, epilogue,
                              _ptr(out), _stream(stream)), "qk_gemv_pair")
    return out


def qk_gemv_pair_timed(w_type, W1, W2, n_out, n_in, xq, ncols, epilogue, out, ev_start, ev_stop,
                       stream=None):
    """qk_gemv_pair with an event pair recorded by its kernel launch."""
    e0 = ctypes.c_void_p(ev_start.cuda_event) if ev_start is not None else None
    e1 = ctypes.c_void_p(ev_stop.cuda_event) if ev_stop is not None else None
    _check(lib().qk_gemv_pair_timed(w_type, _ptr(W1), _ptr(W2), n_out, n_in, _ptr(xq), ncols,
                                    epilogue, _ptr(out), _stream(stream), e0, e1),
           "qk_gemv_pair_timed")
    return out


def qk_read_probe(src, nbytes, out=None, ev_start=None, ev_stop=None, stream=None):
    """Read-stream probe over the first nbytes of src (device): returns out, uint32
    [ceil(nbytes / 2048)], the XOR of each 2048-byte group's 32-bit words.  The
    events (torch.cuda.Event(enable_timing=True)) are recorded by the launch."""
    import torch
    if out is None:
        out = torch.empty(((max(nbytes, 0) + 2047) // 2048,), dtype=torch.int32, device=src.device)
    e0 = ctypes.c_void_p(ev_start.cuda_event) if ev_start is not None else None
    e1 = ctypes.c_void_p(ev_stop.cuda_event) if ev_stop is not None else None
    _check(lib().qk_read_probe(_ptr(src), nbytes, _ptr(out), _stream(stream), e0, e1),
           "qk_read_probe")
    return out


def qk_read_probe_ex(src, nbytes, kb_per_wave=2, grid_blocks=0, nontemporal=0, out=None, ev_start=None,
                     ev_stop=None, stream=None):
    """qk_read_probe with its load pattern as arguments: returns out, uint32
    [ceil(nbytes / (1024 kb_per_wave))], the XOR of each group's 32-bit words."""
    import torch
    gb = 1024 * kb_per_wave
    if out is None:
        out = torch.empty(((max(nbytes, 0) + gb - 1) // gb,), dtype=torch.int32, device=src.device)
    e0 = ctypes.c_void_p(ev_start.cuda_event) if ev_start is not None else None
    e1 = ctypes.c_void_p(ev_stop.cuda_event) if ev_stop is not None else None
    _check(lib().qk_read_probe_ex(_ptr(src), nbytes, _ptr(out), kb_per_wave, grid_blocks, nontemporal,
                                  _stream(stream), e0, e1), "qk_read_probe_ex")
    return out
