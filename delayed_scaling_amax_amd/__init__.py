"""Python binding of libfp8q.so: FP8 delayed scaling on MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/fp8q.h; every step of the
hot path runs in the library's HIP kernels.  torch is used only for device memory and
the current HIP stream.  Functions carry the C names:

  fp8_quantize_amax(src, dst, scale, amax, format)          one tensor, fused amax
  fp8_multi_quantize_amax([(src, dst, scale, amax, format), ...])   one launch
  fp8_multi_quantize_amax_timed(entries, start_event, stop_event)  the same, with
                            torch.cuda.Events set to the kernel's own start/stop
  fp8_gelu_quantize_amax(src, dst, scale, amax, format)     gelu(bf16 src), quantized
  fp8_layernorm_quantize_amax(x, dst, scale, amax, format, gamma=None, beta=None,
                              eps=1e-6, mean=None, rstd=None)  LayerNorm(x), quantized
  fp8_dequantize(src, dst, scale, format)
  fp8_gemm(A, a_format, B, b_format, a_scale, b_scale, C)   C = sa sb A @ B.T (FP8)
  fp8_amax_and_scale_update(amax, amax_history, scale, scale_inv, formats,
                            algo=AMAX_MAX, margin=0, reset_amax=False)
  fp8_quantize_amax_and_update(entries, amax, amax_history, scale, scale_inv, formats,
                               workspace, ...)   both of the above, one launch
  fp8_status_string(status)

`scale` / `amax` are 1-element float32 device tensors (or 1-element views into a
larger buffer); FP8 tensors are torch.uint8 holding the codes.  All calls enqueue on
the current stream of the tensors' device and return without synchronising.  A
missing library raises at import time: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8q.so")

E4M3, E5M2 = 0, 1
BF16, F32 = 0, 1
AMAX_MAX, AMAX_MOST_RECENT = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3

_DTYPE = {torch.bfloat16: BF16, torch.float32: F32}


class Fp8qError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %d (%s)" % (fn, status, fp8_status_string(status)))
        self.status = status


class fp8q_tensor(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("src_dtype", ctypes.c_int32), ("format", ctypes.c_int32),
                ("scale", ctypes.c_void_p), ("amax", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfp8q.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fp8_quantize_amax.argtypes = [vp, i32, vp, i64, i32, vp, vp, vp]
    lib.fp8_multi_quantize_amax.argtypes = [ctypes.POINTER(fp8q_tensor), i32, vp]
    lib.fp8_multi_quantize_amax_timed.argtypes = [ctypes.POINTER(fp8q_tensor), i32, vp, vp, vp]
    lib.fp8_gelu_quantize_amax.argtypes = [vp, i32, vp, i64, i32, vp, vp, vp]
    lib.fp8_layernorm_quantize_amax.argtypes = [vp, i32, vp, vp, ctypes.c_float, i64, i64, vp,
                                                i32, vp, vp, vp, vp, vp]
    lib.fp8_dequantize.argtypes = [vp, i32, vp, i32, i64, vp, vp]
    lib.fp8_gemm.argtypes = [vp, i32, vp, i32, i64, i64, i64, vp, vp, vp, i32, vp]
    lib.fp8_amax_and_scale_update.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, vp]
    lib.fp8_quantize_amax_and_update.argtypes = [ctypes.POINTER(fp8q_tensor), i32, vp, vp, vp,
                                                 vp, vp, i64, i64, i32, i32, i32, vp, vp, vp,
                                                 vp]
    lib.fp8_status_string.argtypes = [i32]
    lib.fp8_status_string.restype = ctypes.c_char_p
    for f in ("fp8_quantize_amax", "fp8_multi_quantize_amax", "fp8_multi_quantize_amax_timed",
              "fp8_gelu_quantize_amax",
              "fp8_layernorm_quantize_amax", "fp8_gemm", "fp8_dequantize", "fp8_amax_and_scale_update",
              "fp8_quantize_amax_and_update"):
        getattr(lib, f).restype = i32
    return lib


lib = _load()


def fp8_status_string(status: int) -> str:
    return lib.fp8_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Fp8qError(fn, status)


def _dense(t: torch.Tensor, name: str) -> int:
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _one_float(t: torch.Tensor, name: str) -> int:
    if t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError("%s must be a 1-element float32 tensor" % name)
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def fp8_quantize_amax(src: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                      amax: torch.Tensor, format: int) -> None:
    if dst.dtype != torch.uint8 or dst.numel() != src.numel():
        raise ValueError("dst must be uint8 with src.numel() elements")
    with torch.cuda.device(src.device):
        _check("fp8_quantize_amax", lib.fp8_quantize_amax(
            _dense(src, "src"), _DTYPE.get(src.dtype, -1), _dense(dst, "dst"), src.numel(),
            int(format), _one_float(scale, "scale"), _one_float(amax, "amax"),
            _stream(src.device)))


def fp8_gelu_quantize_amax(src: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                           amax: torch.Tensor, format: int) -> None:
    if dst.dtype != torch.uint8 or dst.numel() != src.numel():
        raise ValueError("dst must be uint8 with src.numel() elements")
    with torch.cuda.device(src.device):
        _check("fp8_gelu_quantize_amax", lib.fp8_gelu_quantize_amax(
            _dense(src, "src"), _DTYPE.get(src.dtype, -1), _dense(dst, "dst"), src.numel(),
            int(format), _one_float(scale, "scale"), _one_float(amax, "amax"),
            _stream(src.device)))


def _opt_f32(t, n: int, name: str) -> int | None:
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() != n:
        raise ValueError("%s must be a float32 tensor of %d elements" % (name, n))
    return _dense(t, name)


def fp8_layernorm_quantize_amax(x: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                                amax: torch.Tensor, format: int, gamma=None, beta=None,
                                eps: float = 1e-6, mean=None, rstd=None) -> None:
    """LayerNorm over the last axis of x, quantized; mean/rstd (rows elements each) are
    optional outputs."""
    if x.dim() < 1:
        raise ValueError("x must have a last axis")
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if dst.dtype != torch.uint8 or dst.numel() != x.numel():
        raise ValueError("dst must be uint8 with x.numel() elements")
    with torch.cuda.device(x.device):
        _check("fp8_layernorm_quantize_amax", lib.fp8_layernorm_quantize_amax(
            _dense(x, "x"), _DTYPE.get(x.dtype, -1), _opt_f32(gamma, hidden, "gamma"),
            _opt_f32(beta, hidden, "beta"), float(eps), rows, hidden, _dense(dst, "dst"),
            int(format), _one_float(scale, "scale"), _one_float(amax, "amax"),
            _opt_f32(mean, rows, "mean"), _opt_f32(rstd, rows, "rstd"), _stream(x.device)))


def fp8_gemm(A: torch.Tensor, a_format: int, B: torch.Tensor, b_format: int,
             a_scale: torch.Tensor, b_scale: torch.Tensor, C: torch.Tensor) -> None:
    """C (M, N) bf16/fp32 = a_scale * b_scale * decode(A) @ decode(B).T for uint8 code
    tensors A (M, K) and B (N, K)."""
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("A, B and C must be 2-D")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shapes: A (M, K), B (N, K), C (M, N)")
    if A.dtype != torch.uint8 or B.dtype != torch.uint8:
        raise ValueError("A and B hold FP8 codes as uint8")
    with torch.cuda.device(A.device):
        _check("fp8_gemm", lib.fp8_gemm(
            _dense(A, "A"), int(a_format), _dense(B, "B"), int(b_format), M, N, K,
            _one_float(a_scale, "a_scale"), _one_float(b_scale, "b_scale"), _dense(C, "C"),
            _DTYPE.get(C.dtype, -1), _stream(A.device)))


def _entry_table(entries):
    arr = (fp8q_tensor * len(entries))()
    for i, (src, dst, scale, amax, fmt) in enumerate(entries):
        if dst.dtype != torch.uint8 or dst.numel() != src.numel():
            raise ValueError("entry %d: dst must be uint8 with src.numel() elements" % i)
        arr[i] = fp8q_tensor(_dense(src, "src"), _dense(dst, "dst"), src.numel(),
                             _DTYPE.get(src.dtype, -1), int(fmt), _one_float(scale, "scale"),
                             _one_float(amax, "amax"))
    return arr


def fp8_multi_quantize_amax(entries) -> None:
    """entries: sequence of (src, dst, scale, amax, format)."""
    entries = list(entries)
    if not entries:
        return
    arr = _entry_table(entries)
    dev = entries[0][0].device
    with torch.cuda.device(dev):
        _check("fp8_multi_quantize_amax",
               lib.fp8_multi_quantize_amax(arr, len(entries), _stream(dev)))


def _event_handle(ev) -> int | None:
    """hipEvent_t of a torch.cuda.Event (created with enable_timing=True), or None."""
    if ev is None:
        return None
    if ev.cuda_event == 0:  # torch creates the event at its first record
        ev.record()
    return int(ev.cuda_event)


def fp8_multi_quantize_amax_timed(entries, start_event, stop_event) -> None:
    """fp8_multi_quantize_amax whose kernel launches set two torch.cuda.Event objects
    (enable_timing=True; either may be None) to the kernels' own start and stop times:
    start_event.elapsed_time(stop_event) is the kernels' duration without the dispatch
    latency that events recorded on the stream around the call also span."""
    entries = list(entries)
    dev = entries[0][0].device if entries else torch.device("cuda", torch.cuda.current_device())
    arr = _entry_table(entries)
    with torch.cuda.device(dev):
        _check("fp8_multi_quantize_amax_timed",
               lib.fp8_multi_quantize_amax_timed(arr, len(entries), _stream(dev),
                                                 _event_handle(start_event),
                                                 _event_handle(stop_event)))


def fp8_dequantize(src: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                   format: int) -> None:
    if src.dtype != torch.uint8 or dst.numel() != src.numel():
        raise ValueError("src must be uint8 and dst must have src.numel() elements")
    with torch.cuda.device(src.device):
        _check("fp8_dequantize", lib.fp8_dequantize(
            _dense(src, "src"), int(format), _dense(dst, "dst"), _DTYPE.get(dst.dtype, -1),
            src.numel(), _one_float(scale, "scale"), _stream(src.device)))


def _update_shape(amax, amax_history, scale, scale_inv, formats):
    if amax_history.dim() != 2:
        raise ValueError("amax_history must be [history_len, n]")
    H, n = amax_history.shape
    for t, name in ((amax, "amax"), (scale, "scale"), (scale_inv, "scale_inv")):
        if t.dtype != torch.float32 or t.numel() != n:
            raise ValueError("%s must be float32 with n elements" % name)
    if amax_history.dtype != torch.float32:
        raise ValueError("amax_history must be float32")
    if formats.dtype != torch.uint8 or formats.numel() != n:
        raise ValueError("formats must be uint8 with n elements")
    return H, n


def fp8_amax_and_scale_update(amax: torch.Tensor, amax_history: torch.Tensor,
                              scale: torch.Tensor, scale_inv: torch.Tensor,
                              formats: torch.Tensor, algo: int = AMAX_MAX, margin: int = 0,
                              reset_amax: bool = False) -> None:
    H, n = _update_shape(amax, amax_history, scale, scale_inv, formats)
    with torch.cuda.device(amax.device):
        _check("fp8_amax_and_scale_update", lib.fp8_amax_and_scale_update(
            _dense(amax, "amax"), _dense(amax_history, "amax_history"), _dense(scale, "scale"),
            _dense(scale_inv, "scale_inv"), _dense(formats, "formats"), n, H, int(algo),
            int(margin), int(bool(reset_amax)), _stream(amax.device)))



def fp8_quantize_amax_and_update(entries, amax: torch.Tensor, amax_history: torch.Tensor,
                                 scale: torch.Tensor, scale_inv: torch.Tensor,
                                 formats: torch.Tensor, workspace: torch.Tensor,
                                 algo: int = AMAX_MAX, margin: int = 0,
                                 reset_amax: bool = False, start_event=None,
                                 stop_event=None) -> None:
    """One delayed-scaling step: fp8_multi_quantize_amax(entries) then
    fp8_amax_and_scale_update(...), in one kernel launch when it fits.  workspace: a
    1-element int32/uint32 device tensor holding 0 (every call leaves it 0)."""
    entries = list(entries)
    H, n = _update_shape(amax, amax_history, scale, scale_inv, formats)
    if workspace.numel() != 1 or workspace.element_size() != 4:
        raise ValueError("workspace must be one 4-byte element")
    arr = _entry_table(entries)
    with torch.cuda.device(amax.device):
        _check("fp8_quantize_amax_and_update", lib.fp8_quantize_amax_and_update(
            arr, len(entries), _dense(amax, "amax"), _dense(amax_history, "amax_history"),
            _dense(scale, "scale"), _dense(scale_inv, "scale_inv"), _dense(formats, "formats"),
            n, H, int(algo), int(margin), int(bool(reset_amax)), _dense(workspace, "workspace"),
            _stream(amax.device), _event_handle(start_event), _event_handle(stop_event)))


__all__ = ["fp8_quantize_amax", "fp8_multi_quantize_amax", "fp8_multi_quantize_amax_timed",
           "fp8_quantize_amax_and_update",
           "fp8_gelu_quantize_amax",
           "fp8_layernorm_quantize_amax", "fp8_gemm", "fp8_dequantize",
           "fp8_amax_and_scale_update", "fp8_status_string", "fp8q_tensor", "Fp8qError",
           "E4M3", "E5M2", "BF16", "F32", "AMAX_MAX", "AMAX_MOST_RECENT", "LIB_PATH", "lib"]
