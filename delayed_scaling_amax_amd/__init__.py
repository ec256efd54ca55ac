"""Python binding of libfp8q.so: FP8 delayed scaling on MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/fp8q.h; every step of the
hot path runs in the library's HIP kernels.  torch is used only for device memory and
the current HIP stream.  Functions carry the C names:

  fp8_quantize_amax(src, dst, scale, amax, format)          one tensor, fused amax
  fp8_multi_quantize_amax([(src, dst, scale, amax, format), ...])   one launch
  fp8_multi_quantize_amax_timed(entries, start_event, stop_event)  the same, with
                            torch.cuda.Events set to the kernel's own start/stop
  fp8_multi_quantize_plan(entries) -> Plan     up to 2048 entries laid out once in a
                                               device workspace
  fp8_multi_quantize_amax_planned(plan)        the whole planned list, one launch
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


class fp8q_plan(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 16)]


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
    lib.fp8_multi_quantize_plan_bytes.argtypes = [ctypes.POINTER(fp8q_tensor), i32]
    lib.fp8_multi_quantize_plan_bytes.restype = i64
    lib.fp8_multi_quantize_plan.argtypes = [ctypes.POINTER(fp8q_tensor), i32, vp, i64,
                                            ctypes.POINTER(fp8q_plan), vp]
    lib.fp8_multi_quantize_amax_planned.argtypes = [ctypes.POINTER(fp8q_plan), vp]
    lib.fp8_multi_quantize_amax_noalloc.argtypes = [ctypes.POINTER(fp8q_tensor), i32, vp]
    lib.fp8_status_string.argtypes = [i32]
    lib.fp8_status_string.restype = ctypes.c_char_p
    for f in ("fp8_quantize_amax", "fp8_multi_quantize_amax", "fp8_multi_quantize_amax_timed",
              "fp8_gelu_quantize_amax",
              "fp8_layernorm_quantize_amax", "fp8_gemm", "fp8_dequantize", "fp8_amax_and_scale_update",
              "fp8_quantize_amax_and_update", "fp8_multi_quantize_plan",
              "fp8_multi_quantize_amax_planned", "fp8_multi_quantize_amax_noalloc"):
        getattr(lib, f).restype = i32
    return lib


lib = _load()


def fp8_status_string(status: int) -> str:
    return lib.fp8_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Fp8qError(fn, status)


def _on(t: torch.Tensor, name: str, dev: torch.device) -> None:
    """Every tensor of a call must live on the call's GPU: a host pointer or another
    device's pointer handed to a kernel would fault the GPU instead of raising."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (got device %s)" % (name, t.device))
    if t.device != dev:
        raise ValueError("%s is on %s, the call runs on %s" % (name, t.device, dev))


def _device(t: torch.Tensor, name: str) -> torch.device:
    """The GPU a call runs on: the device of its first tensor argument."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (got %s)" % (
            name, t.device if isinstance(t, torch.Tensor) else type(t).__name__))
    return t.device


def _dense(t: torch.Tensor, name: str, dev: torch.device) -> int:
    _on(t, name, dev)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _one_float(t: torch.Tensor, name: str, dev: torch.device) -> int:
    _on(t, name, dev)
    if t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError("%s must be a 1-element float32 tensor" % name)
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _single(fn: str, src, dst, scale, amax, format) -> None:
    dev = _device(src, "src")
    if not isinstance(dst, torch.Tensor) or dst.dtype != torch.uint8 or dst.numel() != src.numel():
        raise ValueError("dst must be uint8 with src.numel() elements")
    args = (_dense(src, "src", dev), _DTYPE.get(src.dtype, -1), _dense(dst, "dst", dev),
            src.numel(), int(format), _one_float(scale, "scale", dev),
            _one_float(amax, "amax", dev))
    with torch.cuda.device(dev):
        _check(fn, getattr(lib, fn)(*args, _stream(dev)))


def fp8_quantize_amax(src: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                      amax: torch.Tensor, format: int) -> None:
    _single("fp8_quantize_amax", src, dst, scale, amax, format)


def fp8_gelu_quantize_amax(src: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                           amax: torch.Tensor, format: int) -> None:
    _single("fp8_gelu_quantize_amax", src, dst, scale, amax, format)


def _opt_f32(t, n: int, name: str, dev: torch.device) -> int | None:
    if t is None:
        return None
    _on(t, name, dev)
    if t.dtype != torch.float32 or t.numel() != n:
        raise ValueError("%s must be a float32 tensor of %d elements" % (name, n))
    return _dense(t, name, dev)


def fp8_layernorm_quantize_amax(x: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                                amax: torch.Tensor, format: int, gamma=None, beta=None,
                                eps: float = 1e-6, mean=None, rstd=None) -> None:
    """LayerNorm over the last axis of x, quantized; mean/rstd (rows elements each) are
    optional outputs."""
    dev = _device(x, "x")
    if x.dim() < 1:
        raise ValueError("x must have a last axis")
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if not isinstance(dst, torch.Tensor) or dst.dtype != torch.uint8 or dst.numel() != x.numel():
        raise ValueError("dst must be uint8 with x.numel() elements")
    args = (_dense(x, "x", dev), _DTYPE.get(x.dtype, -1), _opt_f32(gamma, hidden, "gamma", dev),
            _opt_f32(beta, hidden, "beta", dev), float(eps), rows, hidden,
            _dense(dst, "dst", dev), int(format), _one_float(scale, "scale", dev),
            _one_float(amax, "amax", dev), _opt_f32(mean, rows, "mean", dev),
            _opt_f32(rstd, rows, "rstd", dev))
    with torch.cuda.device(dev):
        _check("fp8_layernorm_quantize_amax",
               lib.fp8_layernorm_quantize_amax(*args, _stream(dev)))


def fp8_gemm(A: torch.Tensor, a_format: int, B: torch.Tensor, b_format: int,
             a_scale: torch.Tensor, b_scale: torch.Tensor, C: torch.Tensor) -> None:
    """C (M, N) bf16/fp32 = a_scale * b_scale * decode(A) @ decode(B).T for uint8 code
    tensors A (M, K) and B (N, K)."""
    dev = _device(A, "A")
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("A, B and C must be 2-D")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shapes: A (M, K), B (N, K), C (M, N)")
    if A.dtype != torch.uint8 or B.dtype != torch.uint8:
        raise ValueError("A and B hold FP8 codes as uint8")
    args = (_dense(A, "A", dev), int(a_format), _dense(B, "B", dev), int(b_format), M, N, K,
            _one_float(a_scale, "a_scale", dev), _one_float(b_scale, "b_scale", dev),
            _dense(C, "C", dev), _DTYPE.get(C.dtype, -1))
    with torch.cuda.device(dev):
        _check("fp8_gemm", lib.fp8_gemm(*args, _stream(dev)))


def _entry_table(entries, dev: torch.device):
    arr = (fp8q_tensor * len(entries))()
    for i, (src, dst, scale, amax, fmt) in enumerate(entries):
        name = "entry %d " % i
        _on(src, name + "src", dev)
        if not isinstance(dst, torch.Tensor) or dst.dtype != torch.uint8 or dst.numel() != src.numel():
            raise ValueError("entry %d: dst must be uint8 with src.numel() elements" % i)
        arr[i] = fp8q_tensor(_dense(src, name + "src", dev), _dense(dst, name + "dst", dev),
                             src.numel(), _DTYPE.get(src.dtype, -1), int(fmt),
                             _one_float(scale, name + "scale", dev),
                             _one_float(amax, name + "amax", dev))
    return arr


def fp8_multi_quantize_amax(entries) -> None:
    """entries: sequence of (src, dst, scale, amax, format)."""
    entries = list(entries)
    if not entries:
        return
    dev = _device(entries[0][0], "entry 0 src")
    arr = _entry_table(entries, dev)
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
    dev = (_device(entries[0][0], "entry 0 src") if entries
           else torch.device("cuda", torch.cuda.current_device()))
    arr = _entry_table(entries, dev)
    with torch.cuda.device(dev):
        _check("fp8_multi_quantize_amax_timed",
               lib.fp8_multi_quantize_amax_timed(arr, len(entries), _stream(dev),
                                                 _event_handle(start_event),
                                                 _event_handle(stop_event)))


class Plan:
    """A list of quantize entries laid out once in a device workspace
    (fp8_multi_quantize_plan): fp8_multi_quantize_amax_planned(plan) quantizes the whole
    list in one launch.  Holds the workspace and the entries' tensors, so the pointers the
    plan records stay valid while it lives."""

    def __init__(self, entries, workspace, desc, device):
        self.entries = entries
        self.workspace = workspace
        self.desc = desc
        self.device = device


def fp8_multi_quantize_plan(entries, workspace: torch.Tensor | None = None) -> Plan:
    """entries: sequence of (src, dst, scale, amax, format), at most 2048.  workspace: a
    device uint8 tensor of at least fp8_multi_quantize_plan_bytes(entries) bytes, or
    None to allocate one.  Set-up call (the layout is copied from host memory, which HIP
    does synchronously); reuse the Plan every step."""
    entries = list(entries)
    dev = (_device(entries[0][0], "entry 0 src") if entries
           else torch.device("cuda", torch.cuda.current_device()))
    arr = _entry_table(entries, dev)
    need = int(lib.fp8_multi_quantize_plan_bytes(arr, len(entries)))
    if need < 0:
        raise Fp8qError("fp8_multi_quantize_plan_bytes", need)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _on(workspace, "workspace", dev)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace must hold %d bytes" % need)
    desc = fp8q_plan()
    with torch.cuda.device(dev):
        _check("fp8_multi_quantize_plan", lib.fp8_multi_quantize_plan(
            arr, len(entries), _dense(workspace, "workspace", dev), need, ctypes.byref(desc),
            _stream(dev)))
    return Plan(entries, workspace, desc, dev)


def fp8_multi_quantize_plan_bytes(entries) -> int:
    entries = list(entries)
    dev = (_device(entries[0][0], "entry 0 src") if entries
           else torch.device("cuda", torch.cuda.current_device()))
    need = int(lib.fp8_multi_quantize_plan_bytes(_entry_table(entries, dev), len(entries)))
    if need < 0:
        raise Fp8qError("fp8_multi_quantize_plan_bytes", need)
    return need


def fp8_multi_quantize_amax_planned(plan: Plan) -> None:
    """fp8_multi_quantize_amax over every entry of the plan, in one kernel launch."""
    if not isinstance(plan, Plan):
        raise ValueError("plan must come from fp8_multi_quantize_plan")
    with torch.cuda.device(plan.device):
        _check("fp8_multi_quantize_amax_planned", lib.fp8_multi_quantize_amax_planned(
            ctypes.byref(plan.desc), _stream(plan.device)))


def fp8_multi_quantize_amax_noalloc(entries) -> None:
    """fp8_multi_quantize_amax in one launch with the plan in the library's fixed device
    array (no device allocation; at most 2048 entries).  Calls that may overlap on one
    device race on that array."""
    entries = list(entries)
    if not entries:
        return
    dev = _device(entries[0][0], "entry 0 src")
    arr = _entry_table(entries, dev)
    with torch.cuda.device(dev):
        _check("fp8_multi_quantize_amax_noalloc",
               lib.fp8_multi_quantize_amax_noalloc(arr, len(entries), _stream(dev)))


def fp8_dequantize(src: torch.Tensor, dst: torch.Tensor, scale: torch.Tensor,
                   format: int) -> None:
    dev = _device(src, "src")
    if src.dtype != torch.uint8 or not isinstance(dst, torch.Tensor) or dst.numel() != src.numel():
        raise ValueError("src must be uint8 and dst must have src.numel() elements")
    args = (_dense(src, "src", dev), int(format), _dense(dst, "dst", dev),
            _DTYPE.get(dst.dtype, -1), src.numel(), _one_float(scale, "scale", dev))
    with torch.cuda.device(dev):
        _check("fp8_dequantize", lib.fp8_dequantize(*args, _stream(dev)))


def _update_args(amax, amax_history, scale, scale_inv, formats):
    """(device, H, n, pointers...) of the update's five arrays, all checked."""
    dev = _device(amax, "amax")
    for t, name in ((amax_history, "amax_history"), (scale, "scale"),
                    (scale_inv, "scale_inv"), (formats, "formats")):
        _on(t, name, dev)
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
    ptrs = (_dense(amax, "amax", dev), _dense(amax_history, "amax_history", dev),
            _dense(scale, "scale", dev), _dense(scale_inv, "scale_inv", dev),
            _dense(formats, "formats", dev))
    return dev, H, n, ptrs


def fp8_amax_and_scale_update(amax: torch.Tensor, amax_history: torch.Tensor,
                              scale: torch.Tensor, scale_inv: torch.Tensor,
                              formats: torch.Tensor, algo: int = AMAX_MAX, margin: int = 0,
                              reset_amax: bool = False) -> None:
    dev, H, n, ptrs = _update_args(amax, amax_history, scale, scale_inv, formats)
    with torch.cuda.device(dev):
        _check("fp8_amax_and_scale_update", lib.fp8_amax_and_scale_update(
            *ptrs, n, H, int(algo), int(margin), int(bool(reset_amax)), _stream(dev)))


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
    dev, H, n, ptrs = _update_args(amax, amax_history, scale, scale_inv, formats)
    _on(workspace, "workspace", dev)
    if workspace.numel() != 1 or workspace.element_size() != 4:
        raise ValueError("workspace must be one 4-byte element")
    arr = _entry_table(entries, dev)
    ws = _dense(workspace, "workspace", dev)
    with torch.cuda.device(dev):
        _check("fp8_quantize_amax_and_update", lib.fp8_quantize_amax_and_update(
            arr, len(entries), *ptrs, n, H, int(algo), int(margin), int(bool(reset_amax)), ws,
            _stream(dev), _event_handle(start_event), _event_handle(stop_event)))


__all__ = ["fp8_quantize_amax", "fp8_multi_quantize_amax", "fp8_multi_quantize_amax_timed",
           "fp8_multi_quantize_plan", "fp8_multi_quantize_plan_bytes",
           "fp8_multi_quantize_amax_planned", "Plan", "fp8q_plan",
           "fp8_multi_quantize_amax_noalloc",
           "fp8_quantize_amax_and_update",
           "fp8_gelu_quantize_amax",
           "fp8_layernorm_quantize_amax", "fp8_gemm", "fp8_dequantize",
           "fp8_amax_and_scale_update", "fp8_status_string", "fp8q_tensor", "Fp8qError",
           "E4M3", "E5M2", "BF16", "F32", "AMAX_MAX", "AMAX_MOST_RECENT", "LIB_PATH", "lib"]
