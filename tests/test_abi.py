"""The C-ABI library loads without a GPU, exports what include/fp8q.h declares, and
rejects invalid arguments on the host before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fp8_quantize_amax", "fp8_multi_quantize_amax", "fp8_multi_quantize_amax_timed",
        "fp8_gelu_quantize_amax", "fp8_layernorm_quantize_amax", "fp8_quantize_amax_and_update", "fp8_dequantize", "fp8_amax_and_scale_update",
        "fp8_gemm", "fp8_status_string", "fp8_multi_quantize_plan_bytes",
        "fp8_multi_quantize_plan", "fp8_multi_quantize_amax_planned",
        "fp8_multi_quantize_amax_noalloc"])


def test_library_exports_every_declared_symbol():
    import delayed_scaling_amax_amd as d
    out = subprocess.run(["nm", "-D", "--defined-only", d.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    missing = set(declared_functions()) - exported
    assert not missing, missing
    for name in declared_functions():
        assert hasattr(d.lib, name)


def test_header_compiles_as_c_and_cxx(tmp_path):
    for lang, comp in (("c", "gcc"), ("c++", "g++")):
        src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
        src.write_text('#include "fp8q.h"\nint main(void){ fp8q_tensor t; (void)t; '
                       'return FP8Q_OK + (int)sizeof(fp8q_tensor) - 48; }\n')
        exe = tmp_path / ("t_" + lang)
        subprocess.run([comp, "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src),
                        "-o", str(exe)], check=True)
        assert subprocess.run([str(exe)]).returncode == 0


def test_struct_layout_matches_binding():
    import delayed_scaling_amax_amd as d
    assert ctypes.sizeof(d.fp8q_tensor) == 48
    assert [f[0] for f in d.fp8q_tensor._fields_] == ["src", "dst", "numel", "src_dtype",
                                                        "format", "scale", "amax"]


def test_status_strings():
    import delayed_scaling_amax_amd as d
    assert d.fp8_status_string(0) == "ok"
    for st in (-1, -2, -3, 7):
        assert isinstance(d.fp8_status_string(st), str) and d.fp8_status_string(st)


BAD = 0x1000  # a non-NULL pointer value that is never dereferenced (validation fails first)


@pytest.mark.parametrize("args", [
    (None, 0, None, 10, 0, BAD, BAD),        # NULL src/dst with numel > 0
    (BAD, 0, BAD, -1, 0, BAD, BAD),          # negative numel
    (BAD, 2, BAD, 10, 0, BAD, BAD),          # bad src dtype
    (BAD, 0, BAD, 10, 2, BAD, BAD),          # bad format
    (BAD, 0, BAD, 10, 0, None, BAD),         # NULL scale
    (BAD, 0, BAD, 10, 0, BAD, None),         # NULL amax
])
def test_quantize_rejects_invalid(args):
    import delayed_scaling_amax_amd as d
    assert d.lib.fp8_quantize_amax(*args, None) == d.EINVAL
    assert d.lib.fp8_gelu_quantize_amax(*args, None) == d.EINVAL


def _ln(d, x=BAD, dt=0, g=None, b=None, eps=1e-6, rows=4, H=64, dst=BAD, fmt=0, s=BAD,
        a=BAD):
    return d.lib.fp8_layernorm_quantize_amax(x, dt, g, b, eps, rows, H, dst, fmt, s, a, None,
                                             None, None)


def test_layernorm_quantize_validation():
    import delayed_scaling_amax_amd as d
    assert _ln(d, rows=-1) == d.EINVAL
    assert _ln(d, H=-8) == d.EINVAL
    assert _ln(d, fmt=2) == d.EINVAL
    assert _ln(d, dt=2) == d.EINVAL
    assert _ln(d, s=None) == d.EINVAL and _ln(d, a=None) == d.EINVAL
    assert _ln(d, eps=-1.0) == d.EINVAL and _ln(d, eps=float("nan")) == d.EINVAL
    assert _ln(d, eps=float("inf")) == d.EINVAL
    assert _ln(d, x=None) == d.EINVAL and _ln(d, dst=None) == d.EINVAL
    assert _ln(d, dt=d.F32) == d.EUNSUPPORTED
    assert _ln(d, H=12) == d.EUNSUPPORTED          # not a multiple of 8
    assert _ln(d, H=16392) == d.EUNSUPPORTED       # longer rows than the kernel holds
    assert _ln(d, x=BAD + 8) == d.EUNSUPPORTED     # x not 16-byte aligned
    assert _ln(d, dst=BAD + 4) == d.EUNSUPPORTED   # dst not 8-byte aligned
    assert _ln(d, rows=2 ** 62, H=8) == d.EINVAL   # rows * hidden overflows
    # empty is a no-op that touches nothing
    assert _ln(d, x=None, dst=None, rows=0) == d.OK
    assert _ln(d, x=None, dst=None, H=0) == d.OK


def _gemm(d, A=BAD, fa=0, B=BAD, fb=0, M=4, N=4, K=32, sa=BAD, sb=BAD, C=BAD, ct=0):
    return d.lib.fp8_gemm(A, fa, B, fb, M, N, K, sa, sb, C, ct, None)


def test_gemm_validation():
    import delayed_scaling_amax_amd as d
    assert _gemm(d, M=-1) == d.EINVAL and _gemm(d, N=-1) == d.EINVAL and _gemm(d, K=-16) == d.EINVAL
    assert _gemm(d, fa=2) == d.EINVAL and _gemm(d, fb=-1) == d.EINVAL
    assert _gemm(d, ct=2) == d.EINVAL
    assert _gemm(d, sa=None) == d.EINVAL and _gemm(d, sb=None) == d.EINVAL
    assert _gemm(d, C=None) == d.EINVAL
    assert _gemm(d, A=None) == d.EINVAL and _gemm(d, B=None) == d.EINVAL
    assert _gemm(d, K=24) == d.EUNSUPPORTED                    # K not a multiple of 16
    assert _gemm(d, K=(1 << 23) + 16) == d.EUNSUPPORTED
    assert _gemm(d, A=BAD + 8) == d.EUNSUPPORTED and _gemm(d, B=BAD + 4) == d.EUNSUPPORTED
    assert _gemm(d, C=BAD + 1, ct=0) == d.EINVAL              # bf16 C misaligned
    assert _gemm(d, C=BAD + 2, ct=1) == d.EINVAL              # fp32 C misaligned
    assert _gemm(d, A=None, B=None, C=None, M=0) == d.OK      # empty: nothing enqueued
    assert _gemm(d, A=None, B=None, C=None, N=0) == d.OK


def test_gelu_quantize_takes_bf16_only():
    import delayed_scaling_amax_amd as d
    assert d.lib.fp8_gelu_quantize_amax(BAD, d.F32, BAD, 10, 0, BAD, BAD, None) == d.EUNSUPPORTED
    assert d.lib.fp8_gelu_quantize_amax(None, d.F32, None, 0, 0, BAD, BAD, None) == d.EUNSUPPORTED
    assert d.lib.fp8_gelu_quantize_amax(None, d.BF16, None, 0, 1, BAD, BAD, None) == d.OK


def test_multi_rejects_before_enqueue():
    import delayed_scaling_amax_amd as d
    arr = (d.fp8q_tensor * 3)()
    # entries 0 and 1 would be valid zero-size no-ops; entry 2 is invalid -> EINVAL for all
    for i in range(3):
        arr[i] = d.fp8q_tensor(None, None, 0, 0, 0, BAD, BAD)
    arr[2].format = 9
    assert d.lib.fp8_multi_quantize_amax(arr, 3, None) == d.EINVAL
    assert d.lib.fp8_multi_quantize_amax(arr, -1, None) == d.EINVAL
    assert d.lib.fp8_multi_quantize_amax(None, 2, None) == d.EINVAL
    # the profiling form validates the same way (events untouched when it rejects)
    assert d.lib.fp8_multi_quantize_amax_timed(arr, 3, None, BAD, BAD) == d.EINVAL
    assert d.lib.fp8_multi_quantize_amax_timed(arr, -1, None, BAD, BAD) == d.EINVAL
    assert d.lib.fp8_multi_quantize_amax_timed(None, 2, None, BAD, BAD) == d.EINVAL


def test_zero_size_is_noop_without_device():
    import delayed_scaling_amax_amd as d
    arr = (d.fp8q_tensor * 2)()
    for i in range(2):
        arr[i] = d.fp8q_tensor(None, None, 0, 1, 1, BAD, BAD)
    assert d.lib.fp8_multi_quantize_amax(arr, 2, None) == d.OK
    assert d.lib.fp8_multi_quantize_amax(None, 0, None) == d.OK
    assert d.lib.fp8_multi_quantize_amax_timed(arr, 2, None, None, None) == d.OK
    assert d.lib.fp8_quantize_amax(None, 0, None, 0, 0, BAD, BAD, None) == d.OK
    assert d.lib.fp8_dequantize(None, 0, None, 1, 0, BAD, None) == d.OK
    assert d.lib.fp8_amax_and_scale_update(None, None, None, None, None, 0, 4, 0, 0, 0,
                                           None) == d.OK


@pytest.mark.parametrize("args", [
    (BAD, 0, BAD, 1, -1, BAD),    # negative numel
    (BAD, 3, BAD, 1, 10, BAD),    # bad format
    (BAD, 0, BAD, 5, 10, BAD),    # bad dst dtype
    (BAD, 0, BAD, 1, 10, None),   # NULL scale
    (None, 0, BAD, 1, 10, BAD),   # NULL src
])
def test_dequantize_rejects_invalid(args):
    import delayed_scaling_amax_amd as d
    assert d.lib.fp8_dequantize(*args, None) == d.EINVAL


@pytest.mark.parametrize("n,H,algo,margin,ptrs", [
    (-1, 4, 0, 0, 5), (4, 0, 0, 0, 5), (4, 4, 2, 0, 5), (4, 4, 0, 127, 5), (4, 4, 0, -127, 5),
    (4, 4, 0, 0, 4),
])
def test_update_rejects_invalid(n, H, algo, margin, ptrs):
    import delayed_scaling_amax_amd as d
    p = [BAD] * 5
    if ptrs < 5:
        p[ptrs] = None
    assert d.lib.fp8_amax_and_scale_update(*p, n, H, algo, margin, 0, None) == d.EINVAL


def test_update_refuses_histories_past_32bit_offsets():
    """history_len * n >= 2^29 (2 GiB of history): FP8Q_EUNSUPPORTED before anything is
    enqueued, from the update and from the one-launch step."""
    import delayed_scaling_amax_amd as d
    p = [BAD] * 5
    assert d.lib.fp8_amax_and_scale_update(*p, 1 << 10, 1 << 19, 0, 0, 0, None) == d.EUNSUPPORTED
    assert d.lib.fp8_amax_and_scale_update(*p, 1152, 466034, 0, 0, 0, None) == d.EUNSUPPORTED
    arr = (d.fp8q_tensor * 1)()
    arr[0] = d.fp8q_tensor(BAD, BAD, 1 << 20, 0, 0, BAD, BAD)
    assert _step(d, arr, 1, n=1 << 10, H=1 << 19) == d.EUNSUPPORTED


def _step(d, arr, nt, n=3, H=4, algo=0, margin=0, ws=BAD, ptrs=5):
    p = [BAD] * 5
    if ptrs < 5:
        p[ptrs] = None
    return d.lib.fp8_quantize_amax_and_update(arr, nt, *p, n, H, algo, margin, 1, ws, None,
                                              None, None)


def test_fused_step_rejects_before_enqueue():
    """Invalid entries, invalid update arguments or a NULL workspace: EINVAL with nothing
    enqueued (no device exists here, so any enqueue would fail as EHIP instead)."""
    import delayed_scaling_amax_amd as d
    arr = (d.fp8q_tensor * 2)()
    for i in range(2):
        arr[i] = d.fp8q_tensor(None, None, 0, 0, 0, BAD, BAD)
    bad = (d.fp8q_tensor * 2)()
    for i in range(2):
        bad[i] = d.fp8q_tensor(None, None, 0, 0, 0, BAD, BAD)
    bad[1].src_dtype = 7
    assert _step(d, bad, 2) == d.EINVAL               # invalid entry
    assert _step(d, arr, -1) == d.EINVAL              # negative tensor count
    assert _step(d, arr, 2, n=-1) == d.EINVAL         # negative update size
    assert _step(d, arr, 2, H=0) == d.EINVAL          # empty history
    assert _step(d, arr, 2, algo=5) == d.EINVAL       # unknown algo
    assert _step(d, arr, 2, margin=200) == d.EINVAL   # margin out of range
    assert _step(d, arr, 2, ptrs=2) == d.EINVAL       # NULL scale
    assert _step(d, arr, 2, ws=None) == d.EINVAL      # NULL workspace
    # empty tensors and an empty update: nothing to enqueue
    assert _step(d, arr, 2, n=0) == d.OK


def test_plan_layout_and_validation():
    """Plans: the descriptor is 128 bytes, the workspace 96 bytes per entry (rounded to
    16) plus 4 per full chunk; invalid lists,
    too many entries, a missing, misaligned or short workspace, or a descriptor no plan
    call filled are refused before anything is copied or launched."""
    import ctypes
    import delayed_scaling_amax_amd as d
    assert ctypes.sizeof(d.fp8q_plan) == 128
    plan = d.fp8q_plan()
    arr = (d.fp8q_tensor * 2049)()
    for i in range(2049):
        arr[i] = d.fp8q_tensor(None, None, 0, i % 2, i % 2, BAD, BAD)
    B = d.lib.fp8_multi_quantize_plan_bytes
    assert B(arr, 0) == 0
    assert B(arr, 3) == 3 * 96 + 0      # empty tensors: no chunks (288 is a multiple of 16)
    assert B(arr, 1) == 96
    assert B(arr, 2049) == d.EUNSUPPORTED
    # a bf16 tensor of 3 * 16384 + 5 elements at a 16-byte aligned address: 3 full chunks
    one = (d.fp8q_tensor * 1)()
    one[0] = d.fp8q_tensor(0x20000, 0x40000, 3 * 16384 + 5, 0, 0, BAD, BAD)
    assert B(one, 1) == 96 + 3 * 4
    one[0].src_dtype = 7
    assert B(one, 1) == d.EINVAL
    ws = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)
    P = d.lib.fp8_multi_quantize_plan
    assert P(arr, 2049, ws, 1 << 30, ctypes.byref(plan), None) == d.EUNSUPPORTED
    assert P(arr, 4, None, 1 << 20, ctypes.byref(plan), None) == d.EINVAL      # no workspace
    assert P(arr, 4, ws + 8, 1 << 20, ctypes.byref(plan), None) == d.EINVAL    # misaligned
    assert P(arr, 4, ws, 4 * 96 - 1, ctypes.byref(plan), None) == d.EINVAL     # too short
    assert P(arr, 4, ws, 4 * 96, None, None) == d.EINVAL                       # no descriptor
    assert P(arr, -1, ws, 1 << 20, ctypes.byref(plan), None) == d.EINVAL
    bad = (d.fp8q_tensor * 1)()
    bad[0] = d.fp8q_tensor(None, None, 5, 0, 0, BAD, BAD)                       # NULL src
    assert P(bad, 1, ws, 1 << 20, ctypes.byref(plan), None) == d.EINVAL
    bad[0] = d.fp8q_tensor(BAD, BAD, 5, 0, 9, BAD, BAD)                         # bad format
    assert P(bad, 1, ws, 1 << 20, ctypes.byref(plan), None) == d.EINVAL
    assert all(w == 0 for w in plan.opaque)                                     # untouched
    assert d.lib.fp8_multi_quantize_amax_planned(ctypes.byref(plan), None) == d.EINVAL
    assert d.lib.fp8_multi_quantize_amax_planned(None, None) == d.EINVAL
    # an empty list needs no workspace, copies nothing and launches nothing
    assert P(arr, 0, None, 0, ctypes.byref(plan), None) == d.OK
    assert d.lib.fp8_multi_quantize_amax_planned(ctypes.byref(plan), None) == d.OK


def test_noalloc_refuses_before_enqueue():
    """The allocation-free multi-tensor quantize: an invalid list (EINVAL), more than 2048
    entries or more than 2^18 full chunks (EUNSUPPORTED) are refused before anything is
    copied or launched; an empty list is a no-op."""
    import delayed_scaling_amax_amd as d
    N = d.lib.fp8_multi_quantize_amax_noalloc
    arr = (d.fp8q_tensor * 2049)()
    for i in range(2049):
        arr[i] = d.fp8q_tensor(None, None, 0, 0, 0, BAD, BAD)
    assert N(arr, 2049, None) == d.EUNSUPPORTED
    assert N(arr, 0, None) == d.OK
    big = (d.fp8q_tensor * 2)()
    # bf16 at 16-byte aligned addresses: (2^18 + 1) full chunks of 16384 elements
    big[0] = d.fp8q_tensor(0x100000, 0x200000, ((1 << 18) + 1) * 16384, 0, 0, BAD, BAD)
    big[1] = d.fp8q_tensor(None, None, 0, 0, 0, BAD, BAD)
    assert N(big, 2, None) == d.EUNSUPPORTED
    big[0].format = 5
    assert N(big, 2, None) == d.EINVAL
    assert N(None, 3, None) == d.EINVAL


def test_import_fails_loudly_without_the_library(tmp_path):
    """The package has no fallback: a copy of it without libfp8q.so refuses to import."""
    import shutil
    import sys
    import delayed_scaling_amax_amd as d
    pkg = tmp_path / "delayed_scaling_amax_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(os.path.dirname(d.__file__), "__init__.py"), pkg / "__init__.py")
    out = subprocess.run([sys.executable, "-c", "import delayed_scaling_amax_amd"],
                         capture_output=True, text=True, cwd=str(tmp_path),
                         env=dict(os.environ, PYTHONPATH=str(tmp_path)))
    assert out.returncode != 0
    assert "ImportError" in out.stderr and "libfp8q.so is not built" in out.stderr, out.stderr
