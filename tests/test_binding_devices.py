"""The Python binding rejects tensors that are not on the call's GPU before it calls
into the library: a host pointer handed to a kernel would fault the GPU instead of
raising.  Runs without a GPU: the library object is replaced by a recorder, so any call
that got past the checks would show up as a recorded call."""
import pytest
import torch

import delayed_scaling_amax_amd as d


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*a):
            self.calls.append(name)
            return 0
        return f


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(d, "lib", r)
    return r


def _cpu(n, dtype=torch.float32):
    return torch.zeros(n, dtype=dtype)


CASES = {
    "quantize": lambda: d.fp8_quantize_amax(_cpu(16, torch.bfloat16), _cpu(16, torch.uint8),
                                            _cpu(1), _cpu(1), d.E4M3),
    "gelu": lambda: d.fp8_gelu_quantize_amax(_cpu(16, torch.bfloat16), _cpu(16, torch.uint8),
                                             _cpu(1), _cpu(1), d.E4M3),
    "layernorm": lambda: d.fp8_layernorm_quantize_amax(
        _cpu(64, torch.bfloat16).view(8, 8), _cpu(64, torch.uint8), _cpu(1), _cpu(1), d.E4M3),
    "multi": lambda: d.fp8_multi_quantize_amax(
        [(_cpu(16, torch.bfloat16), _cpu(16, torch.uint8), _cpu(1), _cpu(1), d.E4M3)]),
    "multi_timed": lambda: d.fp8_multi_quantize_amax_timed(
        [(_cpu(16, torch.bfloat16), _cpu(16, torch.uint8), _cpu(1), _cpu(1), d.E4M3)],
        None, None),
    "plan": lambda: d.fp8_multi_quantize_plan(
        [(_cpu(16, torch.bfloat16), _cpu(16, torch.uint8), _cpu(1), _cpu(1), d.E4M3)]),
    "dequantize": lambda: d.fp8_dequantize(_cpu(16, torch.uint8), _cpu(16), _cpu(1), d.E4M3),
    "gemm": lambda: d.fp8_gemm(_cpu(256, torch.uint8).view(16, 16), d.E4M3,
                               _cpu(256, torch.uint8).view(16, 16), d.E4M3, _cpu(1), _cpu(1),
                               _cpu(256, torch.bfloat16).view(16, 16)),
    "update": lambda: d.fp8_amax_and_scale_update(_cpu(3), _cpu(48).view(16, 3), _cpu(3),
                                                  _cpu(3), _cpu(3, torch.uint8)),
    "step": lambda: d.fp8_quantize_amax_and_update(
        [(_cpu(16, torch.bfloat16), _cpu(16, torch.uint8), _cpu(1), _cpu(1), d.E4M3)],
        _cpu(1), _cpu(16).view(16, 1), _cpu(1), _cpu(1), _cpu(1, torch.uint8),
        _cpu(1, torch.int32)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_host_tensors_rejected_before_the_library(rec, case):
    with pytest.raises(ValueError, match="GPU tensor"):
        CASES[case]()
    assert rec.calls == []


def test_mixed_devices_rejected(rec, monkeypatch):
    """A host tensor among GPU ones is caught too: the first tensor fixes the device and
    every other one is compared with it (checked here with a stand-in for a GPU tensor,
    since this machine has none)."""
    class FakeCuda(torch.Tensor):
        @property
        def is_cuda(self):
            return True

        @property
        def device(self):
            return torch.device("cuda", 0)

    src = torch.zeros(16, dtype=torch.bfloat16).as_subclass(FakeCuda)
    with pytest.raises(ValueError, match="dst must be a GPU tensor"):
        d.fp8_quantize_amax(src, _cpu(16, torch.uint8), _cpu(1), _cpu(1), d.E4M3)
    assert rec.calls == []
