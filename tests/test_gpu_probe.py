"""The device-ceiling probes (libcce_probe.so, bench.py --hw-probe and the
measured MFMA peak of every bench line) return success and rates inside what
an MI355X can physically do: bf16 MFMA below the 2.5 PFLOP/s spec, loads from
L2 above loads from past it, past-L2 loads below the 8 TB/s HBM spec plus
the memory-side cache's share."""
import pytest

pytestmark = pytest.mark.gpu


def _lib():
    import torch
    torch.cuda.init()
    import bench
    lib = bench._probe_lib()
    assert lib is not None, "libcce_probe.so is not built"
    return bench, lib


def test_mfma_probe_rate_is_physical():
    bench, lib = _lib()
    ms, flops = bench._probe_call(lib.cce_probe_mfma, 0)
    rate = flops / (ms * 1e-3) / 1e12
    assert 500.0 < rate < 2600.0, rate
    ms0, flops0 = bench._probe_call(lib.cce_probe_mfma, 1)
    assert flops0 == flops


def test_lds_probe_rate_is_physical():
    bench, lib = _lib()
    ms, b = bench._probe_call(lib.cce_probe_lds)
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_cu = b / (ms * 1e-3) / cus
    # at most 256 bytes per clock per CU at 2.4 GHz
    assert 50e9 < per_cu < 256 * 2.4e9, per_cu


def test_stream_probe_l2_beats_past_l2():
    bench, lib = _lib()
    ms_l2, b_l2 = bench._probe_call(lib.cce_probe_stream, 1 << 20, 1, 1)
    ms_far, b_far = bench._probe_call(lib.cce_probe_stream, 4 << 20, 0, 1)
    l2 = b_l2 / (ms_l2 * 1e-3)
    far = b_far / (ms_far * 1e-3)
    assert l2 > 1.5 * far, (l2, far)
    assert 1e12 < far < 20e12, far


def test_stream_probe_rejects_bad_windows():
    import ctypes
    bench, lib = _lib()
    ms, b = ctypes.c_float(), ctypes.c_double()
    for win in (0, 1000, 16384 + 8, 32 << 20):
        assert lib.cce_probe_stream(win, 1, 1, ctypes.byref(ms), ctypes.byref(b)) != 0, win
