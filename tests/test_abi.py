"""Host-side tests of the C ABI: exports, workspace sizing, argument checks.

None of these launches a kernel: every call either only queries sizes or is
rejected by the host-side validation before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

from linear_cross_entropy_amd import _lib
from linear_cross_entropy_amd.build import LIB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "cce.h")).read()
    return sorted(set(re.findall(r"\b(cce_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "build libcce.so first"
    lib = ctypes.CDLL(LIB)
    names = _declared()
    assert "cce_forward" in names and "cce_backward" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_probe_library_exports_its_probes():
    """libcce_probe.so (device ceilings for the roofline; not on the loss path)
    is built beside libcce.so and exports the three probes bench.py calls."""
    from linear_cross_entropy_amd.build import PROBE_LIB
    assert os.path.exists(PROBE_LIB), "build libcce_probe.so first"
    lib = ctypes.CDLL(PROBE_LIB)
    for n in ("cce_probe_mfma", "cce_probe_lds", "cce_probe_stream"):
        assert hasattr(lib, n), n
    # nothing of the loss path lives there
    assert not hasattr(lib, "cce_forward")


def _ws(N, V, D):
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = _lib.load().cce_workspace_bytes(N, V, D, ctypes.byref(f), ctypes.byref(b))
    return rc, f.value, b.value


def test_workspace_never_scales_with_N_times_V():
    rc, f, b = _ws(8192, 256000, 2304)
    assert rc == 0
    logits_bytes = 8192 * 256000 * 4  # the fp32 logit matrix: 8000 MiB
    assert logits_bytes == 8000 * 2 ** 20
    # forward: O(N) partials plus the compacted copy of E (N x D bf16)
    assert f < 8 * 2 ** 20 + 8192 * 2304 * 2 + 8192 * 12
    # backward at the Gemma-2-2B head shape: two 8192-wide chunks of fp16
    # G-hat (256 MiB), E^T, two C^T chunks, the fp32 dE accumulator and the
    # compacted E: under 480 MiB, so that with the outputs (dE + dC in bf16,
    # the CCE blog post's lower bound "The memory numbers hold up") the peak
    # stays within 1.5 x that bound
    outputs = (8192 * 2304 + 256000 * 2304) * 2
    assert b < 480 * 2 ** 20
    assert max(f, b) + outputs < 1.5 * outputs
    # doubling V past the chunk size leaves the backward workspace unchanged
    # but for a few bytes per chunk; doubling N doubles it at most
    _, f2, b2 = _ws(8192, 512000, 2304)
    # only the per-chunk scale slots and the sorted backward's O(V) entry
    # positions grow with V
    assert 0 <= b2 - b <= 4 * 256000 + 4096
    _, f3, b3 = _ws(16384, 256000, 2304)
    assert b3 <= 2 * b + 4096
    # the forward's never depends on V beyond its O(N) slab partials
    assert f2 == f


def test_backward_workspace_of_a_long_batch_is_blocked_over_tokens():
    # Past 16,384 rows the backward takes the tokens in blocks of at most
    # 8,192: at the Llama-3 head shape with 65,536 tokens the workspace holds
    # G-hat for one block only (2 x 8192 x 8192 fp16 = 256 MiB, against 2 GiB
    # for every row), the fp32 dE accumulator (512 MiB), E^T and the
    # compacted E (256 MiB each), two C^T chunks and the chunk's fp32 dC
    # accumulator (64 MiB each): under 1.5 GiB
    rc, _, b = _ws(65536, 128256, 2048)
    assert rc == 0
    assert b < 1.5 * 2 ** 30
    assert b > (512 + 256 + 256 + 256 + 64 + 64) * 2 ** 20
    # up to 16,384 rows nothing is blocked: from there on the workspace grows
    # by the rows' O(N * D) parts only, not by G-hat's O(N * chunk)
    _, _, b16 = _ws(16384, 128256, 2048)
    _, _, b17 = _ws(16640, 128256, 2048)
    assert b17 < b16
    _, _, b32 = _ws(32768, 128256, 2048)
    assert b32 - b16 < 16384 * (2048 * (4 + 2 + 2) + 64)


def test_rejects_bad_arguments_before_launch():
    lib = _lib.load()
    vp = ctypes.c_void_p
    fake = vp(0x1000)  # never dereferenced: validation fails first
    ws = vp(0x2000)
    # bad shapes
    assert _ws(-1, 10, 8)[0] == 2
    assert _ws(4, 0, 8)[0] == 2
    assert _ws(4, 10, 12)[0] == 2
    # null pointers
    rc = lib.cce_forward(vp(0), fake, fake, 4, 10, 8, -100, 1, fake, fake, ws, 1 << 20, vp(0))
    assert rc == 1
    # bad reduction
    rc = lib.cce_forward(fake, fake, fake, 4, 10, 8, -100, 7, fake, fake, ws, 1 << 20, vp(0))
    assert rc == 3
    # misaligned
    rc = lib.cce_forward(vp(0x1002), fake, fake, 4, 10, 8, -100, 1, fake, fake, ws, 1 << 20, vp(0))
    assert rc == 4
    # workspace too small
    rc = lib.cce_forward(fake, fake, fake, 4, 10, 8, -100, 1, fake, fake, ws, 8, vp(0))
    assert rc == 6
    # bad eps
    for eps in (-1.0, float("nan"), float("inf")):
        rc = lib.cce_backward(fake, fake, fake, fake, fake, 4, 10, 8, -100, 1, eps, fake, fake,
                              vp(0), ws, 1 << 30, vp(0))
        assert rc == 5
    # bad filter mode (cce_backward_ex): rejected before anything is enqueued
    for mode in (-1, 3):
        rc = lib.cce_backward_ex(fake, fake, fake, fake, fake, 4, 10, 8, -100, 1, 2.0 ** -12,
                                 mode, fake, fake, vp(0), ws, 1 << 30, vp(0))
        assert rc == 8
    # vocabulary order and the sorted backward: null order, misaligned order,
    # bad shape, a C too large for 32-bit row offsets, small workspace
    rc = lib.cce_vocab_order(fake, fake, fake, 4, 10, 8, -100, vp(0), ws, 1 << 30, vp(0))
    assert rc == 1
    rc = lib.cce_vocab_order(fake, fake, fake, 4, 10, 8, -100, vp(0x1002), ws, 1 << 30, vp(0))
    assert rc == 4
    rc = lib.cce_vocab_order(fake, fake, fake, 4, 10, 12, -100, fake, ws, 1 << 30, vp(0))
    assert rc == 2
    rc = lib.cce_vocab_order(fake, fake, fake, 4, 10, 8, -100, fake, ws, 8, vp(0))
    assert rc == 6
    rc = lib.cce_backward_sorted(fake, fake, fake, fake, fake, 4, 10, 8, -100, 1, 2.0 ** -12, 0,
                                 vp(0), fake, fake, vp(0), ws, 1 << 30, vp(0))
    assert rc == 1
    rc = lib.cce_backward_sorted(fake, fake, fake, fake, fake, 4, 10, 8, -100, 1, 2.0 ** -12, 0,
                                 vp(0x1002), fake, fake, vp(0), ws, 1 << 30, vp(0))
    assert rc == 4
    rc = lib.cce_backward_sorted(fake, fake, fake, fake, fake, 4, 262144, 4096, -100, 1,
                                 2.0 ** -12, 0, fake, fake, fake, vp(0), ws, 1 << 30, vp(0))
    assert rc == 2
    rc = lib.cce_backward_sorted(fake, fake, fake, fake, fake, 4, 10, 8, -100, 1, 2.0 ** -12, 5,
                                 fake, fake, fake, vp(0), ws, 1 << 30, vp(0))
    assert rc == 8
    assert lib.cce_status_string(8).decode().startswith("filter_mode")
    assert lib.cce_status_string(6).decode().startswith("workspace")


def test_python_wrapper_rejects_bad_dtypes():
    import torch
    import linear_cross_entropy_amd as lce
    E = torch.zeros(4, 8)
    C = torch.zeros(10, 8, dtype=torch.bfloat16)
    x = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(TypeError):
        lce.cce_forward(E, C, x)
    with pytest.raises(ValueError):
        lce.linear_cross_entropy(E.bfloat16(), C, x, reduction="avg")
    with pytest.raises(ValueError):
        lce.linear_cross_entropy(E.bfloat16(), C, x, filter_mode="kahan")
    with pytest.raises(ValueError):  # host tensors: rejected before any call
        lce.cce_vocab_order(E.bfloat16(), C, x)


def test_bench_runs_on_one_gpu_only():
    """bench.py --gpus N with N > 1 exits with a message before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
