"""The forward entry point that allocates nothing (cce_forward_noalloc, for
callers that cannot allocate) against cce_forward, through the C ABI: two calls
in a row on one GPU, the second with a smaller input, each bit for bit equal
to cce_forward on the same inputs (the same kernels and launch plan, with the
workspace in the library's static per-GPU scratch); a shape whose forward
workspace exceeds the scratch is rejected before anything is enqueued."""
import ctypes

import pytest
import torch

import synthetic_inputs as si
from linear_cross_entropy_amd import _lib

pytestmark = pytest.mark.gpu

IGN = -100
DEV = "cuda:0"
RED = {"none": 0, "mean": 1, "sum": 2}


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)


def _both(w):
    lib = _lib.load()
    E, C, x = (t.to(DEV) for t in si.generate(w))
    N, D = E.shape
    V = C.shape[0]
    red = RED[w.reduction]
    nl = N if red == 0 else 1
    f = ctypes.c_size_t(0)
    assert lib.cce_workspace_bytes(N, V, D, ctypes.byref(f), None) == 0
    ws = torch.empty(f.value, dtype=torch.uint8, device=DEV)
    outs = {}
    for name in ("ws", "noalloc"):
        loss = torch.full((nl,), float("nan"), device=DEV)
        lse = torch.full((N,), float("nan"), device=DEV)
        if name == "ws":
            rc = lib.cce_forward(_p(E), _p(C), _p(x), N, V, D, IGN, red, _p(loss), _p(lse), _p(ws),
                                 ws.numel(), _stream())
        else:
            rc = lib.cce_forward_noalloc(_p(E), _p(C), _p(x), N, V, D, IGN, red, _p(loss), _p(lse),
                                         _stream())
        assert rc == 0, (name, rc)
        outs[name] = (loss, lse)
    torch.cuda.synchronize()
    return outs


def test_forward_noalloc_matches_forward_twice_then_smaller():
    big = si.GEMMA  # 8192 x 2304 tokens, 256,000 entries: about 37 MiB of scratch
    small = si.Workload("noalloc-small", 700, 9001, 136, logit_std=3.0, ignore_rows=40,
                        tail_targets=8, tail_width=200, reduction="none", seed=61)
    for w in (big, small):
        o = _both(w)
        for a, b in zip(o["ws"], o["noalloc"]):
            assert torch.equal(a, b), w.name
        assert not torch.isnan(o["noalloc"][1]).any()


@pytest.mark.parametrize("N,V,D", [(65536, 128256, 2048),   # 256 MiB for the copy of E alone
                                    (16384, 201088, 2880)])  # about 91 MiB
def test_forward_noalloc_rejects_shapes_beyond_the_scratch(N, V, D):
    lib = _lib.load()
    f = ctypes.c_size_t(0)
    assert lib.cce_workspace_bytes(N, V, D, ctypes.byref(f), None) == 0
    assert f.value > 64 << 20  # CCE_NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    fake = vp(0x1000)  # never dereferenced: the check comes first
    rc = lib.cce_forward_noalloc(fake, fake, fake, N, V, D, IGN, 1, fake, fake, vp(0))
    assert rc == 9 and lib.cce_status_string(rc).decode().startswith("the forward's workspace")
