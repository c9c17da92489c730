"""Cut Cross-Entropy on MI355X: Python binding of libcce.so.

Argument marshalling only: every step of the loss and its gradient runs in
the HIP kernels of ``csrc/cce.hip`` behind the C ABI of ``include/cce.h``.
PyTorch supplies device memory and the current stream.

    loss = linear_cross_entropy(E, C, x)          # E [N,D] bf16, C [V,D] bf16, x [N] int64
    loss.backward()                                # dE, dC land in .grad

The call shape and the gradient landing in the classifier's ``.grad`` follow
the kernel card "cut-cross-entropy" (Usage); ``ignore_index`` and the three
reductions follow its Correctness section; ``filter_eps`` = 2**-12 is the
threshold of the CCE blog post ("Gradient filtering") and the "Cut Your
Losses" digest ("Gradient Filtering").  ``filter_mode`` picks the
contractions that take the filtered gradient (digest, "Numerical Stability
Variants"): "both" (basic CCE), "full_c" (dC unfiltered, the digest's
pretraining recommendation) or "full_e" (dE unfiltered).  ``vocab_sort``
(digest, "Vocabulary Sorting") takes the backward's vocabulary in the order
of descending average logit, from ``cce_vocab_order``.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import CCEError, FilterStats  # noqa: F401

__all__ = [
    "linear_cross_entropy", "cce_forward", "cce_forward_noalloc", "cce_backward", "cce_vocab_order",
    "cce_workspace_bytes",
    "profile_enable", "profile_query", "CCEError", "DEFAULT_FILTER_EPS", "FILTER_MODES",
]

DEFAULT_FILTER_EPS = 2.0 ** -12
REDUCTIONS = {"none": 0, "mean": 1, "sum": 2}
FILTER_MODES = {"both": 0, "full_c": 1, "full_e": 2}  # cce_filter_mode


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def cce_workspace_bytes(N: int, V: int, D: int):
    """(forward bytes, backward bytes) of workspace for these sizes."""
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _lib.check(_lib.load().cce_workspace_bytes(N, V, D, ctypes.byref(f), ctypes.byref(b)),
               "cce_workspace_bytes")
    return f.value, b.value


def _check_inputs(E, C, x):
    if E.dtype != torch.bfloat16 or C.dtype != torch.bfloat16:
        raise TypeError("E and C must be bfloat16")
    if x.dtype != torch.int64:
        raise TypeError("targets must be int64")
    if E.dim() != 2 or C.dim() != 2 or x.dim() != 1:
        raise ValueError("expected E [N, D], C [V, D], x [N]")
    if E.shape[1] != C.shape[1] or E.shape[0] != x.shape[0]:
        raise ValueError(f"shape mismatch: E {tuple(E.shape)}, C {tuple(C.shape)}, x {tuple(x.shape)}")
    if not (E.is_cuda and C.is_cuda and x.is_cuda):
        raise ValueError("E, C and x must be device tensors")
    return E.contiguous(), C.contiguous(), x.contiguous()


def cce_forward(E, C, x, ignore_index: int = -100, reduction: str = "mean", workspace=None):
    """Returns (loss, lse): loss is [N] for 'none', a 0-d tensor otherwise; lse is [N] fp32."""
    E, C, x = _check_inputs(E, C, x)
    N, D = E.shape
    V = C.shape[0]
    red = REDUCTIONS[reduction]
    dev = E.device
    loss = torch.empty((N,) if red == 0 else (1,), dtype=torch.float32, device=dev)
    lse = torch.empty((N,), dtype=torch.float32, device=dev)
    fb, _ = cce_workspace_bytes(N, V, D)
    ws = workspace if workspace is not None else torch.empty(max(fb, 256), dtype=torch.uint8, device=dev)
    rc = _lib.load().cce_forward(_ptr(E), _ptr(C), _ptr(x), N, V, D, ignore_index, red,
                                 _ptr(loss), _ptr(lse), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(rc, "cce_forward")
    return (loss if red == 0 else loss.reshape(())), lse


def cce_forward_noalloc(E, C, x, ignore_index: int = -100, reduction: str = "mean", loss=None,
                        lse=None):
    """cce_forward without a workspace (the library's static per-GPU scratch):
    for callers that cannot allocate.  loss / lse may be passed in (then this
    call allocates nothing either); returns (loss, lse) as cce_forward does."""
    E, C, x = _check_inputs(E, C, x)
    N, D = E.shape
    V = C.shape[0]
    red = REDUCTIONS[reduction]
    dev = E.device
    if loss is None:
        loss = torch.empty((N,) if red == 0 else (1,), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((N,), dtype=torch.float32, device=dev)
    if loss.numel() != (N if red == 0 else 1) or lse.numel() != N:
        raise ValueError("loss must hold N values for 'none' (else 1), lse N values")
    rc = _lib.load().cce_forward_noalloc(_ptr(E), _ptr(C), _ptr(x), N, V, D, ignore_index, red,
                                         _ptr(loss), _ptr(lse), _stream(dev))
    _lib.check(rc, "cce_forward_noalloc")
    return (loss if red == 0 else loss.reshape(())), lse


def cce_vocab_order(E, C, x, ignore_index: int = -100, workspace=None):
    """Vocabulary ids by descending average logit over the valid rows, equal
    averages by id: int32 [V] on the device (cce_vocab_order)."""
    E, C, x = _check_inputs(E, C, x)
    N, D = E.shape
    V = C.shape[0]
    dev = E.device
    order = torch.empty((V,), dtype=torch.int32, device=dev)
    _, bb = cce_workspace_bytes(N, V, D)
    ws = workspace if workspace is not None else torch.empty(max(bb, 256), dtype=torch.uint8, device=dev)
    rc = _lib.load().cce_vocab_order(_ptr(E), _ptr(C), _ptr(x), N, V, D, ignore_index, _ptr(order),
                                     _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(rc, "cce_vocab_order")
    return order


def cce_backward(E, C, x, lse, grad, ignore_index: int = -100, reduction: str = "mean",
                 filter_eps: float = DEFAULT_FILTER_EPS, with_stats: bool = False, workspace=None,
                 filter_mode: str = "both", vocab_order=None):
    """Returns (dE bf16 [N,D], dC bf16 [V,D]) and, if with_stats, a dict of filter counts.
    filter_mode "both" calls cce_backward, "full_c" / "full_e" cce_backward_ex;
    a vocab_order (int32 [V] device permutation) calls cce_backward_sorted."""
    if filter_mode not in FILTER_MODES:
        raise ValueError(f"filter_mode must be one of {sorted(FILTER_MODES)}")
    E, C, x = _check_inputs(E, C, x)
    N, D = E.shape
    V = C.shape[0]
    red = REDUCTIONS[reduction]
    dev = E.device
    g = grad.to(device=dev, dtype=torch.float32).contiguous().reshape(-1)
    if red == 0 and g.numel() != N:
        raise ValueError("reduction 'none' takes an upstream gradient of shape [N]")
    if red != 0 and g.numel() != 1:
        raise ValueError("mean/sum take a scalar upstream gradient")
    dE = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    dC = torch.empty((V, D), dtype=torch.bfloat16, device=dev)
    _, bb = cce_workspace_bytes(N, V, D)
    ws = workspace if workspace is not None else torch.empty(max(bb, 256), dtype=torch.uint8, device=dev)
    st = torch.zeros(3, dtype=torch.int64, device=dev) if with_stats else None
    lib = _lib.load()
    args = (_ptr(E), _ptr(C), _ptr(x), _ptr(lse.contiguous()), _ptr(g), N, V, D, ignore_index,
            red, float(filter_eps))
    outs = (_ptr(dE), _ptr(dC), _ptr(st), _ptr(ws), ws.numel(), _stream(dev))
    if vocab_order is not None:
        if vocab_order.dtype != torch.int32 or vocab_order.shape != (V,) or not vocab_order.is_cuda:
            raise ValueError("vocab_order must be an int32 device tensor of shape [V]")
        vo = vocab_order.contiguous()
        rc = lib.cce_backward_sorted(*args, FILTER_MODES[filter_mode], _ptr(vo), *outs)
        _lib.check(rc, "cce_backward_sorted")
    elif filter_mode == "both":
        rc = lib.cce_backward(*args, *outs)
        _lib.check(rc, "cce_backward")
    else:
        rc = lib.cce_backward_ex(*args, FILTER_MODES[filter_mode], *outs)
        _lib.check(rc, "cce_backward_ex")
    if not with_stats:
        return dE, dC
    h = st.cpu()
    packed = int(h[2])
    stats = {"units_total": int(h[0]), "units_skipped": int(h[1]),
             "unit_rows": packed & 0xFFFFFFFF, "unit_cols": (packed >> 32) & 0xFFFFFFFF}
    return dE, dC, stats


class _CCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, E, C, x, ignore_index, reduction, filter_eps, filter_mode, vocab_sort):
        loss, lse = cce_forward(E, C, x, ignore_index, reduction)
        # the order comes from the same forward inputs, as the digest gathers
        # its averages in the forward pass
        order = cce_vocab_order(E, C, x, ignore_index) if vocab_sort else None
        ctx.save_for_backward(E, C, x, lse, order)
        ctx.cfg = (ignore_index, reduction, filter_eps, filter_mode)
        return loss

    @staticmethod
    def backward(ctx, grad):
        E, C, x, lse, order = ctx.saved_tensors
        ignore_index, reduction, filter_eps, filter_mode = ctx.cfg
        dE, dC = cce_backward(E, C, x, lse, grad, ignore_index, reduction, filter_eps,
                              filter_mode=filter_mode, vocab_order=order)
        return dE, dC, None, None, None, None, None, None


def linear_cross_entropy(E, C, x, ignore_index: int = -100, reduction: str = "mean",
                         filter_eps: float = DEFAULT_FILTER_EPS, filter_mode: str = "both",
                         vocab_sort: bool = False):
    """Cross-entropy of softmax(E C^T) against targets x without forming the logits."""
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    if filter_mode not in FILTER_MODES:
        raise ValueError(f"filter_mode must be one of {sorted(FILTER_MODES)}")
    return _CCE.apply(E, C, x, ignore_index, reduction, filter_eps, filter_mode, bool(vocab_sort))


def profile_enable(on: bool = True, roles: bool = False):
    """Start (clearing) or stop per-kernel timing; roles=True also runs each role
    of the backward step in a launch of its own ("bwd_de", "bwd_dc", "bwd_g",
    "bwd_t")."""
    _lib.check(_lib.load().cce_profile_enable((2 if roles else 1) if on else 0),
               "cce_profile_enable")


def profile_query(name: str):
    """(launches, total milliseconds) recorded for a kernel family since profile_enable."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _lib.check(_lib.load().cce_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)),
               "cce_profile_query")
    return n.value, ms.value
