"""fp64 CPU oracle for Cut Cross-Entropy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP path in
``linear_cross_entropy_amd`` and neither imports the other.

The arithmetic lives in ``cce_oracle.c`` (plain C, double precision, OpenMP);
this file only compiles it with gcc and marshals numpy arrays through ctypes.
What each function computes, with the passages it follows:

* ``forward``  -- lse, per-row loss = lse - target logit, and the none / mean /
  sum reductions with ignore_index rows contributing nothing ("Cut Your Losses"
  digest, "The Mathematical Decomposition" and Algorithm 2; kernel card
  "cut-cross-entropy", "Correctness").
* ``grad_logits`` -- G = softmax - onehot(x), 0 on ignored rows (CCE blog post,
  "Gradient filtering"; digest, Algorithm 4; the sign is that of the gradient
  of the loss, see the readings in the design notes).
* ``backward`` -- dE = diag(s) G C and dC = G^T diag(s) E with the tile filter
  (digest, Algorithms 3 and 4 and "Gradient Filtering"), applied to both
  contractions or, as in the FullC / FullE variants (digest, "Numerical
  Stability Variants"), to dE only or dC only; by default the ignored rows
  are removed before the filter units are cut (digest, Table A1).
* ``average_logits`` / ``vocab_order`` -- each vocabulary entry's logit summed
  over the valid rows and divided by their count, and the vocabulary ids by
  descending average, ties by ascending id (digest, "Vocabulary Sorting").
* ``backward(..., vocab_order=...)`` -- the same backward with the vocabulary
  taken in that order (digest, "Vocabulary Sorting": the filter units are cut
  from the reordered vocabulary); dC is returned in the original row order.
* ``dC_columns`` -- the same dC restricted to chosen 32-wide vocabulary blocks,
  given the lse that ``forward`` returned: plain numpy fp64 over all rows of
  those columns, for checking dC at sizes where the full backward would take
  too long.  Pinned to ``backward`` on small inputs.

Parity unpinned: none (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cce_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

REDUCTIONS = {"none": 0, "mean": 1, "sum": 2}
# which contractions take the filtered G ("Cut Your Losses" digest,
# "Numerical Stability Variants"): both, dE only (FullC: dC unfiltered) or
# dC only (FullE: dE unfiltered)
FILTER_MODES = {"both": 0, "full_c": 1, "full_e": 2}

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = [
        "gcc", "-O3", "-march=x86-64-v2", "-fopenmp", "-fPIC", "-shared",
        "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.oracle_forward.argtypes = [dp, dp, ip, i64, i64, i64, i64,
                                       ctypes.c_int, dp, dp, ip]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_grad_logits.argtypes = [dp, dp, ip, i64, i64, i64, i64, dp]
        lib.oracle_grad_logits.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [dp, dp, ip, i64, i64, i64, i64,
                                        ctypes.c_int, dp, ctypes.c_double,
                                        ctypes.c_int, ctypes.c_int, i64, i64, dp, dp, ip, ip]
        lib.oracle_backward.restype = ctypes.c_int
        _lib = lib
        return lib


def _f64(a):
    a = np.asarray(a)
    if hasattr(a, "dtype") and a.dtype != np.float64:
        a = a.astype(np.float64)
    return np.ascontiguousarray(a)


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _p(a, t=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(t))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def forward(E, C, x, ignore_index=-100, reduction="mean"):
    """Returns (loss, lse, n_valid); loss is shape [N] for 'none', a float otherwise."""
    E, C, x = _f64(E), _f64(C), _i64(x)
    N, D = E.shape
    V = C.shape[0]
    assert C.shape[1] == D and x.shape == (N,)
    red = REDUCTIONS[reduction]
    loss = np.zeros(max(N, 1) if red == 0 else 1, dtype=np.float64)
    lse = np.zeros(max(N, 1), dtype=np.float64)
    nv = np.zeros(1, dtype=np.int64)
    rc = _load().oracle_forward(_p(E), _p(C), _p(x, ctypes.c_int64), N, V, D,
                                ignore_index, red, _p(loss), _p(lse),
                                _p(nv, ctypes.c_int64))
    _check(rc, "forward")
    if red == 0:
        return loss[:N], lse[:N], int(nv[0])
    return float(loss[0]), lse[:N], int(nv[0])


def grad_logits(E, C, x, ignore_index=-100):
    """G = softmax(E C^T) - onehot(x) per valid row, zero rows where ignored."""
    E, C, x = _f64(E), _f64(C), _i64(x)
    N, D = E.shape
    V = C.shape[0]
    G = np.zeros((max(N, 1), V), dtype=np.float64)
    rc = _load().oracle_grad_logits(_p(E), _p(C), _p(x, ctypes.c_int64), N, V,
                                    D, ignore_index, _p(G))
    _check(rc, "grad_logits")
    return G[:N]


def _valid_rows(x, V, ignore_index):
    # rows that take part: not ignored and with a target inside the vocabulary
    return (x != ignore_index) & (x >= 0) & (x < V)


def average_logits(E, C, x, ignore_index=-100, row_chunk=256):
    """a[v] = (1/N_v) sum over valid rows n of C[v] . E[n], the logit of entry v
    averaged over the tokens ("Cut Your Losses" digest, "Vocabulary Sorting":
    per entry the sum and the count of the logits the forward pass sees,
    divided).  Rows that are ignored or whose target is outside [0, V) do not
    count; with no valid row every average is 0."""
    E, C, x = _f64(E), _f64(C), _i64(x)
    V = C.shape[0]
    rows = np.nonzero(_valid_rows(x, V, ignore_index))[0]
    total = np.zeros(V, dtype=np.float64)
    for r0 in range(0, rows.size, row_chunk):
        total += (E[rows[r0:r0 + row_chunk]] @ C.T).sum(axis=0)
    return total / rows.size if rows.size else total


def vocab_order(E, C, x, ignore_index=-100):
    """(order, averages): order lists the vocabulary ids by descending average
    logit, equal averages by ascending id (digest, "Vocabulary Sorting")."""
    a = average_logits(E, C, x, ignore_index)
    return np.argsort(-a, kind="stable"), a


def _check_order(order, V):
    order = np.asarray(order, dtype=np.int64)
    assert order.shape == (V,) and np.array_equal(np.sort(order), np.arange(V)), \
        "vocab_order must be a permutation of 0 .. V-1"
    return order


def backward(E, C, x, grad, ignore_index=-100, reduction="mean", eps=0.0,
             unit_rows=32, unit_cols=32, filter_mode="both", compact=True, vocab_order=None):
    """Returns (dE, dC, units_total, units_skipped) in float64.  filter_mode
    ("both", "full_c", "full_e") names the contractions that take the
    filtered G; units_skipped counts the units filtered out of them.  With
    compact (the default) the ignored rows are removed before the filter
    units are cut ("Cut Your Losses" digest, Table A1: ignored tokens dropped
    ahead of the loss), so a unit is unit_rows consecutive valid rows.
    vocab_order (a permutation of the vocabulary ids) reorders the vocabulary
    first (digest, "Vocabulary Sorting"): position i holds entry
    vocab_order[i], targets follow their entry, the filter units are cut
    along the new order, and dC comes back in the original row order."""
    E, C, x = _f64(E), _f64(C), _i64(x)
    N, D = E.shape
    V = C.shape[0]
    if vocab_order is not None:
        order = _check_order(vocab_order, V)
        pos = np.empty(V, dtype=np.int64)
        pos[order] = np.arange(V)
        ok = (x >= 0) & (x < V)
        xs = np.where(ok, pos[np.where(ok, x, 0)], x)  # ignored / out-of-range rows as they were
        dE, dCs, tot, skp = backward(E, C[order], xs, grad, ignore_index, reduction, eps,
                                     unit_rows, unit_cols, filter_mode, compact)
        dC = np.empty_like(dCs)
        dC[order] = dCs
        return dE, dC, tot, skp
    red = REDUCTIONS[reduction]
    g = _f64(np.atleast_1d(grad))
    if red == 0:
        assert g.shape == (N,), "reduction 'none' takes one upstream value per row"
    if g.size == 0:
        g = np.zeros(1)
    dE = np.zeros((max(N, 1), D), dtype=np.float64)
    dC = np.zeros((V, D), dtype=np.float64)
    tot = np.zeros(1, dtype=np.int64)
    skp = np.zeros(1, dtype=np.int64)
    rc = _load().oracle_backward(_p(E), _p(C), _p(x, ctypes.c_int64), N, V, D,
                                 ignore_index, red, _p(g), float(eps),
                                 FILTER_MODES[filter_mode], int(bool(compact)), unit_rows, unit_cols,
                                 _p(dE), _p(dC),
                                 _p(tot, ctypes.c_int64), _p(skp, ctypes.c_int64))
    _check(rc, "backward")
    return dE[:N], dC, int(tot[0]), int(skp[0])


def dC_columns(E, C, x, lse, grad, ignore_index=-100, reduction="mean", eps=0.0,
               blocks=(), unit_rows=32, unit_cols=32, compact=True, vocab_order=None):
    """dC rows of whole vocabulary blocks [unit_cols*b, unit_cols*(b+1)), from
    G = exp(E C_b^T - lse) - onehot(x) on every row (digest, "The Mathematical
    Decomposition" and Algorithm 4), the unit filter of "Gradient Filtering"
    applied per (unit_rows x unit_cols) block of that G (the row blocks cut
    from the valid rows only when compact, as in ``backward``), then
    dC_b = G_b^T diag(s) E.  `lse` must come from ``forward`` on the same
    inputs.  With vocab_order, block b holds the entries vocab_order[v0:v1]
    (as in ``backward``) and its rows are theirs, in that order.  Returns
    {b: array [rows of block b, D]} in float64."""
    E, C, x = _f64(E), _f64(C), _i64(x)
    lse = _f64(lse)
    N, D = E.shape
    V = C.shape[0]
    valid = x != ignore_index
    nv = int(valid.sum())
    g = _f64(np.atleast_1d(grad))
    if reduction == "mean":
        s = np.where(valid, g[0] / max(nv, 1), 0.0)
    elif reduction == "sum":
        s = np.where(valid, g[0], 0.0)
    else:
        assert g.shape == (N,), "reduction 'none' takes one upstream value per row"
        s = np.where(valid, g, 0.0)
    out = {}
    for b in blocks:
        v0 = int(b) * unit_cols
        v1 = min(V, v0 + unit_cols)
        assert 0 <= v0 < V, "block outside the vocabulary"
        cols = np.arange(v0, v1) if vocab_order is None else _check_order(vocab_order, V)[v0:v1]
        A = E @ C[cols].T
        G = np.exp(A - np.where(valid, lse, 0.0)[:, None])
        G -= (x[:, None] == cols[None, :]).astype(np.float64)
        G[~valid] = 0.0
        rows = np.nonzero(valid)[0] if compact else np.arange(N)
        Gr = G[rows]
        if eps > 0.0:
            for r0 in range(0, rows.size, unit_rows):
                unit = Gr[r0:r0 + unit_rows]
                if unit.size and np.max(np.abs(unit)) < eps:
                    unit[:] = 0.0
        out[int(b)] = (s[rows, None] * Gr).T @ E[rows]
    return out

