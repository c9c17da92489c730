"""fp64 CPU oracle for Cut Cross-Entropy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP path in
``linear_cross_entropy_amd`` and neither imports the other.

The plain arithmetic lives in ``cce_oracle.c`` (plain C, double precision,
OpenMP), which this file compiles with gcc and calls through ctypes; the
blocked versions below take the same steps with fp64 matrix products.  What
each function computes, with the passages it follows:

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
* ``forward_blocked`` / ``backward_blocked`` -- the same definitions as
  ``forward`` / ``backward``, computed with fp64 matrix products (PyTorch CPU,
  a library matmul as the step A = E C^T, G C and G^T E) on blocks of rows,
  for the full-size parity checks where the plain loops take too long.  They
  follow the same steps in the same order per row and are pinned by the same
  tests as the plain functions.
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
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
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


def threads():
    """Threads the plain oracle's OpenMP loops run on."""
    return int(_load().oracle_threads())


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



# ---- blocked fp64 versions (library matmul per block of rows) --------------

def _t64(a):
    import torch
    return torch.from_numpy(_f64(a))


def forward_blocked(E, C, x, ignore_index=-100, reduction="mean", block=256, progress=None):
    """``forward`` with A = E C^T formed by an fp64 matrix product per block of
    rows ("Cut Your Losses" digest, "The Mathematical Decomposition"):
    lse = m + log sum exp(A - m), and the loss as (m - t) + log(exp(t - m) +
    sum over v != x of exp(A - m)), which is lse - t written so that it keeps
    full relative accuracy when the target dominates.  Returns (loss, lse,
    n_valid) like ``forward``.  progress(rows done, rows), if given, is called
    after each block (reporting only)."""
    import torch
    x = _i64(x)
    N = x.shape[0]
    Et, Ct = _t64(E), _t64(C)
    V = Ct.shape[0]
    valid = x != ignore_index
    if np.any(valid & ((x < 0) | (x >= V))):
        raise ValueError("oracle forward_blocked: target outside [0, V)")
    lse = np.zeros(N)
    row_loss = np.zeros(N)
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, block):
        r = rows[r0:r0 + block]
        A = Et[torch.from_numpy(r)] @ Ct.T
        m = A.amax(dim=1, keepdim=True)
        P = torch.exp(A - m)
        xi = torch.from_numpy(x[r])
        t = A.gather(1, xi[:, None])
        lse[r] = (m + torch.log(P.sum(dim=1, keepdim=True)))[:, 0].numpy()
        P.scatter_(1, xi[:, None], 0.0)
        off = P.sum(dim=1, keepdim=True)  # the other entries' mass, summed on its own
        # target at the maximum: the loss is log1p of the other entries' mass
        at_max = (t >= m)[:, 0]
        l = (m - t) + torch.log(torch.exp(t - m) + off)
        l[at_max] = torch.log1p(off[at_max])
        row_loss[r] = l[:, 0].numpy()
        if progress is not None:
            progress(min(r0 + block, rows.size), rows.size)
    nv = int(rows.size)
    red = REDUCTIONS[reduction]
    if red == 0:
        return row_loss, lse, nv
    tot = float(row_loss[rows].sum())
    return (tot if red == 2 else tot / max(nv, 1)), lse, nv


def block_grad(E, C, x, rows, lse=None, ignore_index=-100):
    """G = exp(A - lse) - onehot(x) for the given rows (all valid), fp64,
    A = E[rows] C^T by one matrix product (digest, Algorithm 4).  With lse None
    it is formed from the same A."""
    import torch
    Et = E if isinstance(E, torch.Tensor) else _t64(E)
    Ct = C if isinstance(C, torch.Tensor) else _t64(C)
    ri = torch.from_numpy(np.asarray(rows, dtype=np.int64))
    A = Et[ri] @ Ct.T
    if lse is None:
        m = A.amax(dim=1, keepdim=True)
        l = m + torch.log(torch.exp(A - m).sum(dim=1, keepdim=True))
    else:
        l = torch.from_numpy(_f64(lse)[rows])[:, None]
    G = torch.exp(A - l)
    xi = torch.from_numpy(_i64(x)[rows])
    G[torch.arange(len(rows)), xi] -= 1.0
    return G


def _unit_filter(G, eps, unit_rows, unit_cols):
    """Zero every unit_rows x unit_cols unit of G (rows from 0, columns from 0,
    clipped) whose every |G| < eps; returns (filtered copy, units dropped)."""
    import torch
    R, V = G.shape
    ru = (R + unit_rows - 1) // unit_rows
    cu = (V + unit_cols - 1) // unit_cols
    P = torch.zeros(ru * unit_rows, cu * unit_cols, dtype=G.dtype)
    P[:R, :V] = G.abs()
    mx = P.reshape(ru, unit_rows, cu, unit_cols).amax(dim=(1, 3))
    drop = mx < eps
    keep = (~drop).repeat_interleave(unit_rows, 0).repeat_interleave(unit_cols, 1)[:R, :V]
    return G * keep, int(drop.sum())


def backward_blocked(E, C, x, grad, ignore_index=-100, reduction="mean", eps=0.0,
                     unit_rows=32, unit_cols=32, filter_mode="both", compact=True,
                     block_units=8, lse=None, progress=None):
    """``backward`` with fp64 matrix products per block of rows (digest,
    Algorithms 3 and 4 and "Gradient Filtering"): per block of block_units
    filter-unit rows, G = exp(E C^T - lse) - onehot, the unit filter on the
    unscaled G, then dE = s G C and dC += (s G)^T E.  `eps` may be a list:
    then the G of each block is formed once and one (dE, dC, total, skipped)
    is returned per threshold.  lse (optional) is the forward's lse to use in
    G; by default it is formed from the same logits.  progress(rows done,
    rows), if given, is called after each block (reporting only)."""
    import torch
    x = _i64(x)
    N = x.shape[0]
    Et, Ct = _t64(E), _t64(C)
    V, D = Ct.shape
    valid = x != ignore_index
    if np.any(valid & ((x < 0) | (x >= V))):
        raise ValueError("oracle backward_blocked: target outside [0, V)")
    eps_list = list(eps) if isinstance(eps, (list, tuple)) else [eps]
    FILTER_MODES[filter_mode]  # KeyError for an unknown mode, as in ``backward``
    nv = int(valid.sum())
    red = REDUCTIONS[reduction]
    g = _f64(np.atleast_1d(grad))
    if red == 0:
        assert g.shape == (N,), "reduction 'none' takes one upstream value per row"
        s = np.where(valid, g, 0.0)
    elif red == 2:
        s = np.where(valid, g[0], 0.0)
    else:
        s = np.where(valid, g[0] / max(nv, 1), 0.0)
    rows_all = np.nonzero(valid)[0] if compact else np.arange(N)
    out = [[torch.zeros(N, D, dtype=torch.float64), torch.zeros(V, D, dtype=torch.float64), 0]
           for _ in eps_list]
    step = unit_rows * block_units
    for r0 in range(0, rows_all.size, step):
        r = rows_all[r0:r0 + step]
        rv = r[valid[r]]
        G = torch.zeros(len(r), V, dtype=torch.float64)
        if rv.size:
            G[torch.from_numpy(np.nonzero(valid[r])[0])] = block_grad(Et, Ct, x, rv, lse,
                                                                     ignore_index)
        sr = torch.from_numpy(s[r])[:, None]
        Er = Et[torch.from_numpy(r)]
        for o, e in zip(out, eps_list):
            if e > 0.0:
                Gf, skipped = _unit_filter(G, e, unit_rows, unit_cols)
                o[2] += skipped
            else:
                Gf = G
            GE = G if filter_mode == "full_e" else Gf
            GC = G if filter_mode == "full_c" else Gf
            o[0][torch.from_numpy(r)] = sr * (GE @ Ct)
            o[1].addmm_((sr * GC).T, Er)
        if progress is not None:
            progress(min(r0 + step, rows_all.size), rows_all.size)
    total = ((rows_all.size + unit_rows - 1) // unit_rows) * ((V + unit_cols - 1) // unit_cols)
    res = [(o[0].numpy(), o[1].numpy(), total, o[2]) for o in out]
    return res if isinstance(eps, (list, tuple)) else res[0]
