"""GPU parity on seeded random shapes: N, V, D, the generator, ignored rows,
the reduction, the filter threshold and the filter variant all drawn per case,
compared element by element with the blocked fp64 oracle ("Cut Your Losses"
digest, Algorithms 1-4 and "Numerical Stability Variants"; the kernel card's
"Correctness" tolerances).  The cases cover combinations the hand-picked tests
do not: ragged sizes on every axis at once, D from 8 to 640, one-row batches,
vocabularies shorter than a tile or spanning several chunks; and, past 16,384
rows, the backward's token blocks with up to 60% of the rows ignored."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
IGN = -100
EPS = 2.0 ** -12


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _case(i):
    r = np.random.default_rng(7000 + i)
    while True:
        N, V, D = int(r.integers(1, 1500)), int(r.integers(2, 30000)), 8 * int(r.integers(1, 81))
        if N * V * D <= 3e9:
            break
    kind = "tiny" if r.random() < 0.5 else "peaked"
    ign = int(r.integers(0, N // 3 + 1)) if r.random() < 0.6 else 0
    w = si.Workload(f"random{i}", N, V, D, kind=kind, ignore_rows=ign,
                    reduction=str(r.choice(["none", "mean", "sum"])),
                    logit_std=float(r.choice([1.0, 3.0, 6.0])), seed=300 + i)
    eps = EPS if r.random() < 0.7 else 0.0
    mode = str(r.choice(["both", "full_c", "full_e"]))
    return w, eps, mode


def _case_blocked(i):
    """Past 16,384 rows (token blocks), kept small in V and D for the oracle."""
    r = np.random.default_rng(7500 + i)
    N, V, D = int(r.integers(16385, 26000)), int(r.integers(300, 6000)), 8 * int(r.integers(1, 33))
    ign = int(r.integers(0, int(0.6 * N))) if r.random() < 0.7 else 0
    w = si.Workload(f"random-blocked{i}", N, V, D, kind="peaked", ignore_rows=ign,
                    reduction=str(r.choice(["none", "mean", "sum"])),
                    logit_std=float(r.choice([3.0, 6.0])), seed=400 + i)
    eps = EPS if r.random() < 0.8 else 0.0
    mode = str(r.choice(["both", "full_c", "full_e"]))
    return w, eps, mode


CASES = list(range(16))
CASES_BLOCKED = list(range(4))


@pytest.mark.parametrize("i", CASES)
def test_random_shape(i):
    _check(*_case(i))


@pytest.mark.parametrize("i", CASES_BLOCKED)
def test_random_blocked_shape(i):
    _check(*_case_blocked(i))


def _check(w, eps, mode):
    import linear_cross_entropy_amd as lce
    E, C, x = si.generate(w)
    g = si.upstream_grad(w, "random")
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    loss, lse = lce.cce_forward(Ed, Cd, xd, IGN, w.reduction)
    rows, _ = lce.cce_forward(Ed, Cd, xd, IGN, "none")
    dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, g.to(DEV), IGN, w.reduction, eps,
                                  with_stats=True, filter_mode=mode)
    torch.cuda.synchronize()
    E64, C64, xs = E.double().numpy(), C.double().numpy(), x.numpy()
    ref_rows, ref_lse, _ = oracle.forward_blocked(E64, C64, xs, IGN, "none")
    ref_dE, ref_dC, tot, skp = oracle.backward_blocked(E64, C64, xs, g.double().numpy(), IGN,
                                                       w.reduction, eps=eps, filter_mode=mode)
    valid = xs != IGN
    print(f"{w.name}: N={w.N} V={w.V} D={w.D} {w.kind} ignored={w.ignore_rows} {w.reduction} "
          f"eps={eps:g} {mode}", flush=True)
    lse_h, rows_h = lse.cpu().double().numpy(), rows.cpu().double().numpy()
    if valid.any():
        assert np.max(np.abs(lse_h[valid] - ref_lse[valid])) <= 1e-5
    assert _rel(rows_h, ref_rows) <= 1e-5
    if w.reduction != "none":
        ref = ref_rows[valid].sum() / (max(int(valid.sum()), 1) if w.reduction == "mean" else 1)
        assert abs(float(loss) - ref) <= 1e-5 * abs(ref) + 1e-30
    got_dE, got_dC = dE.cpu().double().numpy(), dC.cpu().double().numpy()
    eE, eC = _rel(got_dE, ref_dE), _rel(got_dC, ref_dC)
    print(f"  dE rel {eE:.2e}, dC rel {eC:.2e}; units skipped {st['units_skipped']} "
          f"(oracle {skp}) of {tot}", flush=True)
    assert eE <= 3e-3 and eC <= 3e-3, (eE, eC)
    assert np.all(got_dE[~valid] == 0.0)
    assert st["units_total"] == tot
    assert abs(st["units_skipped"] - skp) <= max(2, 0.002 * tot), (st, skp)
