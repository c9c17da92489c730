"""GPU parity of vocabulary sorting ("Cut Your Losses" digest, "Vocabulary
Sorting"), through cce_vocab_order and cce_backward_sorted.

* The order: several orders are correct where averages tie within rounding,
  so the GPU's order is checked for what is unique: it is a permutation, and
  the oracle's fp64 averages taken along it never rise by more than the fp32
  error bound of the two entries involved (derived below); wherever the GPU
  and the oracle's order differ, the two entries' averages lie within that
  bound.
* The sorted backward: the order comes from the oracle (or is a seeded
  permutation) and goes to both sides; dE and dC against the oracle's sorted
  backward at the tolerances of the other parity tests (3e-3 relative
  Frobenius, ignored rows exactly zero), the unit counts as there.
* A constructed input whose high-probability entries are scattered over the
  ids: sorting must raise the skipped units from under half to over 90%.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

IGN = -100
EPS = 2.0 ** -12
DEV = "cuda:0"
U32 = 2.0 ** -24  # fp32 unit roundoff


def _lce():
    import linear_cross_entropy_amd as lce
    return lce


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _avg_bound(E64, C64, x64):
    """Per-entry bound on the fp32 average logit's error: the mean row is fp32
    partial sums over at most rows_per rows (then fp64), so each component is
    off by at most rows_per * u * mean|E_d| + u |mean_d|; the dot product over
    D terms in fp32 adds D * u * sum_d |C_vd mean_d|.  Doubled for margin."""
    N, D = E64.shape
    V = C64.shape[0]
    valid = (x64 != IGN) & (x64 >= 0) & (x64 < V)
    Ev = E64[valid]
    nrb = min(-(-N // 64), 256) if N else 1
    rows_per = -(-N // nrb) if N else 0
    mean = Ev.mean(axis=0) if Ev.shape[0] else np.zeros(D)
    mabs = np.abs(Ev).mean(axis=0) if Ev.shape[0] else np.zeros(D)
    dmean = rows_per * U32 * mabs + U32 * np.abs(mean)
    return 2.0 * (D * U32 * (np.abs(C64) @ np.abs(mean)) + np.abs(C64) @ dmean)


def _check_order(got, a, tol):
    V = a.shape[0]
    assert got.shape == (V,) and np.array_equal(np.sort(got), np.arange(V))
    step = a[got[1:]] - a[got[:-1]]
    slack = tol[got[1:]] + tol[got[:-1]]
    assert np.all(step <= slack), float(np.max(step - slack))
    ref = np.argsort(-a, kind="stable")
    diff = np.nonzero(got != ref)[0]
    assert np.all(np.abs(a[got[diff]] - a[ref[diff]]) <= 2 * tol.max()), diff[:8]
    return diff.size


@pytest.mark.parametrize("name,N,V,D,ign,seed", [
    ("ragged", 300, 5000, 72, 9, 61),        # one global bitonic step, D % 64 != 0
    ("multichunk", 200, 20000, 128, 10, 62),  # three global steps per late stage
    ("empty", 0, 3000, 64, 0, 63),            # no rows: the identity
])
def test_vocab_order_against_oracle(name, N, V, D, ign, seed):
    w = si.Workload(name, N, V, D, logit_std=4.0, ignore_rows=ign, seed=seed)
    E, C, x = si.generate(w)
    E64, C64, x64 = E.double().numpy(), C.double().numpy(), x.numpy()
    got = _lce().cce_vocab_order(E.to(DEV), C.to(DEV), x.to(DEV), IGN).cpu().numpy()
    again = _lce().cce_vocab_order(E.to(DEV), C.to(DEV), x.to(DEV), IGN).cpu().numpy()
    np.testing.assert_array_equal(got, again)  # bitwise reproducible
    if N == 0:
        np.testing.assert_array_equal(got, np.arange(V))
        return
    _, a = oracle.vocab_order(E64, C64, x64, IGN)
    nd = _check_order(got, a, _avg_bound(E64, C64, x64))
    print(f"{name}: {nd} of {V} positions differ from the fp64 order (within the bound)",
          flush=True)


def _sorted_run(E, C, x, reduction, eps, grad, order):
    lce = _lce()
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    _, lse = lce.cce_forward(Ed, Cd, xd, IGN, reduction)
    od = torch.from_numpy(np.asarray(order, dtype=np.int32)).to(DEV)
    dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, grad.to(DEV), IGN, reduction, eps,
                                  with_stats=True, vocab_order=od)
    torch.cuda.synchronize()
    return dE.cpu().double().numpy(), dC.cpu().double().numpy(), st


def _check_sorted(w, eps, order_kind, E=None, C=None, x=None):
    if E is None:
        E, C, x = si.generate(w)
    g = si.upstream_grad(w, "random")
    E64, C64, x64 = E.double().numpy(), C.double().numpy(), x.numpy()
    if order_kind == "oracle":
        order, _ = oracle.vocab_order(E64, C64, x64, IGN)
    elif order_kind == "identity":
        order = np.arange(w.V)
    else:
        order = np.random.default_rng(w.seed + 500).permutation(w.V)
    dE, dC, st = _sorted_run(E, C, x, w.reduction, eps, g, order)
    ref_dE, ref_dC, tot, skp = oracle.backward(E64, C64, x64, g.double().numpy(), IGN,
                                               w.reduction, eps=eps, vocab_order=order)
    print(f"{w.name} eps={eps:g} {order_kind}: dE rel {_rel(dE, ref_dE):.2e} dC rel "
          f"{_rel(dC, ref_dC):.2e} skipped {st['units_skipped']} (oracle {skp}) of {tot}",
          flush=True)
    assert _rel(dE, ref_dE) <= 3e-3 and _rel(dC, ref_dC) <= 3e-3
    assert np.all(dE[x64 == IGN] == 0.0)
    assert st["units_total"] == tot
    if eps == 0:
        assert st["units_skipped"] == 0
    else:
        assert abs(st["units_skipped"] - skp) <= max(2, 0.002 * tot), (st, skp)
    return st, skp


@pytest.mark.parametrize("eps,order_kind", [(0.0, "random"), (EPS, "random"), (EPS, "oracle")])
def test_sorted_backward_tiny(eps, order_kind):
    _check_sorted(si.TINY, eps, order_kind)


@pytest.mark.parametrize("order_kind", ["random", "oracle"])
def test_sorted_backward_multi_chunk(order_kind):
    # three backward chunks (the last ragged), ignored rows, targets in the tail
    w = si.Workload("multichunk", 200, 20000, 128, logit_std=5.0, ignore_rows=10,
                    tail_targets=20, tail_width=300, seed=22)
    _check_sorted(w, EPS, order_kind)


def _scattered(N, V, D, frac, seed):
    """Entries of a random subset (frac of V, scattered over the ids) get
    logits about 12 above the rest on every row: each E row and each chosen C
    row carry a shared direction u (bf16 inputs)."""
    r = np.random.default_rng(seed)
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    C = 0.02 * r.standard_normal((V, D))
    hot = r.choice(V, size=int(frac * V), replace=False)
    C[hot] += 0.5 * u
    E = 0.5 * r.standard_normal((N, D)) / (0.02 * np.sqrt(D)) + 24.0 * u
    x = r.choice(hot, size=N).astype(np.int64)
    to_bf16 = lambda a: torch.from_numpy(a.astype(np.float32)).bfloat16()
    return to_bf16(E), to_bf16(C), torch.from_numpy(x), hot


def test_sorting_gathers_scattered_entries():
    # In id order about 3% hot entries touch most 32-wide vocabulary units;
    # sorted by average logit they fill the first few units and the rest is
    # filtered.  Parity of both runs against the oracle.
    N, V, D = 512, 16384, 128
    E, C, x, hot = _scattered(N, V, D, 0.03, seed=64)
    w = si.Workload("scattered", N, V, D, seed=64)
    st_plain, _ = _check_sorted(w, EPS, "random", E, C, x)  # a random order: still scattered
    st_sorted, _ = _check_sorted(w, EPS, "oracle", E, C, x)
    got = _lce().cce_vocab_order(E.to(DEV), C.to(DEV), x.to(DEV), IGN).cpu().numpy()
    assert set(got[:hot.size].tolist()) == set(hot.tolist())
    tot = st_sorted["units_total"]
    print(f"skipped units: random order {st_plain['units_skipped']}, sorted "
          f"{st_sorted['units_skipped']} of {tot}", flush=True)
    assert st_plain["units_skipped"] < 0.5 * tot < 0.9 * tot < st_sorted["units_skipped"]


def test_sorting_with_likely_entries():
    # The generator's entry_bias: a per-entry logit bias shared by all tokens
    # (likely entries, scattered over the ids).  Sorted by average logit the
    # likely entries share units, so more units are filtered than in id order
    # (the CPU probe of this input: 99.2% kept in id order, 80.9% sorted).
    # Parity of both runs against the oracle.
    w = si.Workload("entry-bias", 512, 20000, 256, entry_bias=1.5, seed=65)
    st_id, _ = _check_sorted(w, EPS, "identity")
    st_so, _ = _check_sorted(w, EPS, "oracle")
    tot = st_so["units_total"]
    print(f"entry bias: skipped units {st_id['units_skipped']} in id order, "
          f"{st_so['units_skipped']} sorted, of {tot}", flush=True)
    assert st_so["units_skipped"] > st_id["units_skipped"] + 0.1 * tot


def test_sorted_backward_full_size_qwen():
    # Qwen2.5-0.5B head shape through the launches bench.py times: the GPU's
    # order against the oracle's averages; with the oracle's order, dE unit
    # row blocks against the oracle's sorted backward on those rows, every
    # ignored row zero, and <dC, C> = <dE, E> (true in any order)
    import dataclasses
    lce = _lce()
    w = dataclasses.replace(si.QWEN, ignore_rows=205)
    E, C, x = si.generate(w)
    E64, C64, xs = E.double().numpy(), C.double().numpy(), x.numpy()
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    got = lce.cce_vocab_order(Ed, Cd, xd, IGN).cpu().numpy()
    order, a = oracle.vocab_order(E64, C64, xs, IGN)
    nd = _check_order(got, a, _avg_bound(E64, C64, xs))
    print(f"qwen: GPU order differs from the fp64 one at {nd} positions (within bound)", flush=True)
    g = si.upstream_grad(w, "random")
    gd = g.to(DEV)
    _, lse = lce.cce_forward(Ed, Cd, xd, IGN, w.reduction)
    od = torch.from_numpy(order.astype(np.int32)).to(DEV)
    dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, gd, IGN, w.reduction, EPS, with_stats=True,
                                  vocab_order=od)
    a_, b_ = (dC.double() * Cd.double()).sum().item(), (dE.double() * Ed.double()).sum().item()
    torch.cuda.synchronize()
    assert abs(a_ - b_) <= 2e-3 * abs(b_), (a_, b_)
    valid = xs != IGN
    assert torch.count_nonzero(dE[torch.from_numpy(~valid).to(DEV)]).item() == 0
    vidx = np.nonzero(valid)[0]
    assert st["units_total"] == ((vidx.size + 31) // 32) * ((w.V + 31) // 32)
    valid_n = int(valid.sum())
    s = np.where(valid, float(g) / valid_n, 0.0)
    for b in (0, (vidx.size + 31) // 32 - 1):
        rows = vidx[32 * b:32 * b + 32]
        ref = oracle.backward(E64[rows], C64, xs[rows], s[rows], IGN, "none", eps=EPS,
                              vocab_order=order)[0]
        r = _rel(dE[torch.from_numpy(rows).to(DEV)].double().cpu().numpy(), ref)
        print(f"qwen sorted: dE unit block {b} rel {r:.2e}", flush=True)
        assert r <= 3e-3


def test_sorted_backward_full_size_gemma_likely_entries():
    # Gemma-2-2B head shape with likely entries (the generator's entry_bias:
    # a per-entry logit bias of std 1 shared by all tokens), where sorting has
    # something to gather, through the launches bench.py times: the GPU's order
    # against the oracle's averages; with the oracle's order the sorted backward
    # keeps fewer units than the plain one, <dC, C> = <dE, E>, and the first and
    # last dE unit row blocks match the oracle's sorted backward on those rows
    lce = _lce()
    w = si.GEMMA_BIASED
    E, C, x = si.generate(w)
    E64, C64, xs = E.double().numpy(), C.double().numpy(), x.numpy()
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    got = lce.cce_vocab_order(Ed, Cd, xd, IGN).cpu().numpy()
    order, a = oracle.vocab_order(E64, C64, xs, IGN)
    nd = _check_order(got, a, _avg_bound(E64, C64, xs))
    print(f"gemma likely entries: GPU order differs from the fp64 one at {nd} positions "
          f"(within bound)", flush=True)
    g = si.upstream_grad(w)
    gd = g.to(DEV)
    _, lse = lce.cce_forward(Ed, Cd, xd, IGN, w.reduction)
    _, _, st_plain = lce.cce_backward(Ed, Cd, xd, lse, gd, IGN, w.reduction, EPS, with_stats=True)
    od = torch.from_numpy(order.astype(np.int32)).to(DEV)
    dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, gd, IGN, w.reduction, EPS, with_stats=True,
                                  vocab_order=od)
    a_, b_ = (dC.double() * Cd.double()).sum().item(), (dE.double() * Ed.double()).sum().item()
    torch.cuda.synchronize()
    tot = st["units_total"]
    assert tot == st_plain["units_total"] == (w.N // 32) * (w.V // 32)
    print(f"gemma likely entries: kept {1 - st_plain['units_skipped'] / tot:.4f} in id order, "
          f"{1 - st['units_skipped'] / tot:.4f} sorted", flush=True)
    assert st["units_skipped"] > st_plain["units_skipped"] + 0.05 * tot
    assert abs(a_ - b_) <= 2e-3 * abs(b_), (a_, b_)
    s = np.full(w.N, float(g) / w.N)
    for b in (0, w.N // 32 - 1):
        rows = np.arange(32 * b, 32 * b + 32)
        ref = oracle.backward(E64[rows], C64, xs[rows], s[rows], IGN, "none", eps=EPS,
                              vocab_order=order)[0]
        r = _rel(dE[torch.from_numpy(rows).to(DEV)].double().cpu().numpy(), ref)
        print(f"gemma likely entries sorted: dE unit block {b} rel {r:.2e}", flush=True)
        assert r <= 3e-3


def test_autograd_wrapper_with_vocab_sort():
    # linear_cross_entropy(..., vocab_sort=True): the order is taken from the
    # forward inputs and the backward runs sorted; against the oracle's
    # sorted backward with the oracle's own order
    lce = _lce()
    w = si.Workload("autograd-sort", 300, 5000, 72, logit_std=5.0, ignore_rows=9, seed=65)
    E, C, x = si.generate(w)
    Ed = E.to(DEV).requires_grad_(True)
    Cd = C.to(DEV).requires_grad_(True)
    loss = lce.linear_cross_entropy(Ed, Cd, x.to(DEV), IGN, "mean", vocab_sort=True)
    loss.backward()
    torch.cuda.synchronize()
    E64, C64, x64 = E.double().numpy(), C.double().numpy(), x.numpy()
    ref_loss, _, _ = oracle.forward(E64, C64, x64, IGN, "mean")
    order, _ = oracle.vocab_order(E64, C64, x64, IGN)
    ref_dE, ref_dC, _, _ = oracle.backward(E64, C64, x64, 1.0, IGN, "mean", eps=EPS,
                                           vocab_order=order)
    assert abs(float(loss.detach()) - ref_loss) <= 1e-5 * abs(ref_loss)
    assert _rel(Ed.grad.double().cpu().numpy(), ref_dE) <= 3e-3
    assert _rel(Cd.grad.double().cpu().numpy(), ref_dC) <= 3e-3


def test_order_that_is_not_a_permutation_stays_in_bounds():
    # The documented behaviour for a bad order: entries outside [0, V) are
    # never used as an index (their positions read as zero rows and write no
    # dC row) and the results are unspecified.  The call returns, and a
    # following correct call on the same workspace is exact again.
    lce = _lce()
    w = si.Workload("bad-order", 256, 3000, 64, logit_std=4.0, seed=66)
    E, C, x = si.generate(w)
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    _, lse = lce.cce_forward(Ed, Cd, xd, IGN, "mean")
    g = torch.ones((), device=DEV)
    bad = torch.arange(w.V, dtype=torch.int32)
    bad[0], bad[1], bad[2], bad[-1] = -5, w.V, 7, 2 ** 30  # out of range and a duplicate
    ws = torch.empty(lce.cce_workspace_bytes(w.N, w.V, w.D)[1], dtype=torch.uint8, device=DEV)
    lce.cce_backward(Ed, Cd, xd, lse, g, IGN, "mean", EPS, workspace=ws, vocab_order=bad.to(DEV))
    torch.cuda.synchronize()
    ident = torch.arange(w.V, dtype=torch.int32, device=DEV)
    dE1, dC1 = lce.cce_backward(Ed, Cd, xd, lse, g, IGN, "mean", EPS, workspace=ws,
                                vocab_order=ident)
    dE0, dC0 = lce.cce_backward(Ed, Cd, xd, lse, g, IGN, "mean", EPS, workspace=ws)
    torch.cuda.synchronize()
    # the identity order is the unsorted backward, bit for bit
    assert torch.equal(dE1, dE0) and torch.equal(dC1, dC0)
