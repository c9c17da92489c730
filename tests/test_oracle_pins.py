"""Pins of the fp64 oracle against things other than itself.

Each test ties the oracle to what the pages and mathematics fix:

* a textbook dense log-softmax / NLL from PyTorch (float64, CPU, autograd),
* the closed form at E = 0 (every logit 0: lse = ln V, G = 1/V - onehot,
  dC = 0 exactly),
* the row-sum invariant of G (softmax rows sum to 1, the one-hot to 1),
* central finite differences of the loss,
* the masking, reduction and permutation properties the kernel card lists
  ("cut-cross-entropy", Correctness) and the "Cut Your Losses" digest implies
  (Vocabulary Sorting: a permutation of the vocabulary leaves the loss alone),
* the tile filter on a constructed case whose filtered units are known,
* vocabulary sorting (digest, "Vocabulary Sorting"): averages by plain loops, a
  closed-form order, the order-invariance of the unfiltered gradient, and a
  constructed case whose units sorting turns from mixed into skippable.

A plausible mistake in the oracle (dropped term, flipped sign of G, wrong
index or transposed operand, wrong mean denominator, filter on S instead of
|G|, filter on scaled instead of unscaled G) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle

IGN = -100


def _bwd_blocked_small(*a, **k):
    # one filter-unit row per block, so that block boundaries fall inside the tiny cases
    return oracle.backward_blocked(*a, block_units=1, **k)


# Both forms of the oracle answer to the same pins: the plain loops (C) and the
# blocked fp64 matrix products (the full-size parity checks use those).
IMPLS = {
    "loops": (oracle.forward, oracle.backward),
    "blocked": (oracle.forward_blocked, _bwd_blocked_small),
}
impl_names = pytest.mark.parametrize("impl", list(IMPLS))


def _rand(N, V, D, seed, ignore=(), scale=1.0):
    r = np.random.default_rng(seed)
    E = r.standard_normal((N, D)) * scale
    C = r.standard_normal((V, D)) * (scale / math.sqrt(D)) * 2.0
    x = r.integers(0, V, size=N).astype(np.int64)
    for i in ignore:
        x[i] = IGN
    return E, C, x


def _torch_dense(E, C, x, reduction, grad):
    """Textbook dense reference: materialised logits, F.cross_entropy, autograd."""
    Et = torch.tensor(E, dtype=torch.float64, requires_grad=True)
    Ct = torch.tensor(C, dtype=torch.float64, requires_grad=True)
    xt = torch.tensor(x)
    logits = Et @ Ct.T
    loss = torch.nn.functional.cross_entropy(logits, xt, ignore_index=IGN,
                                             reduction=reduction)
    lse = torch.logsumexp(logits, dim=1)
    g = torch.tensor(grad, dtype=torch.float64)
    if reduction == "none":
        (loss * g).sum().backward()
    else:
        (loss * g.reshape(())).backward()
    return loss.detach().numpy(), lse.detach().numpy(), Et.grad.numpy(), Ct.grad.numpy()


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@impl_names
def test_matches_dense_log_softmax(reduction, impl):
    forward, backward = IMPLS[impl]
    N, V, D = 40, 300, 24
    E, C, x = _rand(N, V, D, seed=1, ignore=(3, 17, 18))
    grad = np.random.default_rng(2).uniform(0.5, 1.5, N) if reduction == "none" else np.array(0.7)
    ref_loss, ref_lse, ref_dE, ref_dC = _torch_dense(E, C, x, reduction, grad)
    loss, lse, nv = forward(E, C, x, IGN, reduction)
    assert nv == N - 3
    valid = x != IGN
    np.testing.assert_allclose(lse[valid], ref_lse[valid], rtol=1e-13, atol=0)
    assert np.all(lse[~valid] == 0.0)
    np.testing.assert_allclose(loss, ref_loss, rtol=1e-12, atol=1e-14)
    dE, dC, tot, skp = backward(E, C, x, grad, IGN, reduction, eps=0.0)
    assert skp == 0 and tot == math.ceil(N / 32) * math.ceil(V / 32)
    np.testing.assert_allclose(dE, ref_dE, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dC, ref_dC, rtol=1e-11, atol=1e-14)


@impl_names
def test_E_zero_closed_form(impl):
    forward, backward = IMPLS[impl]
    # Tiny shape: V = 2048 -> every logit 0, lse = ln 2048 exactly.
    N, V, D = 16, 2048, 64
    _, C, x = _rand(N, V, D, seed=3, ignore=(5,))
    E = np.zeros((N, D))
    loss, lse, nv = forward(E, C, x, IGN, "none")
    valid = x != IGN
    assert abs(math.log(2048) - 7.624618986159398) < 1e-15
    np.testing.assert_allclose(lse[valid], math.log(V), rtol=2e-16)
    np.testing.assert_allclose(loss[valid], math.log(V), rtol=1e-15)
    assert loss[5] == 0.0
    mean_loss, _, _ = forward(E, C, x, IGN, "mean")
    assert abs(mean_loss - math.log(V)) < 1e-14
    g = 1.3
    dE, dC, _, _ = backward(E, C, x, g, IGN, "mean", eps=0.0)
    assert np.all(dC == 0.0)  # E = 0 makes every dC term 0 exactly
    s = g / nv
    cbar = C.mean(axis=0)
    for n in range(N):
        if x[n] == IGN:
            assert np.all(dE[n] == 0.0)
        else:
            np.testing.assert_allclose(dE[n], s * (cbar - C[x[n]]), rtol=1e-12, atol=1e-15)
    G = oracle.grad_logits(E, C, x, IGN)
    for n in range(N):
        if x[n] == IGN:
            continue
        expect = np.full(V, 1.0 / V)
        expect[x[n]] -= 1.0
        np.testing.assert_allclose(G[n], expect, rtol=1e-14, atol=1e-17)


def test_G_rows_sum_to_zero_and_sign():
    N, V, D = 24, 500, 32
    E, C, x = _rand(N, V, D, seed=4, ignore=(0,))
    G = oracle.grad_logits(E, C, x, IGN)
    assert np.all(G[0] == 0.0)
    sums = G[1:].sum(axis=1)
    assert np.max(np.abs(sums)) < V * 2.0 ** -52 * 4
    # sign: gradient of the loss, softmax minus onehot -> target entry negative, rest positive
    for n in range(1, N):
        assert G[n, x[n]] < 0
        assert np.all(np.delete(G[n], x[n]) > 0)


@impl_names
def test_central_finite_differences(impl):
    forward, backward = IMPLS[impl]
    N, V, D = 8, 64, 16
    E, C, x = _rand(N, V, D, seed=5, ignore=(6,))
    h = 1e-5

    def f(E_, C_):
        return forward(E_, C_, x, IGN, "mean")[0]

    dE, dC, _, _ = backward(E, C, x, 1.0, IGN, "mean", eps=0.0)
    fdE = np.zeros_like(E)
    for i in range(N):
        for d in range(D):
            Ep, Em = E.copy(), E.copy()
            Ep[i, d] += h
            Em[i, d] -= h
            fdE[i, d] = (f(Ep, C) - f(Em, C)) / (2 * h)
    fdC = np.zeros_like(C)
    for v in range(V):
        for d in range(D):
            Cp, Cm = C.copy(), C.copy()
            Cp[v, d] += h
            Cm[v, d] -= h
            fdC[v, d] = (f(E, Cp) - f(E, Cm)) / (2 * h)
    scale = max(np.abs(dE).max(), np.abs(dC).max())
    assert np.max(np.abs(fdE - dE)) <= 1e-8 * scale + 1e-11
    assert np.max(np.abs(fdC - dC)) <= 1e-8 * scale + 1e-11
    assert np.all(dE[6] == 0.0)


@impl_names
def test_masking_properties(impl):
    forward, backward = IMPLS[impl]
    N, V, D = 33, 200, 16
    E, C, x = _rand(N, V, D, seed=6, ignore=(0, 7, 32))
    loss, lse, _ = forward(E, C, x, IGN, "none")
    assert loss[0] == loss[7] == loss[32] == 0.0
    dE, dC, _, _ = backward(E, C, x, np.ones(N), IGN, "none", eps=0.0)
    assert np.all(dE[[0, 7, 32]] == 0.0)
    E2 = E.copy()
    E2[[0, 7, 32]] *= 1e3
    loss2, lse2, _ = forward(E2, C, x, IGN, "none")
    dE2, dC2, _, _ = backward(E2, C, x, np.ones(N), IGN, "none", eps=0.0)
    assert np.array_equal(loss, loss2) and np.array_equal(dC, dC2)
    # fully masked batch: zero loss, zero and finite gradients
    xm = np.full(N, IGN, dtype=np.int64)
    for red in ("mean", "sum"):
        l, _, nv = forward(E, C, xm, IGN, red)
        assert l == 0.0 and nv == 0
        dE, dC, _, _ = backward(E, C, xm, 1.0, IGN, red, eps=0.0)
        assert np.all(dE == 0.0) and np.all(dC == 0.0)
    # empty batch
    l, lse0, nv = forward(np.zeros((0, D)), C, np.zeros(0, np.int64), IGN, "mean")
    assert l == 0.0 and nv == 0 and lse0.shape == (0,)


@impl_names
def test_reduction_consistency(impl):
    forward, backward = IMPLS[impl]
    N, V, D = 30, 150, 20
    E, C, x = _rand(N, V, D, seed=7, ignore=(2, 4))
    none, _, nv = forward(E, C, x, IGN, "none")
    s, _, _ = forward(E, C, x, IGN, "sum")
    m, _, _ = forward(E, C, x, IGN, "mean")
    assert nv == 28
    assert abs(s - none.sum()) <= 1e-12 * abs(s)
    assert abs(m - s / nv) <= 1e-12 * abs(m)
    dEm, dCm, _, _ = backward(E, C, x, 2.0, IGN, "mean", eps=0.0)
    dEs, dCs, _, _ = backward(E, C, x, 2.0 / nv, IGN, "sum", eps=0.0)
    dEn, dCn, _, _ = backward(E, C, x, np.full(N, 2.0 / nv), IGN, "none", eps=0.0)
    np.testing.assert_allclose(dEm, dEs, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dCm, dCs, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dEn, dEs, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dCn, dCs, rtol=1e-13, atol=1e-16)


def test_permutation_and_row_independence():
    N, V, D = 20, 96, 12
    E, C, x = _rand(N, V, D, seed=8, ignore=(9,))
    perm = np.random.default_rng(9).permutation(V)  # new row j holds old row perm[j]
    inv = np.argsort(perm)
    Cp = C[perm]
    xp = np.where(x == IGN, IGN, inv[np.where(x == IGN, 0, x)])
    l1, lse1, _ = oracle.forward(E, C, x, IGN, "none")
    l2, lse2, _ = oracle.forward(E, Cp, xp, IGN, "none")
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-14)
    _, dC1, _, _ = oracle.backward(E, C, x, np.ones(N), IGN, "none", eps=0.0)
    _, dC2, _, _ = oracle.backward(E, Cp, xp, np.ones(N), IGN, "none", eps=0.0)
    np.testing.assert_allclose(dC2, dC1[perm], rtol=1e-12, atol=1e-15)
    rp = np.random.default_rng(10).permutation(N)
    l3, lse3, _ = oracle.forward(E[rp], C, x[rp], IGN, "none")
    np.testing.assert_allclose(l3, l1[rp], rtol=1e-14, atol=0)
    dE1, _, _, _ = oracle.backward(E, C, x, np.ones(N), IGN, "none", eps=0.0)
    dE3, _, _, _ = oracle.backward(E[rp], C, x[rp], np.ones(N), IGN, "none", eps=0.0)
    np.testing.assert_allclose(dE3, dE1[rp], rtol=1e-12, atol=1e-15)


def _filter_case():
    """64 rows, 128 vocab, 4 vocab units of 32.  Vocab rows 96..127 point away
    from every token, so their softmax entries are about 5e-5, below 2**-12
    but large enough that dropping them moves dE measurably: the
    (row block, unit 3) units are filtered as long as no target lies there."""
    r = np.random.default_rng(11)
    N, V, D = 64, 128, 16
    u = np.ones(D) / math.sqrt(D)
    E = r.standard_normal((N, D)) * 0.3 + 4.0 * u
    C = r.standard_normal((V, D)) * 0.3
    C[96:] = -1.15 * u + r.standard_normal((32, D)) * 0.01
    x = r.integers(0, 96, size=N).astype(np.int64)
    return E, C, x


@impl_names
def test_filter_constructed_case(impl):
    forward, backward = IMPLS[impl]
    E, C, x = _filter_case()
    N, V, D = E.shape[0], C.shape[0], E.shape[1]
    eps = 2.0 ** -12
    dE0, dC0, tot, skp0 = backward(E, C, x, 1.0, IGN, "mean", eps=0.0)
    dE1, dC1, tot1, skp1 = backward(E, C, x, 1.0, IGN, "mean", eps=eps)
    assert tot == tot1 == 2 * 4 and skp0 == 0
    G = oracle.grad_logits(E, C, x, IGN)
    assert 1e-6 < np.abs(G[:, 96:]).max() < eps
    assert skp1 == 2                     # unit 3 of each of the two row blocks
    assert np.all(dC1[96:] == 0.0) and np.any(dC0[96:] != 0.0)
    np.testing.assert_array_equal(dC1[:96], dC0[:96])
    # dE loses exactly the filtered contribution of vocab rows 96..127
    lost = (G[:, 96:] @ C[96:]) / N
    np.testing.assert_allclose(dE0 - dE1, lost, rtol=1e-9, atol=1e-30)
    # a target inside unit 3 keeps that unit (|G| ~ 1 at the target): filter is on |G|, not S
    x2 = x.copy()
    x2[0] = 100
    _, dC2, _, skp2 = backward(E, C, x2, 1.0, IGN, "mean", eps=eps)
    assert skp2 == 1 and np.any(dC2[96:] != 0.0)
    # the filter tests unscaled G: a tiny upstream gradient changes nothing about which units go
    _, _, _, skp3 = backward(E, C, x, 1e-30, IGN, "mean", eps=eps)
    assert skp3 == skp1


@impl_names
def test_filter_extremes_and_monotone(impl):
    forward, backward = IMPLS[impl]
    N, V, D = 70, 400, 16
    E, C, x = _rand(N, V, D, seed=12, ignore=(1,))
    E *= 3.0
    dE0, dC0, tot, _ = backward(E, C, x, 1.0, IGN, "mean", eps=0.0)
    dEa, dCa, _, skpa = backward(E, C, x, 1.0, IGN, "mean", eps=1e-300)
    # eps tiny (every nonzero |G| survives) equals unfiltered
    assert skpa == 0
    np.testing.assert_array_equal(dEa, dE0)
    np.testing.assert_array_equal(dCa, dC0)
    # |G| <= 1 everywhere, so eps > 1 drops every unit
    dEb, dCb, _, skpb = backward(E, C, x, 1.0, IGN, "mean", eps=1.5)
    assert skpb == tot and np.all(dEb == 0) and np.all(dCb == 0)
    prev = -1
    for eps in [2.0 ** -20, 2.0 ** -16, 2.0 ** -12, 2.0 ** -8, 2.0 ** -4, 0.5]:
        skp = backward(E, C, x, 1.0, IGN, "mean", eps=eps)[3]
        assert skp >= prev
        prev = skp


@impl_names
def test_filter_threshold_is_strict(impl):
    # "Gradient filtering" (CCE blog post): a unit is dropped when every entry
    # satisfies |G| < eps.  With eps equal to the largest |G| of one unit that
    # unit stays; one ulp above it, it goes.  A "<=" comparison fails this.
    forward, backward = IMPLS[impl]
    E, C, x = _filter_case()
    N = E.shape[0]
    if impl == "loops":
        G = oracle.grad_logits(E, C, x, IGN)
    else:  # the blocked backward forms G for the 32-row blocks with this routine
        G = np.concatenate([oracle.block_grad(E, C, x, np.arange(r, r + 32)).numpy()
                            for r in range(0, N, 32)])
    m = [np.abs(G[r:r + 32, 96:128]).max() for r in (0, 32)]
    hi = int(np.argmax(m))
    assert m[hi] > m[1 - hi]                    # the two units of vocabulary unit 3 differ
    _, dC_at, _, skp_at = backward(E, C, x, 1.0, IGN, "mean", eps=float(m[hi]))
    _, dC_up, _, skp_up = backward(E, C, x, 1.0, IGN, "mean", eps=float(np.nextafter(m[hi], 2.0)))
    assert skp_at == 1 and skp_up == 2
    assert np.any(dC_at[96:] != 0.0) and np.all(dC_up[96:] == 0.0)


@impl_names
def test_loss_when_the_target_dominates(impl):
    # D = 1, E = 1: the logits are the entries of C exactly.  Target logit 60,
    # every other logit 0: loss = log(1 + (V - 1) e^-60) ~ 1.4e-24, whose
    # relative accuracy lse - t in fp64 would lose entirely (lse ~ 60).
    forward, backward = IMPLS[impl]
    V = 300
    C = np.zeros((V, 1))
    C[7, 0] = 60.0
    E = np.ones((3, 1))
    x = np.array([7, 7, IGN], dtype=np.int64)
    loss, lse, nv = forward(E, C, x, IGN, "none")
    want = math.log1p((V - 1) * math.exp(-60.0))
    assert nv == 2 and loss[2] == 0.0
    np.testing.assert_allclose(loss[:2], want, rtol=1e-13)
    np.testing.assert_allclose(lse[:2], 60.0 + want, rtol=1e-15)
    mean, _, _ = forward(E, C, x, IGN, "mean")
    np.testing.assert_allclose(mean, want, rtol=1e-13)


def test_bad_arguments_rejected():
    E, C, x = _rand(4, 10, 3, seed=13)
    x[0] = 10  # out of range, not the ignore index
    with pytest.raises(ValueError):
        oracle.forward(E, C, x, IGN, "mean")
    with pytest.raises(ValueError):
        oracle.backward(E, C, x, 1.0, IGN, "mean")
    with pytest.raises(ValueError):
        oracle.forward_blocked(E, C, x, IGN, "mean")
    with pytest.raises(ValueError):
        oracle.backward_blocked(E, C, x, 1.0, IGN, "mean")


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_dC_columns_matches_full_backward(reduction):
    # the column-block dC (used at sizes where the full backward is too slow)
    # equals the full oracle's dC block by block, filter off and on; the
    # constructed filter case makes the filtered units known
    E, C, x = _filter_case()
    N, V = E.shape[0], C.shape[0]
    g = np.linspace(0.5, 2.0, N) if reduction == "none" else 1.0
    _, lse, _ = oracle.forward(E, C, x, IGN, reduction)
    for eps in (0.0, 2.0 ** -12):
        _, dC, _, skp = oracle.backward(E, C, x, g, IGN, reduction, eps=eps)
        blocks = list(range((V + 31) // 32))
        cols = oracle.dC_columns(E, C, x, lse, g, IGN, reduction, eps=eps, blocks=blocks)
        for b in blocks:
            ref = dC[32 * b:32 * b + 32]
            np.testing.assert_allclose(cols[b], ref, rtol=1e-10, atol=1e-13 * np.abs(dC).max())
        if eps:
            assert skp > 0 and np.all(cols[3] == 0.0)
    # a ragged final block and ignored rows
    E, C, x = _rand(50, 70, 8, seed=14, ignore=(3, 17))
    _, lse, _ = oracle.forward(E, C, x, IGN, "mean")
    _, dC, _, _ = oracle.backward(E, C, x, 1.0, IGN, "mean")
    cols = oracle.dC_columns(E, C, x, lse, 1.0, IGN, "mean", blocks=[0, 2])
    np.testing.assert_allclose(cols[2], dC[64:70], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(cols[0], dC[:32], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("mode", ["full_c", "full_e"])
@impl_names
def test_filter_variants_against_dense_autograd(mode, impl):
    forward, backward = IMPLS[impl]
    # FullC / FullE ("Cut Your Losses" digest, "Numerical Stability Variants"):
    # one contraction keeps the filter, the other takes the unfiltered G.  With
    # eps above max|G| = 1 every unit is filtered, so the filtered gradient is
    # exactly zero and the other one is the textbook dense gradient.
    N, V, D = 40, 96, 12
    E, C, x = _rand(N, V, D, seed=21, ignore=(3, 17))
    g = np.linspace(0.5, 1.5, N)
    _, _, dE_ref, dC_ref = _torch_dense(E, C, x, "none", g)
    dE, dC, tot, skp = backward(E, C, x, g, IGN, "none", eps=1.5, filter_mode=mode)
    assert skp == tot == 2 * 3
    full, zero = (dC, dE) if mode == "full_c" else (dE, dC)
    ref = dC_ref if mode == "full_c" else dE_ref
    assert np.all(zero == 0.0)
    np.testing.assert_allclose(full, ref, rtol=1e-10, atol=1e-13 * np.abs(ref).max())


@impl_names
def test_filter_variants_constructed_case(impl):
    forward, backward = IMPLS[impl]
    # The constructed case: the units (row block, vocab unit 3) are filtered.
    # FullC keeps them in dC (dC equals the dense gradient, vocab rows 96..127
    # included) and drops them from dE (dE loses exactly G[:, 96:] C[96:] / N);
    # FullE the other way round.  References: dense autograd and a torch
    # softmax, not the oracle.
    E, C, x = _filter_case()
    N = E.shape[0]
    eps = 2.0 ** -12
    _, _, dE_ref, dC_ref = _torch_dense(E, C, x, "mean", np.array(1.0))
    logits = torch.tensor(E) @ torch.tensor(C).T
    G = torch.softmax(logits, dim=1).numpy()
    G[np.arange(N), x] -= 1.0
    lost_E = (G[:, 96:] @ C[96:]) / N
    dC_filtered = dC_ref.copy()
    dC_filtered[96:] = 0.0
    dE_c, dC_c, _, skp_c = backward(E, C, x, 1.0, IGN, "mean", eps=eps, filter_mode="full_c")
    dE_e, dC_e, _, skp_e = backward(E, C, x, 1.0, IGN, "mean", eps=eps, filter_mode="full_e")
    assert skp_c == skp_e == 2
    tol = dict(rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(dC_c, dC_ref, **tol)
    np.testing.assert_allclose(dE_c, dE_ref - lost_E, **tol)
    np.testing.assert_allclose(dE_e, dE_ref, **tol)
    np.testing.assert_allclose(dC_e, dC_filtered, **tol)
    assert np.all(dC_e[96:] == 0.0) and np.any(dC_c[96:] != 0.0)
    # eps = 0: every mode is the unfiltered backward, bit for bit
    base = backward(E, C, x, 1.0, IGN, "mean", eps=0.0)
    for mode in ("full_c", "full_e"):
        got = backward(E, C, x, 1.0, IGN, "mean", eps=0.0, filter_mode=mode)
        np.testing.assert_array_equal(got[0], base[0])
        np.testing.assert_array_equal(got[1], base[1])
        assert got[3] == 0
    with pytest.raises(KeyError):
        backward(E, C, x, 1.0, IGN, "mean", eps=eps, filter_mode="kahan")


def _interleaved_ignores():
    """The constructed filter case with ignored rows spread through it: 64
    valid rows plus 20 ignored ones, so that in the original order the 32-row
    blocks mix rows of both valid blocks."""
    E, C, x = _filter_case()
    r = np.random.default_rng(31)
    N = E.shape[0] + 20
    pos = np.sort(r.choice(N, size=20, replace=False))
    keep = np.setdiff1d(np.arange(N), pos)
    E2 = np.zeros((N, E.shape[1]))
    x2 = np.full(N, IGN, dtype=np.int64)
    E2[keep] = E
    E2[pos] = r.standard_normal((20, E.shape[1]))
    x2[keep] = x
    return E2, C, x2, keep


@impl_names
def test_compaction_equals_the_batch_without_ignored_rows(impl):
    forward, backward = IMPLS[impl]
    # Ignored rows removed ahead of the gradient ("Cut Your Losses" digest,
    # Table A1): the backward with compaction equals the plain backward of the
    # batch that holds only the valid rows (scattered back; ignored rows get
    # 0), filter on and off; the filter units are then 32 consecutive valid
    # rows, which differ from 32-row blocks of the original order here.
    E, C, x, keep = _interleaved_ignores()
    N, V = E.shape[0], C.shape[0]
    g = np.linspace(0.5, 2.0, N)
    for eps in (0.0, 2.0 ** -12):
        for red, gg in (("mean", 1.0), ("none", g)):
            dE, dC, tot, skp = backward(E, C, x, gg, IGN, red, eps=eps)
            sub = gg if red == "mean" else g[keep]
            dEk, dCk, totk, skpk = backward(E[keep], C, x[keep], sub, IGN, red, eps=eps,
                                                    compact=False)
            np.testing.assert_array_equal(dC, dCk)
            np.testing.assert_array_equal(dE[keep], dEk)
            assert np.all(dE[x == IGN] == 0.0)
            assert (tot, skp) == (totk, skpk) == (2 * 4, 2 if eps else 0)
    # without compaction the units straddle the two valid blocks: other decisions
    _, dCu, totu, skpu = backward(E, C, x, 1.0, IGN, "mean", eps=2.0 ** -12, compact=False)
    assert totu == 3 * 4 and skpu != 2
    # and unfiltered, compaction changes nothing at all (up to the order in
    # which the blocked form's matrix products sum over differently cut blocks)
    a = backward(E, C, x, 1.0, IGN, "mean", eps=0.0)
    b = backward(E, C, x, 1.0, IGN, "mean", eps=0.0, compact=False)
    if impl == "loops":
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
    else:
        np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-18)
        np.testing.assert_allclose(a[1], b[1], rtol=1e-12, atol=1e-18)


def test_dC_columns_compaction():
    E, C, x, keep = _interleaved_ignores()
    V = C.shape[0]
    _, lse, _ = oracle.forward(E, C, x, IGN, "mean")
    blocks = list(range((V + 31) // 32))
    for compact in (True, False):
        _, dC, _, _ = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=2.0 ** -12, compact=compact)
        cols = oracle.dC_columns(E, C, x, lse, 1.0, IGN, "mean", eps=2.0 ** -12, blocks=blocks,
                                 compact=compact)
        for b in blocks:
            np.testing.assert_allclose(cols[b], dC[32 * b:32 * b + 32], rtol=1e-10,
                                       atol=1e-13 * np.abs(dC).max())


# ---- vocabulary sorting ("Cut Your Losses" digest, "Vocabulary Sorting") ----

def test_average_logits_brute_force():
    # Each entry's logit summed over the valid rows with plain Python loops and
    # divided by their count; an ignored row and a row whose target is outside
    # the vocabulary carry huge values and must not count.
    E, C, x = _rand(6, 7, 3, seed=41)
    E[2] = 1e6
    x[2] = IGN
    E[4] = -1e6
    x[4] = 7  # == V: outside the vocabulary
    want = []
    for v in range(7):
        tot, cnt = 0.0, 0
        for n in range(6):
            if x[n] == IGN or not 0 <= x[n] < 7:
                continue
            tot += sum(float(C[v, d]) * float(E[n, d]) for d in range(3))
            cnt += 1
        want.append(tot / cnt)
    np.testing.assert_allclose(oracle.average_logits(E, C, x, IGN), want, rtol=1e-12, atol=1e-12)
    x[:] = IGN  # no valid row: every average is 0 and the order is the identity
    assert np.all(oracle.average_logits(E, C, x, IGN) == 0.0)
    np.testing.assert_array_equal(oracle.vocab_order(E, C, x, IGN)[0], np.arange(7))


def test_vocab_order_closed_form():
    # C[v] = alpha_v u and every row has E[n] . u = 1 (plus a part orthogonal
    # to u), so the average logit of entry v is alpha_v: the order is the
    # alphas sorted downwards, the tie (entries 1 and 3) by ascending id.
    alpha = np.array([0.1, 3.0, -2.0, 3.0, 0.5, -0.25])
    u = np.array([0.6, 0.8, 0.0])
    r = np.random.default_rng(42)
    orth = r.standard_normal((5, 1)) * np.array([[0.8, -0.6, 0.0]]) + \
        r.standard_normal((5, 1)) * np.array([[0.0, 0.0, 1.0]])
    E = u[None, :] + orth
    C = alpha[:, None] * u[None, :]
    x = np.array([0, 5, 2, 2, 1], dtype=np.int64)
    order, a = oracle.vocab_order(E, C, x, IGN)
    np.testing.assert_allclose(a, alpha, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(order, [1, 3, 4, 0, 5, 2])


def test_sorted_backward_without_filter_is_the_backward():
    # With eps = 0 no unit is dropped, so the order of the vocabulary cannot
    # change dE or dC (a sum over entries, and dC row by row); a wrong target
    # remap or a wrong scatter of the dC rows fails this.  The identity order
    # is the plain backward bit for bit, also with the filter on.
    E, C, x = _rand(40, 70, 6, seed=43, ignore=(3, 17))
    perm = np.random.default_rng(44).permutation(70)
    base = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=0.0)
    got = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=0.0, vocab_order=perm)
    np.testing.assert_allclose(got[0], base[0], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(got[1], base[1], rtol=1e-10, atol=1e-15)
    assert got[2] == base[2] and got[3] == 0
    for eps in (0.0, 2.0 ** -12):
        a = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=eps)
        b = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=eps, vocab_order=np.arange(70))
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
        assert a[2:] == b[2:]
    with pytest.raises(AssertionError):
        oracle.backward(E, C, x, 1.0, IGN, "mean", vocab_order=np.zeros(70, dtype=np.int64))


def _sorting_case():
    """64 vocabulary entries, 32 tokens: even entries have logits near +10, odd
    ones near -10, so every even probability is about 1/32 and every odd one
    below 1e-9.  Targets are even.  In id order both 32-entry units mix the
    two kinds; sorted by average logit the evens fill the first unit and the
    odd ones the second, which the filter then drops."""
    r = np.random.default_rng(45)
    N, V = 32, 64
    E = np.stack([10.0 + 0.1 * r.standard_normal(N), r.standard_normal(N)], axis=1)
    sign = np.where(np.arange(V) % 2 == 0, 1.0, -1.0)
    C = np.stack([sign, 0.05 * r.standard_normal(V)], axis=1)
    x = (2 * r.integers(0, V // 2, size=N)).astype(np.int64)
    return E, C, x


def test_sorting_clusters_and_filters_the_constructed_case():
    # Reference: dense autograd (torch, fp64); the sorted filtered gradient is
    # the dense one without the odd entries' terms: dC rows of odd entries
    # exactly 0, the even rows dense, dE less G[:, odd] C[odd] / N.
    E, C, x = _sorting_case()
    N, V = E.shape[0], C.shape[0]
    eps = 2.0 ** -12
    order, _ = oracle.vocab_order(E, C, x, IGN)
    assert set(order[:32]) == set(range(0, V, 2))
    _, _, dE_ref, dC_ref = _torch_dense(E, C, x, "mean", np.array(1.0))
    G = torch.softmax(torch.tensor(E) @ torch.tensor(C).T, dim=1).numpy()
    G[np.arange(N), x] -= 1.0
    odd = np.arange(1, V, 2)
    plain = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=eps)
    dE, dC, tot, skp = oracle.backward(E, C, x, 1.0, IGN, "mean", eps=eps, vocab_order=order)
    assert tot == 2 and plain[3] == 0 and skp == 1
    tol = dict(rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(plain[0], dE_ref, **tol)
    np.testing.assert_allclose(dE, dE_ref - (G[:, odd] @ C[odd]) / N, **tol)
    assert np.all(dC[odd] == 0.0)
    np.testing.assert_allclose(dC[0::2], dC_ref[0::2], **tol)
    # dC_columns in the sorted order gives the same rows
    _, lse, _ = oracle.forward(E, C, x, IGN, "mean")
    cols = oracle.dC_columns(E, C, x, lse, 1.0, IGN, "mean", eps=eps, blocks=[0, 1],
                             vocab_order=order)
    np.testing.assert_allclose(cols[0], dC[order[:32]], rtol=1e-10, atol=1e-15)
    assert np.all(cols[1] == 0.0)
