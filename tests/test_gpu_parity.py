"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: loss 1e-5 relative (mean / sum) or 1e-5 relative L2 (none), lse
1e-5 absolute on valid rows, dE and dC 3e-3 relative Frobenius (bf16 outputs),
ignored rows exactly zero.  Filter-on runs are compared with the oracle
applying the same eps and the same 32 x 32 unit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

IGN = -100
EPS = 2.0 ** -12
DEV = "cuda:0"


def _lce():
    import linear_cross_entropy_amd as lce
    return lce


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _run(E, C, x, reduction, eps, grad=None, stats=False, filter_mode="both"):
    lce = _lce()
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    loss, lse = lce.cce_forward(Ed, Cd, xd, IGN, reduction)
    if grad is None:
        grad = torch.ones(()) if reduction != "none" else torch.ones(E.shape[0])
    out = lce.cce_backward(Ed, Cd, xd, lse, grad.to(DEV), IGN, reduction, eps, with_stats=stats,
                           filter_mode=filter_mode)
    torch.cuda.synchronize()
    res = {"loss": loss.cpu().double().numpy(), "lse": lse.cpu().double().numpy(),
           "dE": out[0].cpu().double().numpy(), "dC": out[1].cpu().double().numpy()}
    if stats:
        res["stats"] = out[2]
    return res


def _check_full(w, eps, grad=None, tol_grad=3e-3, filter_mode="both"):
    E, C, x = si.generate(w)
    g = grad if grad is not None else si.upstream_grad(w, "random")
    got = _run(E, C, x, w.reduction, eps, g, stats=True, filter_mode=filter_mode)
    E64, C64, x64 = E.double().numpy(), C.double().numpy(), x.numpy()
    ref_loss, ref_lse, nv = oracle.forward(E64, C64, x64, IGN, w.reduction)
    ref_dE, ref_dC, tot, skp = oracle.backward(E64, C64, x64, g.double().numpy(), IGN,
                                               w.reduction, eps=eps, filter_mode=filter_mode)
    valid = x64 != IGN
    if w.reduction == "none":
        assert _rel(got["loss"], ref_loss) <= 1e-5
        assert np.all(got["loss"][~valid] == 0.0)
    else:
        assert abs(float(got["loss"]) - ref_loss) <= 1e-5 * abs(ref_loss), (got["loss"], ref_loss)
    if valid.any():
        assert np.max(np.abs(got["lse"][valid] - ref_lse[valid])) <= 1e-5
    assert _rel(got["dE"], ref_dE) <= tol_grad, _rel(got["dE"], ref_dE)
    assert _rel(got["dC"], ref_dC) <= tol_grad, _rel(got["dC"], ref_dC)
    assert np.all(got["dE"][~valid] == 0.0)
    st = got["stats"]
    assert st["units_total"] == tot and st["unit_rows"] == 32 and st["unit_cols"] == 32
    if eps == 0:
        assert st["units_skipped"] == 0
    else:
        # decisions at |G| within fp32 rounding of eps may differ (fp32 vs fp64)
        assert abs(st["units_skipped"] - skp) <= max(2, 0.002 * tot), (st, skp)
    return got, st


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_tiny_config(eps):
    _check_full(si.TINY, eps)


# the smallest shapes the ABI takes: one token, a vocabulary shorter than one
# 256-row tile (the forward's ragged slab alone, one partial chunk), D = 8
# (one 16-byte chunk of K), and a vocabulary one row past a tile
SMALLEST = [(1, 7, 8, "mean"), (5, 100, 8, "none"), (3, 257, 24, "sum"), (300, 255, 16, "mean")]


@pytest.mark.parametrize("shape", SMALLEST, ids=[f"N{n}-V{v}-D{d}" for n, v, d, _ in SMALLEST])
@pytest.mark.parametrize("eps", [0.0, EPS])
def test_smallest_shapes(shape, eps):
    N, V, D, reduction = shape
    w = si.Workload("smallest", N, V, D, kind="tiny", reduction=reduction, seed=28)
    _check_full(w, eps)


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_ragged_every_dimension(reduction):
    # N, V not multiples of any tile; D % 64 != 0 exercises the K tail
    w = si.Workload("ragged", 300, 3001, 136, kind="tiny", ignore_rows=9,
                    reduction=reduction, seed=21)
    _check_full(w, 0.0)


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_multi_chunk_peaked(eps):
    # V spans three backward chunks (8192 rows at this N x D, the last ragged)
    # with targets in the tail; logit std 5 leaves about 30% of the units below eps
    w = si.Workload("multichunk", 200, 20000, 128, logit_std=5.0, ignore_rows=10,
                    tail_targets=20, tail_width=300, seed=22)
    got, st = _check_full(w, eps)
    if eps:
        assert st["units_skipped"] > 0


def test_filter_skips_and_matches_same_rule_oracle():
    # a confident softmax (large logit std) leaves many 32x32 units below 2^-12
    w = si.Workload("confident", 256, 9000, 64, logit_std=6.0, seed=23)
    got, st = _check_full(w, EPS)
    assert st["units_skipped"] > 0.2 * st["units_total"]


@pytest.mark.parametrize("mode", ["full_c", "full_e"])
def test_filter_variants(mode):
    # FullC / FullE ("Cut Your Losses" digest, "Numerical Stability Variants"):
    # against the oracle applying the same rule, on a confident softmax over
    # three backward chunks (the last ragged) with ignored rows.  The
    # unfiltered contraction equals the eps = 0 run bit for bit and the
    # filtered one the basic (both filtered) run: the G-hat values do not
    # depend on the mode, only which units each contraction keeps.
    w = si.Workload("variant", 200, 20000, 128, logit_std=6.0, ignore_rows=10,
                    tail_targets=20, tail_width=300, seed=24)
    got, st = _check_full(w, EPS, filter_mode=mode)
    assert st["units_skipped"] > 0.2 * st["units_total"]
    E, C, x = si.generate(w)
    g = si.upstream_grad(w, "random")
    full = _run(E, C, x, w.reduction, 0.0, g)
    both = _run(E, C, x, w.reduction, EPS, g)
    same_full, same_filtered = ("dC", "dE") if mode == "full_c" else ("dE", "dC")
    np.testing.assert_array_equal(got[same_full], full[same_full])
    np.testing.assert_array_equal(got[same_filtered], both[same_filtered])
    assert not np.array_equal(both[same_full], full[same_full])


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_compaction_many_ignored_rows(eps):
    # 70% of the rows ignored at random positions, three backward chunks, per-row
    # upstream gradients: against the oracle (units of 32 consecutive valid
    # rows), and bit for bit against the same call on the batch that holds only
    # the valid rows (ignored rows are removed before any tile runs, so every
    # tile sees the same rows in the same order)
    w = si.Workload("sparse", 700, 20000, 128, logit_std=3.0, ignore_rows=490,
                    tail_targets=20, tail_width=300, reduction="none", seed=28)
    got, st = _check_full(w, eps)
    E, C, x = si.generate(w)
    g = si.upstream_grad(w, "random")
    valid = (x != IGN).numpy()
    assert st["units_total"] == ((int(valid.sum()) + 31) // 32) * ((w.V + 31) // 32)
    vt = torch.from_numpy(valid)
    sub = _run(E[vt], C, x[vt], "none", eps, g[vt])
    full = _run(E, C, x, "none", eps, g)
    for k in ("loss", "lse", "dE"):
        np.testing.assert_array_equal(full[k][valid], sub[k])
        assert np.all(full[k][~valid] == 0.0)
    np.testing.assert_array_equal(full["dC"], sub["dC"])


def test_masking_and_empty():
    lce = _lce()
    w = si.Workload("mask", 64, 500, 64, kind="tiny", seed=24)
    E, C, x = si.generate(w)
    xm = torch.full_like(x, IGN)
    for red in ("mean", "sum"):
        got = _run(E, C, xm, red, EPS)
        assert float(got["loss"]) == 0.0
        assert np.all(got["dE"] == 0.0) and np.all(got["dC"] == 0.0)
    got = _run(E, C, xm, "none", EPS)
    assert np.all(got["loss"] == 0.0) and np.all(got["lse"] == 0.0)
    # scaling an ignored row's E changes nothing
    x2 = x.clone()
    x2[[0, 5]] = IGN
    E2 = E.clone()
    E2[[0, 5]] = (E2[[0, 5]].float() * 100).bfloat16()
    a = _run(E, C, x2, "mean", 0.0)
    b = _run(E2, C, x2, "mean", 0.0)
    assert np.array_equal(a["loss"], b["loss"]) and np.array_equal(a["dC"], b["dC"])
    # ... nor do non-finite values there: ignored rows never enter the arithmetic
    E3 = E.clone()
    E3[0] = float("inf")
    E3[5] = float("nan")
    c = _run(E3, C, x2, "mean", EPS)
    d = _run(E, C, x2, "mean", EPS)
    for k in ("loss", "lse", "dE", "dC"):
        assert np.array_equal(c[k], d[k]), k
    # empty batch
    E0 = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    x0 = torch.zeros(0, dtype=torch.int64, device=DEV)
    Cd = C.to(DEV)
    loss, lse = lce.cce_forward(E0, Cd, x0, IGN, "mean")
    dE, dC = lce.cce_backward(E0, Cd, x0, lse, torch.ones((), device=DEV), IGN, "mean", EPS)
    torch.cuda.synchronize()
    assert float(loss) == 0.0 and dE.shape == (0, 64)
    assert torch.count_nonzero(dC).item() == 0


def test_E_zero_closed_form_on_gpu():
    V = 2048
    _, C, x = si.generate(si.Workload("z", 128, V, 64, kind="tiny", seed=25))
    E = torch.zeros(128, 64, dtype=torch.bfloat16)
    got = _run(E, C, x, "none", 0.0)
    assert np.max(np.abs(got["lse"] - math.log(V))) <= 2e-6
    assert np.max(np.abs(got["loss"] - math.log(V))) <= 2e-6
    assert np.all(got["dC"] == 0.0)


def test_bitwise_repeatable():
    w = si.Workload("rep", 300, 9000, 192, logit_std=3.0, ignore_rows=5, seed=26)
    E, C, x = si.generate(w)
    a = _run(E, C, x, "mean", EPS)
    b = _run(E, C, x, "mean", EPS)
    for k in ("loss", "lse", "dE", "dC"):
        assert np.array_equal(a[k], b[k]), k


def test_autograd_wrapper_and_profiler():
    lce = _lce()
    w = si.Workload("ag", 128, 4000, 64, kind="tiny", seed=27)
    E, C, x = si.generate(w)
    Ed = E.to(DEV).requires_grad_(True)
    Cd = C.to(DEV).requires_grad_(True)
    lce.profile_enable(True)
    loss = lce.linear_cross_entropy(Ed, Cd, x.to(DEV), filter_eps=0.0)
    loss.backward()
    torch.cuda.synchronize()
    n, ms = lce.profile_query("fwd_lse")
    assert n in (1, 2) and ms > 0  # V = 4000 is ragged: the last slab has its own launch
    n, ms = lce.profile_query("target")
    assert n == 2  # the forward's target logits and the backward's
    n, ms = lce.profile_query("bwd_step")
    assert n >= 1
    lce.profile_enable(False)
    E64, C64, x64 = E.double().numpy(), C.double().numpy(), x.numpy()
    ref_dE, ref_dC, _, _ = oracle.backward(E64, C64, x64, 1.0, IGN, "mean", eps=0.0)
    assert _rel(Ed.grad.double().cpu().numpy(), ref_dE) <= 3e-3
    assert _rel(Cd.grad.double().cpu().numpy(), ref_dC) <= 3e-3


def test_role_split_profile_mode_gives_the_same_results():
    # cce_profile_enable(2) runs each role of the backward step in a launch of
    # its own: the same tiles, so the same bits as the fused launch
    lce = _lce()
    w = si.Workload("roles", 600, 30000, 320, logit_std=3.0, ignore_rows=9, seed=29)
    E, C, x = si.generate(w)
    fused = _run(E, C, x, "mean", EPS)
    lce.profile_enable(True, roles=True)
    split = _run(E, C, x, "mean", EPS)
    counts = {f: lce.profile_query(f)[0] for f in ("bwd_step", "bwd_de", "bwd_dc", "bwd_g", "bwd_t")}
    lce.profile_enable(False)
    for k in ("loss", "lse", "dE", "dC"):
        assert np.array_equal(fused[k], split[k]), k
    # 30000 rows: 4 chunks of 8192, so 5 launches of the step, each role in 4 of them
    assert counts == {"bwd_step": 0, "bwd_de": 4, "bwd_dc": 4, "bwd_g": 4, "bwd_t": 4}, counts


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_upstream_gradients_over_eight_decades(eps):
    # reduction none with per-token upstream gradients spread log-uniformly over
    # 1e-8 .. 1, plus zeros: every row's dE against the oracle's row, relative
    # to that row (how precisely G enters dE must not depend on the row's
    # weight), rows with a zero weight exactly zero, dC as a whole
    w = si.Workload("spread", 300, 20000, 128, logit_std=3.0, ignore_rows=10, tail_targets=20,
                    tail_width=300, reduction="none", seed=29)
    E, C, x = si.generate(w)
    r = np.random.default_rng(5)
    g = (10.0 ** r.uniform(-8.0, 0.0, size=w.N)).astype(np.float32)
    g[r.choice(w.N, 15, replace=False)] = 0.0
    gt = torch.from_numpy(g)
    got = _run(E, C, x, "none", eps, gt)
    E64, C64, x64 = E.double().numpy(), C.double().numpy(), x.numpy()
    ref_dE, ref_dC, _, _ = oracle.backward(E64, C64, x64, g.astype(np.float64), IGN, "none",
                                           eps=eps)
    valid = x64 != IGN
    live = valid & (g > 0)
    num = np.linalg.norm(got["dE"][live] - ref_dE[live], axis=1)
    den = np.linalg.norm(ref_dE[live], axis=1)
    # Besides 3e-3, a row carries the fp32 rounding of its lse (the backward's
    # input): G at the target is p_t - 1 with |d lse| <= 2^-24 |lse|, which is
    # large next to 1 - p_t in rows whose target is nearly certain.
    _, ref_lse, _ = oracle.forward(E64, C64, x64, IGN, "none")
    lse_term = (2.0 ** -23 * np.abs(ref_lse[live]) * g[live] *
                np.linalg.norm(C64[x64[live]], axis=1) / den)
    worst = np.max(num / den)
    ratio = np.max(num / den / (3e-3 + lse_term))
    print(f"spread eps={eps:g}: worst per-row dE rel {worst:.2e} over {live.sum()} rows "
          f"(weights {g[live].min():.1e} .. {g[live].max():.1e}); worst error / bound {ratio:.2f}",
          flush=True)
    assert ratio <= 1.0
    assert np.all(got["dE"][~live] == 0.0)
    assert _rel(got["dC"], ref_dC) <= 3e-3
