"""GPU parity at the full sizes of the head-shaped workloads, through the same
C-ABI calls and launch configuration that bench.py times.

Three kinds of check, all against the fp64 oracle (its blocked form, fp64
matrix products per block of rows):

* full head shapes (Gemma-2-2B, Llama-3 long batch, GPT-OSS):
  - forward: lse and per-token loss of every row; the mean / sum output
    against the per-token one and the oracle's;
  - dE: whole filter-unit row blocks (32 consecutive valid rows; ignored rows
    are removed before the units are cut), filter off and on; every ignored
    row exactly zero;
  - dC: whole 32-row vocabulary blocks on both sides of every multiple of
    8192 (the backward's vocabulary chunks are 8192 or 16384 rows), a random
    block and the last block, against the oracle given its own lse of every
    row (the Llama long batch takes the tokens in eight blocks, so its dC is
    summed over them in the fp32 accumulator); the identity <dC, C> = <dE, E>
    and, unfiltered, sum_v dC_v = 0 (rows of G sum to zero);
* a full head's vocabulary and hidden size at token counts the oracle runs in
  full, compared element by element, filter off and on: the Qwen2.5-0.5B head
  itself (N = 4096, its dE tiles dealt over two parts of each chunk), the
  Llama width (D = 2048, V = 128,256, N = 2048, 5% ignored rows, tail
  targets) and the GPT-OSS width (D = 2880, V = 201,088, N = 2816, flat and
  peaked softmax);
* the "as written" generator (beta = 0.5 sqrt(D)) at all four head shapes:
  lse to 1e-5 absolute and loss to 1e-5 relative, every unit filtered and
  the filtered gradients exactly zero.

Tolerances: lse 1e-5 absolute, loss 1e-5 relative (relative L2 for reduction
none), dE / dC 3e-3 relative Frobenius, ignored rows exactly zero.
"""
import dataclasses
import time

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


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _row_scale(x, g, reduction):
    valid = x != IGN
    g = np.atleast_1d(np.asarray(g, dtype=np.float64))
    if reduction == "mean":
        return np.where(valid, g[0] / max(int(valid.sum()), 1), 0.0)
    if reduction == "sum":
        return np.where(valid, g[0], 0.0)
    return np.where(valid, g, 0.0)


def _run_gpu(E, C, x, reduction, grad, eps_list=(0.0, EPS)):
    """Forward (the workload's reduction and 'none'), then the backward per eps.
    dE / dC come back on the host; <dC, C>, <dE, E> and the dC column sums are
    formed on the device in float64."""
    lce = _lce()
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    loss, lse = lce.cce_forward(Ed, Cd, xd, IGN, reduction)
    loss_rows, _ = lce.cce_forward(Ed, Cd, xd, IGN, "none")
    gd = grad.to(DEV)
    out = {}
    for eps in eps_list:
        dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, gd, IGN, reduction, eps, with_stats=True)
        Ef, Cf = Ed.double(), Cd.double()
        dEf, dCf = dE.double(), dC.double()
        ident = ((dCf * Cf).sum().item(), (dEf * Ef).sum().item())
        colsum = (dCf.sum(0).norm().item(), dCf.abs().sum(0).norm().item())
        out[eps] = {"dE": dE.cpu(), "dC": dC.cpu(), "stats": st, "ident": ident,
                    "colsum": colsum}
        del Ef, Cf, dEf, dCf, dE, dC
    torch.cuda.synchronize()
    return (loss.cpu(), lse.cpu().double().numpy(), loss_rows.cpu().double().numpy(), out)


def _check_forward(w, xs, E64, C64, loss, lse, loss_rows, rows):
    valid = xs != IGN
    t0 = time.time()
    ref_loss, ref_lse, _ = oracle.forward_blocked(E64[rows], C64, xs[rows], IGN, "none")
    vr = valid[rows]
    err_lse = np.max(np.abs(lse[rows][vr] - ref_lse[vr])) if vr.any() else 0.0
    err_loss = _rel(loss_rows[rows], ref_loss)
    _log(f"{w.name}: lse max abs err {err_lse:.2e}, loss rel L2 {err_loss:.2e} over {rows.size} "
         f"rows (oracle {time.time() - t0:.0f}s)")
    assert err_lse <= 1e-5
    assert err_loss <= 1e-5
    assert np.all(loss_rows[~valid] == 0.0) and np.all(lse[~valid] == 0.0)
    if w.reduction in ("mean", "sum"):
        want = loss_rows[valid].sum() / (max(int(valid.sum()), 1) if w.reduction == "mean" else 1)
        assert abs(float(loss) - want) <= 1e-6 * abs(want)
        if rows.size == xs.size:  # the reduced loss against the oracle's
            ref = ref_loss[valid].sum() / (max(int(valid.sum()), 1) if w.reduction == "mean" else 1)
            assert abs(float(loss) - ref) <= 1e-5 * abs(ref), (float(loss), ref)
    return ref_lse, ref_loss


def _dE_blocks(xs, V, rng, count=6):
    """Filter-unit row blocks (32 consecutive valid rows): the first, the last,
    random ones and, when some target lies in the last 256 ids, the block of the
    first such row.  Returns (block ids, the valid rows in order)."""
    vidx = np.nonzero(xs != IGN)[0]
    nb = (vidx.size + 31) // 32
    blocks = {0, nb - 1} | {int(b) for b in rng.integers(0, nb, size=count)}
    tail = np.nonzero(xs >= V - 256)[0]
    if tail.size:
        blocks.add(int(np.searchsorted(vidx, tail[0])) // 32)
    return sorted(blocks), vidx


def _check_dE_blocks(w, xs, E64, C64, grad, out, rng):
    s = _row_scale(xs, grad.numpy(), w.reduction)
    blocks, vidx = _dE_blocks(xs, w.V, rng)
    refs = {0.0: [], EPS: []}
    for b in blocks:
        r = vidx[32 * b:32 * b + 32]
        res = oracle.backward_blocked(E64[r], C64, xs[r], s[r], IGN, "none", eps=[0.0, EPS])
        refs[0.0].append(res[0][0])
        refs[EPS].append(res[1][0])
    brow = np.concatenate([vidx[32 * b:32 * b + 32] for b in blocks])
    valid = torch.from_numpy(xs != IGN)
    for eps in (0.0, EPS):
        got = out[eps]["dE"][brow].double().numpy()
        err = _rel(got, np.concatenate(refs[eps]))
        _log(f"{w.name} eps={eps:g}: dE blocks {blocks} rel {err:.2e}")
        assert err <= 3e-3, (eps, err)
        assert torch.count_nonzero(out[eps]["dE"][~valid]).item() == 0
        st = out[eps]["stats"]
        assert st["units_total"] == ((vidx.size + 31) // 32) * ((w.V + 31) // 32)
        if eps == 0.0:
            assert st["units_skipped"] == 0


def _check_dC_properties(w, out):
    for eps in (0.0, EPS):
        a, b = out[eps]["ident"]
        _log(f"{w.name} eps={eps:g}: <dC,C> {a:.6e} <dE,E> {b:.6e} rel {abs(a - b) / abs(b):.2e}")
        assert abs(a - b) <= 2e-3 * abs(b), (eps, a, b)
    csum, cabs = out[0.0]["colsum"]
    _log(f"{w.name}: |sum_v dC_v| / |sum_v |dC_v|| = {csum / cabs:.2e}")
    assert csum <= 1e-3 * cabs, (csum, cabs)


def _check_dC_blocks(w, xs, E64, C64, grad, ref_lse_all, out, rng):
    """32-row vocabulary blocks of dC on both sides of every multiple of 8192,
    a random block and the last one, against the oracle with its own lse."""
    nvb = (w.V + 31) // 32
    vb = {nvb - 1, int(rng.integers(1, nvb - 1))}
    for c in range(8192, w.V, 8192):
        vb |= {c // 32 - 1, c // 32}
    vb = sorted(vb)
    for eps in (0.0, EPS):
        cols = oracle.dC_columns(E64, C64, xs, ref_lse_all, grad.numpy(), IGN, w.reduction,
                                 eps=eps, blocks=vb)
        ref = np.concatenate([cols[b] for b in vb])
        got = torch.cat([out[eps]["dC"][32 * b:32 * b + 32] for b in vb]).double().numpy()
        err = _rel(got, ref)
        _log(f"{w.name} eps={eps:g}: dC over {len(vb)} vocabulary blocks rel {err:.2e}")
        assert err <= 3e-3, (eps, err)


def _check_head(w):
    rng = np.random.default_rng(1000 + w.seed)
    t0 = time.time()
    E, C, x = si.generate(w)
    grad = si.upstream_grad(w, "random")
    _log(f"{w.name}: generated in {time.time() - t0:.0f}s; GPU run")
    loss, lse, loss_rows, out = _run_gpu(E, C, x, w.reduction, grad)
    xs = x.numpy()
    E64, C64 = E.double().numpy(), C.double().numpy()
    # every row's lse and loss (the dC blocks need the oracle's lse of every row)
    ref_lse, _ = _check_forward(w, xs, E64, C64, loss, lse, loss_rows, np.arange(w.N))
    _check_dE_blocks(w, xs, E64, C64, grad, out, rng)
    _check_dC_properties(w, out)
    _check_dC_blocks(w, xs, E64, C64, grad, ref_lse, out, rng)
    return out


def test_gemma_shape_full_size():
    out = _check_head(si.GEMMA)
    st = out[EPS]["stats"]
    assert 0.2 * st["units_total"] < st["units_skipped"] < 0.8 * st["units_total"]


def test_llama_shape_full_size_ignored_rows_and_tail_targets():
    out = _check_head(si.LLAMA)
    assert out[EPS]["stats"]["units_skipped"] > 0


def test_gpt_oss_shape_full_size_reduction_none():
    _check_head(si.GPTOSS)


# ---- full vocabulary and hidden size at token counts the oracle runs in full ----

REDUCED = [
    # the Qwen2.5-0.5B head itself (its N is small enough to compare in full):
    # 16 x 4 dE tiles per chunk, each dealt over two parts of the chunk
    si.QWEN,
    # the Llama head's width: 8 x 8 tiles of dE per chunk, 4 x 8 grouped tile order
    si.Workload("llama3-width-n2048", 2048, 128256, 2048, ignore_rows=102, tail_targets=64,
                tail_width=256, seed=31),
    # the GPT-OSS head's width, flat softmax, per-token loss (reduction none)
    si.Workload("gpt-oss-width-n2816", 2816, 201088, 2880, logit_std=1.0, reduction="none",
                seed=32),
    # the GPT-OSS width with a peaked softmax (most units kept)
    si.Workload("gpt-oss-width-peaked-n2816", 2816, 201088, 2880, seed=33),
]


# dC / dE walk their tiles in strips of S d-panels, S = 4, 3, 2 or 1 by
# what divides D_pad / 256 (the heads above take S = 4); widths with S = 3
# (the Gemma-2-2B width, 9 d-panels: 99 dE tiles per chunk, unsplit), 1 (5
# d-panels) and 2 (10 d-panels; these two few enough dE tiles to be dealt over
# parts), several token tiles and vocabulary chunks each, compared in full
STRIPS = [
    si.Workload("width-2304-n2816", 2816, 20000, 2304, seed=34),
    si.Workload("width-1280-n600", 600, 12000, 1280, ignore_rows=30, seed=35),
    si.Workload("width-2560-n520", 520, 9500, 2560, logit_std=3.0, seed=36),
]


@pytest.mark.parametrize("w", REDUCED, ids=[w.name for w in REDUCED])
def test_full_vocabulary_reduced_tokens_compared_in_full(w):
    _compare_in_full(w)


@pytest.mark.parametrize("w", STRIPS, ids=[w.name for w in STRIPS])
def test_every_strip_width_compared_in_full(w):
    _compare_in_full(w)


def _compare_in_full(w):
    t0 = time.time()
    E, C, x = si.generate(w)
    grad = si.upstream_grad(w, "random")
    loss, lse, loss_rows, out = _run_gpu(E, C, x, w.reduction, grad)
    xs = x.numpy()
    valid = xs != IGN
    E64, C64 = E.double().numpy(), C.double().numpy()
    _log(f"{w.name}: GPU done in {time.time() - t0:.0f}s; oracle forward")
    _check_forward(w, xs, E64, C64, loss, lse, loss_rows, np.arange(w.N))
    t1 = time.time()
    refs = oracle.backward_blocked(E64, C64, xs, grad.numpy(), IGN, w.reduction, eps=[0.0, EPS])
    _log(f"{w.name}: oracle backward {time.time() - t1:.0f}s")
    for eps, (ref_dE, ref_dC, tot, skp) in zip((0.0, EPS), refs):
        got_dE = out[eps]["dE"].double().numpy()
        got_dC = out[eps]["dC"].double().numpy()
        eE, eC = _rel(got_dE, ref_dE), _rel(got_dC, ref_dC)
        st = out[eps]["stats"]
        _log(f"{w.name} eps={eps:g}: dE rel {eE:.2e} dC rel {eC:.2e}; units skipped "
             f"{st['units_skipped']} (oracle {skp}) of {tot}")
        assert eE <= 3e-3 and eC <= 3e-3, (eps, eE, eC)
        assert np.all(got_dE[~valid] == 0.0)
        assert st["units_total"] == tot
        assert abs(st["units_skipped"] - skp) <= max(2, 0.002 * tot), (st, skp)
        # the worst 32-row vocabulary block of dC: no tile is wrong or missing
        nvb = (w.V + 31) // 32
        pad = np.zeros((nvb * 32 - w.V, w.D))
        dG = np.concatenate([got_dC - ref_dC, pad]).reshape(nvb, 32, w.D)
        nR = np.concatenate([ref_dC, pad]).reshape(nvb, 32, w.D)
        per = np.linalg.norm(dG, axis=(1, 2)) / np.maximum(np.linalg.norm(nR, axis=(1, 2)),
                                                             1e-30)
        big = np.linalg.norm(nR, axis=(1, 2)) > 1e-3 * np.linalg.norm(ref_dC) / np.sqrt(nvb)
        _log(f"{w.name} eps={eps:g}: worst dC vocabulary block rel {per[big].max():.2e}")
        if eps == 0.0:  # with the filter, units decided apart by fp32 rounding move small blocks
            assert per[big].max() <= 1e-2


# ---- the literal ("as written") generator: beta = 0.5 sqrt(D) ----

AS_WRITTEN = [dataclasses.replace(w, name=w.name + "-as-written", beta=None)
              for w in (si.QWEN, si.GEMMA, si.LLAMA, si.GPTOSS)]


@pytest.mark.parametrize("w", AS_WRITTEN, ids=[w.name for w in AS_WRITTEN])
def test_as_written_generator(w):
    # The literal E recipe puts the target 15-27 logit standard deviations
    # above the rest: loss 1e-15 .. 1e-3, lse 24 .. 64, and nearly every unit
    # below eps.  lse and loss of every row against the oracle; the units that
    # can survive the filter lie in rows whose 1 - p_target >= eps, i.e. loss
    # >= -log(1 - eps) ~ eps, so the oracle's backward over the 32-row unit
    # blocks holding a row with loss >= 1e-4 gives every nonzero gradient.
    E, C, x = si.generate(w)
    grad = si.upstream_grad(w, "random")
    loss, lse, loss_rows, out = _run_gpu(E, C, x, w.reduction, grad, eps_list=(EPS,))
    xs = x.numpy()
    E64, C64 = E.double().numpy(), C.double().numpy()
    ref_lse_all_rows, ref_loss = _check_forward(w, xs, E64, C64, loss, lse, loss_rows,
                                                np.arange(w.N))
    vidx = np.nonzero(xs != IGN)[0]
    nb = (vidx.size + 31) // 32
    cand = [b for b in range(nb) if np.max(ref_loss[vidx[32 * b:32 * b + 32]]) >= 1e-4]
    st = out[EPS]["stats"]
    dE, dC = out[EPS]["dE"], out[EPS]["dC"]
    _log(f"{w.name}: units skipped {st['units_skipped']} of {st['units_total']}; "
         f"{len(cand)} row blocks may keep units")
    if not cand:
        assert st["units_skipped"] == st["units_total"]
        assert torch.count_nonzero(dE).item() == 0 and torch.count_nonzero(dC).item() == 0
        return
    rows = np.concatenate([vidx[32 * b:32 * b + 32] for b in cand])
    s = _row_scale(xs, grad.numpy(), w.reduction)
    ref_dE, ref_dC, tot, skp = oracle.backward_blocked(E64[rows], C64, xs[rows], s[rows], IGN,
                                                       "none", eps=EPS)
    kept = tot - skp
    _log(f"{w.name}: oracle keeps {kept} units in those blocks")
    assert abs((st["units_total"] - st["units_skipped"]) - kept) <= 2
    others = np.setdiff1d(np.arange(w.N), rows)
    assert torch.count_nonzero(dE[torch.from_numpy(others)]).item() == 0
    if kept:
        # The backward gets lse in fp32: at the target entry G = p_t - 1 carries
        # the rounding of lse (|d lse| <= 2^-24 |lse|) as an absolute error,
        # which is large next to 1 - p_t ~ eps in these rows.  Bound: 3e-3
        # relative plus, per row, s_n 2^-23 |lse_n| |C[x_n]| in dE and the
        # sum of s_n 2^-23 |lse_n| |E_n| over the rows in dC.
        lse_r = np.abs(ref_lse_all_rows[rows])
        # only rows whose target unit can pass the filter (1 - p_t near eps or above)
        near = -np.expm1(-ref_loss[rows]) >= 0.5 * EPS
        t_err = np.where(near, s[rows] * 2.0 ** -23 * lse_r, 0.0)
        bE = np.sqrt(np.sum((t_err * np.linalg.norm(C64[xs[rows]], axis=1)) ** 2))
        bC = np.sum(t_err * np.linalg.norm(E64[rows], axis=1))
        dEg = dE[torch.from_numpy(rows)].double().numpy()
        aE = np.linalg.norm(dEg - ref_dE)
        aC = np.linalg.norm(dC.double().numpy() - ref_dC)
        nE, nC = np.linalg.norm(ref_dE), np.linalg.norm(ref_dC)
        _log(f"{w.name}: dE rel {aE / nE:.2e} (bound {(3e-3 * nE + bE) / nE:.2e}), dC rel "
             f"{aC / nC:.2e} (bound {(3e-3 * nC + bC) / nC:.2e}) on the blocks that keep units")
        assert aE <= 3e-3 * nE + bE and aC <= 3e-3 * nC + bC


def test_filter_variants_full_size():
    # FullC / FullE at the Qwen2.5-0.5B shape with 5% ignored rows, through the
    # same entry point bench.py times: the unfiltered contraction equals the
    # eps = 0 call and the filtered one the basic call, bit for bit (the G-hat
    # values do not depend on the mode; only which units each contraction keeps)
    lce = _lce()
    w = dataclasses.replace(si.QWEN, ignore_rows=205)
    E, C, x = si.generate(w)
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    gd = si.upstream_grad(w).to(DEV)
    _, lse = lce.cce_forward(Ed, Cd, xd, IGN, w.reduction)
    runs = {}
    for eps, mode in ((0.0, "both"), (EPS, "both"), (EPS, "full_c"), (EPS, "full_e")):
        dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, gd, IGN, w.reduction, eps,
                                      with_stats=True, filter_mode=mode)
        runs[(eps, mode)] = (dE, dC, st)
    torch.cuda.synchronize()
    full, basic = runs[(0.0, "both")], runs[(EPS, "both")]
    c, e = runs[(EPS, "full_c")], runs[(EPS, "full_e")]
    assert torch.equal(c[1], full[1]) and torch.equal(c[0], basic[0])
    assert torch.equal(e[0], full[0]) and torch.equal(e[1], basic[1])
    assert not torch.equal(basic[1], full[1]) and not torch.equal(basic[0], full[0])
    for r in (basic, c, e):
        assert r[2]["units_skipped"] == basic[2]["units_skipped"] > 0
    valid = torch.from_numpy((x != IGN).numpy()).to(DEV)
    assert torch.count_nonzero(c[0][~valid]).item() == 0
