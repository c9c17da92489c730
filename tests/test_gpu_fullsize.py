"""GPU parity at the full sizes of the head-shaped workloads (Qwen2.5-0.5B,
Gemma-2-2B, Llama-3 long batch, GPT-OSS head shapes), through the same C-ABI
calls and launch configuration that bench.py times.

The fp64 oracle cannot run the whole backward at these sizes, so:

* forward: lse and per-token loss of sampled rows (first, last, random,
  ignored and vocabulary-tail-target rows) against the oracle run on those
  rows with the full vocabulary; the mean / sum output against the mean / sum
  of the per-token output;
* dE: whole filter-unit row blocks (32 consecutive valid rows; ignored rows
  are removed before the units are cut) against the oracle's backward on
  those rows with the same per-row scale, filter off and on; every ignored
  row exactly zero;
* dC: the identity <dC, C> = <dE, E> (both sides equal sum_n s_n sum_v G A,
  filtered or not) and, unfiltered, sum_v dC_v = 0 (rows of G sum to zero);
  at the Qwen shape also whole 32-row vocabulary blocks of dC against the
  oracle (its lse from a full fp64 forward);
* the "as written" generator (beta = 0.5 sqrt(D)): lse / loss with an
  absolute bound, every unit filtered, gradients exactly zero with the filter.

Tolerances are those of the parity tests: lse 1e-5 absolute, loss 1e-5
relative L2, dE / dC 3e-3 relative Frobenius, ignored rows exactly zero.
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


def _lce():
    import linear_cross_entropy_amd as lce
    return lce


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _sample_rows(x, rng):
    N = x.shape[0]
    rows = set(range(16)) | set(range(N - 16, N))
    rows |= set(rng.choice(N, size=32, replace=False).tolist())
    ign = np.nonzero(x == IGN)[0]
    rows |= set(ign[:8].tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _dE_blocks(x, V, rng, tail_width=256):
    """Filter-unit row blocks (32 consecutive valid rows: ignored rows are
    removed before the units are cut): a random one, the last one, and (when
    some target lies in the vocabulary tail) the block of the first such row.
    Returns (block ids, the valid rows in order)."""
    vidx = np.nonzero(x != IGN)[0]
    nb = (vidx.size + 31) // 32
    blocks = {int(rng.integers(0, nb)), nb - 1}
    tail = np.nonzero(x >= V - tail_width)[0]
    if tail.size:
        blocks.add(int(np.searchsorted(vidx, tail[0])) // 32)
    return sorted(blocks), vidx


def _row_scale(x, g, reduction):
    valid = x != IGN
    g = np.atleast_1d(np.asarray(g, dtype=np.float64))
    if reduction == "mean":
        return np.where(valid, g[0] / max(int(valid.sum()), 1), 0.0)
    if reduction == "sum":
        return np.where(valid, g[0], 0.0)
    return np.where(valid, g, 0.0)


def _run_gpu(E, C, x, reduction, grad):
    lce = _lce()
    Ed, Cd, xd = E.to(DEV), C.to(DEV), x.to(DEV)
    loss, lse = lce.cce_forward(Ed, Cd, xd, IGN, reduction)
    loss_rows, _ = lce.cce_forward(Ed, Cd, xd, IGN, "none")
    gd = grad.to(DEV)
    out = {}
    for eps in (0.0, EPS):
        dE, dC, st = lce.cce_backward(Ed, Cd, xd, lse, gd, IGN, reduction, eps, with_stats=True)
        # dC properties on the device, in float64
        Ef, Cf = Ed.double(), Cd.double()
        dEf, dCf = dE.double(), dC.double()
        ident = ((dCf * Cf).sum().item(), (dEf * Ef).sum().item())
        colsum = (dCf.sum(0).norm().item(), dCf.abs().sum(0).norm().item())
        out[eps] = {"dE": dE.cpu(), "dC": dC, "stats": st, "ident": ident, "colsum": colsum}
        del Ef, Cf, dEf, dCf
    torch.cuda.synchronize()
    return loss.cpu(), lse.cpu().double().numpy(), loss_rows.cpu().double().numpy(), out


def _check_workload(w, dC_blocks=False):
    rng = np.random.default_rng(1000 + w.seed)
    E, C, x = si.generate(w)
    grad = si.upstream_grad(w, "random")
    loss, lse, loss_rows, out = _run_gpu(E, C, x, w.reduction, grad)
    xs = x.numpy()
    valid = xs != IGN
    C64 = C.double().numpy()

    # forward: sampled rows against the oracle, with the full vocabulary
    rows = _sample_rows(xs, rng)
    E_rows = E[rows].double().numpy()
    ref_loss, ref_lse, _ = oracle.forward(E_rows, C64, xs[rows], IGN, "none")
    vr = xs[rows] != IGN
    print(f"{w.name}: lse max abs err {np.max(np.abs(lse[rows][vr] - ref_lse[vr])):.2e}, "
          f"loss rel {_rel(loss_rows[rows], ref_loss):.2e} over {rows.size} rows", flush=True)
    assert np.max(np.abs(lse[rows][vr] - ref_lse[vr])) <= 1e-5
    assert _rel(loss_rows[rows], ref_loss) <= 1e-5
    assert np.all(loss_rows[~valid] == 0.0) and np.all(lse[~valid] == 0.0)
    if w.reduction == "mean":
        want = loss_rows[valid].sum() / max(int(valid.sum()), 1)
        assert abs(float(loss) - want) <= 1e-6 * abs(want)
    elif w.reduction == "sum":
        want = loss_rows[valid].sum()
        assert abs(float(loss) - want) <= 1e-6 * abs(want)

    # dE: whole 32-row blocks against the oracle's backward on those rows
    s = _row_scale(xs, grad.numpy(), w.reduction)
    blocks, vidx = _dE_blocks(xs, w.V, rng, w.tail_width)
    brow = np.concatenate([vidx[32 * b:32 * b + 32] for b in blocks])
    E_blk = E[brow].double().numpy()
    for eps in (0.0, EPS):
        ref_dE = np.zeros((brow.size, w.D))
        # each unit's rows separately, so the oracle's filter units line up with the GPU's
        o = 0
        for b in blocks:
            r = slice(o, o + vidx[32 * b:32 * b + 32].size)
            o = r.stop
            ref_dE[r] = oracle.backward(E_blk[r], C64, xs[brow][r], s[brow][r], IGN, "none",
                                        eps=eps)[0]
        got = out[eps]["dE"][brow].double().numpy()
        print(f"{w.name} eps={eps:g}: dE blocks {blocks} rel {_rel(got, ref_dE):.2e}", flush=True)
        assert _rel(got, ref_dE) <= 3e-3, (eps, _rel(got, ref_dE))
        assert torch.count_nonzero(out[eps]["dE"][torch.from_numpy(~valid)]).item() == 0
        st = out[eps]["stats"]
        assert st["units_total"] == ((vidx.size + 31) // 32) * ((w.V + 31) // 32)
        if eps == 0.0:
            assert st["units_skipped"] == 0

    # dC: properties that hold at any size
    for eps in (0.0, EPS):
        a, b = out[eps]["ident"]
        print(f"{w.name} eps={eps:g}: <dC,C> {a:.6e} <dE,E> {b:.6e} rel {abs(a - b) / abs(b):.2e}",
              flush=True)
        assert abs(a - b) <= 2e-3 * abs(b), (eps, a, b)
    csum, cabs = out[0.0]["colsum"]
    print(f"{w.name}: |sum_v dC_v| / |sum_v |dC_v|| = {csum / cabs:.2e}", flush=True)
    assert csum <= 1e-3 * cabs, (csum, cabs)

    if dC_blocks:
        # whole 32-row vocabulary blocks of dC against the oracle (full fp64 forward for lse)
        _, lse_all, _ = oracle.forward(E.double().numpy(), C64, xs, IGN, w.reduction)
        vb = [0, 1, int(rng.integers(2, (w.V + 31) // 32 - 1)), (w.V + 31) // 32 - 1]
        for eps in (0.0, EPS):
            cols = oracle.dC_columns(E.double().numpy(), C64, xs, lse_all, grad.numpy(), IGN,
                                     w.reduction, eps=eps, blocks=vb)
            ref = np.concatenate([cols[b] for b in vb])
            got = torch.cat([out[eps]["dC"][32 * b:32 * b + 32] for b in vb]).double().cpu().numpy()
            print(f"{w.name} eps={eps:g}: dC vocab blocks {vb} rel {_rel(got, ref):.2e}", flush=True)
            assert _rel(got, ref) <= 3e-3, (eps, _rel(got, ref))
    return out


def test_qwen_shape_full_size():
    _check_workload(si.QWEN, dC_blocks=True)


def test_gemma_shape_full_size():
    out = _check_workload(si.GEMMA)
    st = out[EPS]["stats"]
    assert 0.2 * st["units_total"] < st["units_skipped"] < 0.8 * st["units_total"]


def test_llama_shape_full_size_ignored_rows_and_tail_targets():
    out = _check_workload(si.LLAMA)
    assert out[EPS]["stats"]["units_skipped"] > 0


def test_gpt_oss_shape_full_size_reduction_none():
    _check_workload(si.GPTOSS)


def test_as_written_generator_is_degenerate():
    # the literal E recipe (beta = 0.5 sqrt(D)): loss ~ 0, every unit below eps
    w = si.Workload("qwen-as-written", 4096, 151936, 896, beta=None, seed=1)
    rng = np.random.default_rng(7)
    E, C, x = si.generate(w)
    grad = si.upstream_grad(w)
    loss, lse, loss_rows, out = _run_gpu(E, C, x, w.reduction, grad)
    xs = x.numpy()
    rows = _sample_rows(xs, rng)
    ref_loss, ref_lse, _ = oracle.forward(E[rows].double().numpy(), C.double().numpy(), xs[rows],
                                          IGN, "none")
    # lse is large here (the target logit dominates): fp32 logits carry ~1e-6 relative error
    assert np.max(np.abs(lse[rows] - ref_lse) / np.maximum(1.0, np.abs(ref_lse))) <= 1e-5
    assert np.max(np.abs(loss_rows[rows] - ref_loss)) <= 1e-5 * np.max(np.abs(ref_lse))
    st = out[EPS]["stats"]
    assert st["units_skipped"] == st["units_total"]
    assert torch.count_nonzero(out[EPS]["dE"]).item() == 0
    assert torch.count_nonzero(out[EPS]["dC"]).item() == 0


def test_filter_variants_full_size():
    # FullC / FullE at the Qwen2.5-0.5B shape with 5% ignored rows, through the
    # same entry point bench.py times: the unfiltered contraction equals the
    # eps = 0 call and the filtered one the basic call, bit for bit (the G-hat
    # values do not depend on the mode; only which units each contraction keeps)
    import dataclasses
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
