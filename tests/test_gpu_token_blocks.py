"""GPU parity of the backward when it takes the tokens in blocks.

Past 16,384 padded rows the backward walks (vocabulary chunk, token block)
pairs, the blocks equal whole 256-row tiles of at most 8,192 rows: G-hat and
its unit maps hold one block, each block's dE tiles keep their own part of the
fp32 accumulator over the chunks, and dC sums over the blocks of a chunk in an
fp32 accumulator of its own before the cast to bf16.  At 16,700 rows that is
three blocks of 5,632 rows.  Every output is compared in full with the fp64
oracle, at the tolerances of the other parity tests (loss and lse 1e-5, dE and
dC 3e-3 relative Frobenius, ignored rows exactly zero).
"""
import pytest

import linear_cross_entropy_amd as lce
import synthetic_inputs as si
from test_gpu_parity import EPS, _check_full
from test_gpu_sorting import _check_sorted

pytestmark = pytest.mark.gpu

N_BLOCKED = 16700  # padded to 16,896 rows: three token blocks
# two chunks (8192 + 808 rows) and D = 296 (two 256-wide column tiles, the
# second ragged)
V_BLOCKED, D_BLOCKED = 9000, 296


def _blocked(name, ignore_rows, reduction="mean", seed=40, N=N_BLOCKED):
    w = si.Workload(name, N, V_BLOCKED, D_BLOCKED, logit_std=5.0,
                    ignore_rows=ignore_rows, tail_targets=40, tail_width=300,
                    reduction=reduction, seed=seed)
    # the plan blocks the tokens: G-hat for all rows in two 8192-wide chunk
    # copies would alone be over 500 MiB
    _, b = lce.cce_workspace_bytes(w.N, w.V, w.D)
    assert b < 2 * (w.N // 256 * 256) * 8192 * 2
    return w


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_token_blocks_match_oracle(eps):
    got, st = _check_full(_blocked("blocks", 40), eps)
    if eps:
        assert st["units_skipped"] > 0


def test_token_blocks_shorter_last_block():
    # 16,500 rows pad to 16,640: blocks of 5,632, 5,632 and 5,376 rows (the
    # last block one tile short of the others)
    _check_full(_blocked("blocks-short-last", 30, reduction="none", seed=45, N=16500), EPS)


def test_token_blocks_last_block_all_ignored():
    # 8,000 ignored rows: after compaction the first block is all valid, the
    # second partly and the third holds ignored rows only (its G-hat tiles do
    # not run and its dC pass adds nothing)
    _check_full(_blocked("blocks-ignored", 8000, reduction="sum", seed=41), EPS)


def test_token_blocks_only_first_block_valid():
    # 12,000 ignored rows: the 4,700 valid rows fill part of the first block;
    # the middle block's dC tiles have nothing to add and return at once, the
    # last block's only cast the accumulator
    _check_full(_blocked("blocks-first-only", 12000, reduction="mean", seed=44), EPS)


@pytest.mark.parametrize("mode", ["full_c", "full_e"])
def test_token_blocks_filter_variants(mode):
    _check_full(_blocked("blocks-mode", 40, seed=42), EPS, filter_mode=mode)


@pytest.mark.parametrize("order_kind", ["random", "oracle"])
def test_token_blocks_sorted_backward(order_kind):
    _check_sorted(_blocked("blocks-sorted", 40, seed=43), EPS, order_kind)
