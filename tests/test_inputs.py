"""The seeded generator: rounding, determinism and the stated distributions."""
import math

import numpy as np
import torch

import synthetic_inputs as si


def test_rne_rounding_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([
        r.standard_normal(100000).astype(np.float32) * 10,
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0,
                  3.0e38, 1e-40], dtype=np.float32),
    ])
    ours = si.bits_to_torch_bf16(si.rne_bf16_bits(a))
    ref = torch.from_numpy(a).to(torch.bfloat16)
    assert torch.equal(ours.view(torch.int16), ref.view(torch.int16))


def test_deterministic_and_shapes():
    w = si.Workload("t", 300, 1000, 64, ignore_rows=7, tail_targets=5, tail_width=100, seed=9)
    E1, C1, x1 = si.generate(w)
    E2, C2, x2 = si.generate(w)
    assert torch.equal(E1.view(torch.int16), E2.view(torch.int16))
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    assert torch.equal(x1, x2)
    assert E1.shape == (300, 64) and C1.shape == (1000, 64) and x1.shape == (300,)
    assert int((x1 == si.IGNORE_INDEX).sum()) == 7
    valid = x1[x1 != si.IGNORE_INDEX]
    assert int(valid.min()) >= 0 and int(valid.max()) < 1000
    assert int((x1 >= 900).sum()) >= 5


def test_zipf_targets_front_loaded():
    r = np.random.default_rng(1)
    x = si.zipf_targets(r, 200000, 256000)
    share = np.mean(x < 256)
    assert 0.60 < share < 0.68
    assert x.min() >= 0 and x.max() < 256000


def test_peaked_logit_std_and_margin():
    w = si.Workload("p", 256, 8192, 512, seed=3)
    E, C, x = si.generate(w)
    A = E.double() @ C.double().T
    t = A[torch.arange(256), x]
    mask = torch.ones_like(A, dtype=torch.bool)
    mask[torch.arange(256), x] = False
    std = A[mask].std().item()
    assert 2.6 < std < 3.4
    margin = (t.mean().item()) / std
    assert 4.5 < margin < 7.5


def test_tiny_distribution():
    E, C, x = si.generate(si.TINY)
    assert abs(E.float().std().item() - 1.0) < 0.02
    assert abs(C.float().std().item() - 64 ** -0.25) < 0.01
    assert int((x == si.IGNORE_INDEX).sum()) == 16


def test_entry_bias_is_a_shared_per_entry_logit_bias():
    """entry_bias leaves every other draw as it was and gives each entry one
    logit offset shared by all tokens, of the stated standard deviation."""
    import dataclasses
    w0 = si.Workload("b", 256, 4096, 512, seed=5)
    w1 = dataclasses.replace(w0, entry_bias=1.0)
    E0, C0, x0 = si.generate(w0)
    E1, C1, x1 = si.generate(w1)
    assert torch.equal(C0.view(torch.int16), C1.view(torch.int16)) and torch.equal(x0, x1)
    d = (E1.double() - E0.double())
    # one shared direction: every row moved by (nearly) the same vector
    assert (d - d.mean(0)).abs().max().item() < 0.05 * d.mean(0).abs().max().item() + 0.02
    bias = C0.double() @ d.mean(0)          # the per-entry offset
    assert 0.85 < bias.std().item() < 1.15
    # the logit difference is that offset for every token
    diff = E1.double() @ C0.double().T - E0.double() @ C0.double().T
    assert (diff - bias).abs().max().item() < 0.1 * bias.abs().max().item() + 0.05
    # the default leaves the five workloads' draws alone
    assert si.Workload("b", 1, 1, 8).entry_bias == 0.0
