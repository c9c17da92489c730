"""Seeded synthetic inputs for the Cut Cross-Entropy hot path.

This module is shared by the tests, the smoke check and the bench; it holds
none of the method's arithmetic (no logits, softmax or gradients), only the
random draws and the fp32 -> bf16 rounding of the inputs.

Workloads follow the shapes the pages measure (the "Cut Your Losses" digest,
Table 1: Gemma 2 2B head; the CCE blog post: Qwen2.5-0.5B head; the kernel
card: a Llama-3-sized vocabulary at 65,536 tokens) and stand in for the real
hidden states and weights used there, which are not available.

Recipe (all draws from numpy Philox streams keyed by (seed, stream)):

* ``tiny``: E ~ N(0, 1); C with variance 1/sqrt(D) (std D**-0.25); targets
  uniform on [0, V); ``ignore_rows`` seeded rows set to the ignore index.
* ``peaked`` (the classifier-head shapes): C ~ N(0, 0.02**2) rounded to bf16;
  targets Zipf(s=1.1) over ranks 1..V with id = rank - 1 (frequent ids low);
  E = sigma * (z + beta * c_hat[x]) with z ~ N(0, I_D), c_hat the unit-norm
  bf16 row of C for the target, sigma = logit_std / (0.02 * sqrt(D + beta**2))
  so that non-target logits have std ~ logit_std, and a target margin of about
  beta logit standard deviations.  beta = 6 by default; beta = 0.5 * sqrt(D)
  is the literal (degenerate) reading.
* Optional: a fraction of rows set to the ignore index (drawn after E), and
  ``tail_targets`` valid rows whose target is moved uniformly into the final
  ``tail_width`` vocabulary ids.
* Optional ``entry_bias`` (logit standard deviations): every hidden state
  also carries one shared direction u (a unit vector, its own stream), E +=
  (entry_bias / 0.02) u, so entry v's logit gains u . C[v] * entry_bias / 0.02,
  a bias of std entry_bias shared by all tokens: some entries are likely
  across the batch, as common tokens are in a real head, which is what
  vocabulary sorting gathers.  0 (the default) leaves every draw unchanged.
* All float tensors are drawn in fp32 and rounded to bf16 (round to nearest
  even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    V: int
    D: int
    kind: str = "peaked"          # "tiny" or "peaked"
    logit_std: float = 3.0
    beta: float | None = 6.0      # None = literal 0.5*sqrt(D)
    ignore_rows: int = 0
    tail_targets: int = 0
    tail_width: int = 256
    reduction: str = "mean"
    seed: int = 0
    entry_bias: float = 0.0       # std of a per-entry logit bias shared by all tokens


# The five workloads (shapes of the pages' heads) ...
TINY = Workload("tiny", 256, 2048, 64, kind="tiny", ignore_rows=16, seed=0)
QWEN = Workload("qwen2.5-0.5b-head", 4096, 151936, 896, seed=1)
GEMMA = Workload("gemma2-2b-head", 8192, 256000, 2304, seed=2)
LLAMA = Workload("llama3-head-long", 65536, 128256, 2048,
                 ignore_rows=3277, tail_targets=256, tail_width=256, seed=3)
GPTOSS = Workload("gpt-oss-head", 16384, 201088, 2880, logit_std=1.0,
                  reduction="none", seed=4)
FULL = [TINY, QWEN, GEMMA, LLAMA, GPTOSS]
# ... and the Gemma-2-2B head with likely entries (a per-entry logit bias of std
# 1, shared across tokens), where vocabulary sorting has entries to gather.
GEMMA_BIASED = Workload("gemma2-2b-head-entry-bias", 8192, 256000, 2304, seed=2, entry_bias=1.0)
VARIANTS = [GEMMA_BIASED]


def rne_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_torch_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[seed, stream]))


def _normal_bf16(rng, rows, cols, std, chunk_rows=4096):
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        out[r0:r1] = rne_bf16_bits(z)
    return out


def zipf_targets(rng, n, V, s=1.1):
    ranks = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    u = rng.random(n) * cdf[-1]
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)


def generate_bits(w: Workload):
    """Returns (E_bits [N,D] uint16, C_bits [V,D] uint16, x [N] int64)."""
    N, V, D = w.N, w.V, w.D
    tail_rows = np.zeros(0, dtype=np.int64)
    if w.kind == "tiny":
        E = _normal_bf16(_rng(w.seed, 1), N, D, 1.0)
        C = _normal_bf16(_rng(w.seed, 2), V, D, D ** -0.25)
        x = _rng(w.seed, 3).integers(0, V, size=N, dtype=np.int64)
    elif w.kind == "peaked":
        C = _normal_bf16(_rng(w.seed, 2), V, D, 0.02)
        x = zipf_targets(_rng(w.seed, 3), N, V)
        if w.tail_targets:
            r = _rng(w.seed, 5)
            rows = r.choice(N, size=min(w.tail_targets, N), replace=False)
            tail_rows = rows
            lo = max(0, V - w.tail_width)
            x[rows] = r.integers(lo, V, size=rows.size, dtype=np.int64)
        beta = 0.5 * math.sqrt(D) if w.beta is None else w.beta
        sigma = w.logit_std / (0.02 * math.sqrt(D + beta * beta))
        rz = _rng(w.seed, 1)
        shift = None
        if w.entry_bias:
            u = _rng(w.seed, 7).standard_normal(D)
            shift = (w.entry_bias / 0.02) * (u / np.linalg.norm(u))
        E = np.empty((N, D), dtype=np.uint16)
        for r0 in range(0, N, 4096):
            r1 = min(N, r0 + 4096)
            z = rz.standard_normal((r1 - r0, D), dtype=np.float32)
            c = bits_to_f32(C[x[r0:r1]]).astype(np.float64)
            c /= np.linalg.norm(c, axis=1, keepdims=True)
            e = sigma * (z.astype(np.float64) + beta * c)
            if shift is not None:
                e += shift
            E[r0:r1] = rne_bf16_bits(e.astype(np.float32))
    else:
        raise ValueError(w.kind)
    if w.ignore_rows:
        # drawn after E; rows whose target was moved into the vocabulary tail stay valid
        pool = np.setdiff1d(np.arange(N), tail_rows)
        rows = _rng(w.seed, 4).choice(pool, size=min(w.ignore_rows, pool.size), replace=False)
        x[rows] = IGNORE_INDEX
    return E, C, x


def generate(w: Workload):
    """Returns CPU torch tensors (E bf16 [N,D], C bf16 [V,D], x int64 [N])."""
    E, C, x = generate_bits(w)
    return bits_to_torch_bf16(E), bits_to_torch_bf16(C), torch.from_numpy(x)


def upstream_grad(w: Workload, kind: str = "ones"):
    """Upstream gradient: a scalar 1.0 for mean/sum, [N] values for 'none'
    (ones, or seeded U(0.5, 1.5) for parity runs)."""
    if w.reduction != "none":
        return torch.ones((), dtype=torch.float32)
    if kind == "ones":
        return torch.ones(w.N, dtype=torch.float32)
    g = _rng(w.seed, 6).uniform(0.5, 1.5, size=w.N).astype(np.float32)
    return torch.from_numpy(g)
