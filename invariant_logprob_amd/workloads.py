"""Seeded synthetic inputs for the selected-token logprob workloads.

This module only draws random inputs; it holds none of the logprob
arithmetic, so the HIP library and the fp64 oracle can both be fed from it.
Every tensor comes from a ``torch.Generator`` seeded explicitly, drawn in
float32 and rounded once (round-to-nearest-even) to bfloat16.

The shapes follow the reinforcement-learning setting the pages describe:
varlen packing and padding, batch 1 vs large, decode vs prefill (page "[RFC]
Batch-Invariant RL Kernel Suite for Train-Inference Consistency", sections
"Problem" and "Scope"), and the fixture fields of page "docs(ws1):
batch-invariance contract RFC", section "InvarianceFixture" (target ids,
an action mask that defines the active token set).  ``N(0, s)`` means
standard deviation ``s``.

Named workloads (sizes as used by the tests and the benchmark):

* ``logits_small``   N=8, V=1024, logits ~ N(0,2), uniform targets, all active.
* ``logits_varlen``  8 sequences of length U{64..1024} packed back to back and
  padded to a multiple of 128 rows; V=32000; logits ~ N(0,3); 5% of rows get
  +20 on one uniformly chosen index before rounding; targets are the row's
  argmax (lowest index on ties) with probability 1/2, else uniform; padding
  rows are masked with target -100.
* ``logits_large``   N=16384, V=151936, logits ~ N(0,4); exactly
  round(0.15 N) = 2458 rows masked at random positions (target -100);
  uniform targets elsewhere.
* ``fused_large``    hidden [8192, 4096] ~ N(0,1), weight [128256, 4096] ~
  N(0, 0.02), uniform targets, all active.
* ``fused_bwd``      hidden [2048, 5120] ~ N(0,1), weight [151936, 5120] ~
  N(0, 0.02), upstream gradient ~ N(0,1) float32, uniform targets.
"""

from dataclasses import dataclass, field
from typing import Optional

import torch

IGNORE_TARGET = -100


def _gen(seed, device):
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type != "cuda" else dev)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, sigma, gen, device, block_rows=1024):
    """float32 N(0, sigma) draws rounded once to bfloat16, drawn row-block by
    row-block so that huge matrices never need a full float32 copy."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    rows = shape[0]
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        blk = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device,
                          dtype=torch.float32)
        if sigma != 1.0:
            blk.mul_(sigma)
        out[r0:r1] = blk.to(torch.bfloat16)
    return out


@dataclass
class LogitsBatch:
    logits: torch.Tensor             # bf16 [N, V]
    targets: torch.Tensor            # int64 [N]
    mask: torch.Tensor               # uint8 [N], 1 = active token
    seq_lens: Optional[list] = None  # packed sequence lengths (varlen workloads)
    grad: Optional[torch.Tensor] = None   # float32 [N] upstream gradient of logp
    meta: dict = field(default_factory=dict)


@dataclass
class FusedBatch:
    hidden: torch.Tensor             # bf16 [N, H]
    weight: torch.Tensor             # bf16 [V, H]
    targets: torch.Tensor            # int64 [N]
    mask: torch.Tensor               # uint8 [N]
    grad: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)


def uniform_targets(n, v, gen, device):
    return torch.randint(0, v, (n,), generator=gen, device=device, dtype=torch.int64)


def upstream_grad(n, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.randn((n,), generator=g, device=device, dtype=torch.float32)


def logits_batch(n, v, sigma, seed=0, device="cpu", n_masked=0):
    """Plain batch: N(0, sigma) logits, uniform targets, ``n_masked`` rows
    masked at seeded random positions (their target is -100)."""
    g = _gen(seed, device)
    logits = normal_bf16((n, v), sigma, g, device)
    targets = uniform_targets(n, v, g, device)
    mask = torch.ones(n, dtype=torch.uint8, device=device)
    if n_masked:
        pos = torch.randperm(n, generator=g, device=device)[:n_masked]
        mask[pos] = 0
        targets[pos] = IGNORE_TARGET
    grad = torch.randn((n,), generator=g, device=device, dtype=torch.float32)
    return LogitsBatch(logits, targets, mask, grad=grad,
                       meta=dict(n=n, v=v, sigma=sigma, seed=seed, n_masked=n_masked))


def logits_small(seed=0, device="cpu"):
    return logits_batch(8, 1024, 2.0, seed, device)


def logits_large(seed=0, device="cpu", n=16384, v=151936):
    return logits_batch(n, v, 4.0, seed, device, n_masked=int(round(0.15 * n)))


def logits_varlen(seed=0, device="cpu", n_seqs=8, v=32000, len_lo=64, len_hi=1024,
                  pad_multiple=128, sigma=3.0, peaked_frac=0.05, peak=20.0):
    g = _gen(seed, device)
    lens = torch.randint(len_lo, len_hi + 1, (n_seqs,), generator=g, device=device).tolist()
    total = sum(lens)
    n = ((total + pad_multiple - 1) // pad_multiple) * pad_multiple
    x = torch.empty((n, v), dtype=torch.bfloat16, device=device)
    n_peaked = int(round(peaked_frac * n))
    peaked_rows = torch.randperm(n, generator=g, device=device)[:n_peaked]
    peaked_cols = torch.randint(0, v, (n_peaked,), generator=g, device=device)
    is_peaked = torch.zeros(n, dtype=torch.bool, device=device)
    is_peaked[peaked_rows] = True
    col_of = torch.zeros(n, dtype=torch.int64, device=device)
    col_of[peaked_rows] = peaked_cols
    for r0 in range(0, n, 512):
        r1 = min(n, r0 + 512)
        blk = torch.randn((r1 - r0, v), generator=g, device=device, dtype=torch.float32) * sigma
        sel = is_peaked[r0:r1]
        if bool(sel.any()):
            idx = torch.nonzero(sel).flatten()
            blk[idx, col_of[r0:r1][idx]] += peak
        x[r0:r1] = blk.to(torch.bfloat16)
    # targets: argmax of the rounded values (torch.argmax returns the first
    # maximal index) with probability 1/2, else uniform
    argmax = torch.empty(n, dtype=torch.int64, device=device)
    for r0 in range(0, n, 512):
        argmax[r0:r0 + 512] = torch.argmax(x[r0:r0 + 512].float(), dim=1)
    coin = torch.rand((n,), generator=g, device=device) < 0.5
    unif = uniform_targets(n, v, g, device)
    targets = torch.where(coin, argmax, unif)
    mask = torch.zeros(n, dtype=torch.uint8, device=device)
    mask[:total] = 1
    targets[total:] = IGNORE_TARGET
    grad = torch.randn((n,), generator=g, device=device, dtype=torch.float32)
    return LogitsBatch(x, targets, mask, seq_lens=lens, grad=grad,
                       meta=dict(n=n, v=v, sigma=sigma, seed=seed, total_tokens=total,
                                 n_peaked=n_peaked))


def fused_batch(n, v, h, seed=0, device="cpu", w_sigma=0.02, h_sigma=1.0, n_masked=0):
    g = _gen(seed, device)
    hidden = normal_bf16((n, h), h_sigma, g, device)
    weight = normal_bf16((v, h), w_sigma, g, device)
    targets = uniform_targets(n, v, g, device)
    mask = torch.ones(n, dtype=torch.uint8, device=device)
    if n_masked:
        pos = torch.randperm(n, generator=g, device=device)[:n_masked]
        mask[pos] = 0
        targets[pos] = IGNORE_TARGET
    grad = torch.randn((n,), generator=g, device=device, dtype=torch.float32)
    return FusedBatch(hidden, weight, targets, mask, grad=grad,
                      meta=dict(n=n, v=v, h=h, seed=seed))


def fused_large(seed=0, device="cpu"):
    return fused_batch(8192, 128256, 4096, seed, device)


def fused_bwd(seed=0, device="cpu"):
    return fused_batch(2048, 151936, 5120, seed, device)


def neighbour_rows(n, v, seed, device="cpu"):
    """Fresh rows of varied content for neighbour-content transforms: normal,
    peaked (+30 on one entry), wide-range (N(0, 60)) and rows that hold -inf
    entries."""
    g = _gen(seed, device)
    x = torch.randn((n, v), generator=g, device=device, dtype=torch.float32) * 3.0
    kind = torch.arange(n, device=device) % 4
    cols = torch.randint(0, v, (n,), generator=g, device=device)
    rows = torch.arange(n, device=device)
    pk = kind == 1
    x[rows[pk], cols[pk]] += 30.0
    x[kind == 2] *= 20.0
    ninf = (kind == 3)
    if bool(ninf.any()):
        drop = torch.rand((n, v), generator=g, device=device) < 0.25
        x[ninf.unsqueeze(1) & drop] = float("-inf")
        x[rows[ninf], cols[ninf]] = 0.0
    targets = torch.randint(0, v, (n,), generator=g, device=device)
    targets = torch.where(ninf, cols, targets)   # keep those rows' targets finite
    return x.to(torch.bfloat16), targets


def bf16_bits_numpy(t):
    """Raw bf16 bits of a tensor as a numpy uint16 array (host copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
