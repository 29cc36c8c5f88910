"""Seeded synthetic inputs for the int2 draft LM head.

This module only draws random numbers and rounds them to bf16. It holds none of the head's
arithmetic, and both sides of every comparison take their inputs from it: the oracle (tests,
CPU baseline) and the HIP library (tests, bench, smoke).

The activations the head was measured on came from a live serve and are not available, so the
inputs below stand in for them with the head's real shapes:

  W[n, k] = bf16(0.02 * z[n, k] * r[n])     z ~ N(0, 1), r[n] = exp(0.3 * u[n]), u ~ N(0, 1)
  x[m, k] = bf16(z'[m, k] * s[k])           z' ~ N(0, 1), s[k] = 20 on `outliers` fixed hidden
                                           channels (the first entries of a seeded permutation
                                           of K, shared by every row), 1 elsewhere

Each tensor is drawn on the CPU from torch.Generator streams with fixed seeds (x: 1, W: 2,
row scales: 3, outlier channels: 4). W is drawn in fixed chunks of W_CHUNK_ROWS rows, chunk c
from its own generator seeded `seed * 1_000_003 + c`, so a large W can be drawn by several
threads and the bits do not depend on the thread count.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np
import torch

SEED_X = 1
SEED_W = 2
SEED_ROWSCALE = 3
SEED_OUTLIER = 4
W_CHUNK_ROWS = 4096

# Workloads of the int2 head. K is the hidden size, N the vocab rows one GPU holds (one rank's
# 124160-row slice of a 248320-row vocab, or the whole vocab), M the draft rows per call.
WORKLOADS = {
    "tiny_head_m1_k512_n4096": dict(M=1, K=512, N=4096, outliers=0, topk=1),
    "draft_slot_m1_k5120_n124160": dict(M=1, K=5120, N=124160, outliers=8, topk=1),
    "draft_band_m16_k5120_n124160": dict(M=16, K=5120, N=124160, outliers=8, topk=1),
    "draft_band_m64_k5120_n124160": dict(M=64, K=5120, N=124160, outliers=8, topk=1),
    "full_vocab_top16_k5120_n248320": dict(M=(1, 2, 4, 8, 16, 32, 64, 72), K=5120, N=248320,
                                           outliers=8, topk=16),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def fp8_head_of(w: torch.Tensor):
    """The per-channel FP8 form of a head w [N, K] (any float dtype, any device): (e4m3 bytes
    uint8 [N, K], scale fp32 [N]) with scale = max |w| / 448 per row and the bytes torch's
    round-to-nearest cast of w / scale (the storage of a compressed-tensors FP8 lm_head)."""
    wf = w.float()
    scale = (wf.abs().amax(dim=1) / 448.0).clamp(min=1e-12)
    w8 = (wf / scale[:, None]).to(torch.float8_e4m3fn)
    return w8.view(torch.uint8), scale.float()


def gen_weight_fp8(N: int, K: int, seed: int = SEED_W, rowscale_seed: int = SEED_ROWSCALE):
    """fp8_head_of(gen_weight(N, K)), on the CPU."""
    return fp8_head_of(gen_weight(N, K, seed, rowscale_seed))


def gen_weight(N: int, K: int, seed: int = SEED_W, rowscale_seed: int = SEED_ROWSCALE) -> torch.Tensor:
    """bf16 [N, K] head weight (rows are vocab tokens), on the CPU."""
    u = torch.randn(N, generator=_gen(rowscale_seed), dtype=torch.float32)
    r = torch.exp(0.3 * u)
    out = torch.empty(N, K, dtype=torch.bfloat16)
    nchunks = (N + W_CHUNK_ROWS - 1) // W_CHUNK_ROWS

    def fill(c: int) -> None:
        a = c * W_CHUNK_ROWS
        b = min(N, a + W_CHUNK_ROWS)
        z = torch.randn(b - a, K, generator=_gen(seed * 1_000_003 + c), dtype=torch.float32)
        out[a:b] = ((0.02 * z) * r[a:b, None]).to(torch.bfloat16)

    if nchunks == 1:
        fill(0)
    else:
        prev = torch.get_num_threads()
        torch.set_num_threads(1)
        try:
            with _cf.ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, range(nchunks)))
        finally:
            torch.set_num_threads(prev)
    return out


def outlier_channels(K: int, count: int, seed: int = SEED_OUTLIER) -> torch.Tensor:
    """The `count` hidden channels that carry outliers (int64 indices into K)."""
    if count <= 0:
        return torch.empty(0, dtype=torch.int64)
    return torch.randperm(K, generator=_gen(seed))[:count].clone()


def gen_x(M: int, K: int, outliers: int = 0, seed: int = SEED_X, batch: int = 0) -> torch.Tensor:
    """bf16 [M, K] draft-head inputs, on the CPU. `batch` selects an independent batch of rows."""
    z = torch.randn(M, K, generator=_gen(seed * 1_000_003 + batch), dtype=torch.float32)
    if outliers > 0:
        z[:, outlier_channels(K, outliers)] *= 20.0
    return z.to(torch.bfloat16)


def gen_scores(M: int, N: int, seed: int = 11) -> torch.Tensor:
    """fp32 [M, N] random scores, used to drive the candidate steps on their own."""
    return torch.randn(M, N, generator=_gen(seed), dtype=torch.float32)


def gen_rows(M: int, R: int, N: int, seed: int = 12) -> torch.Tensor:
    """int32 [M, R]: per row, R distinct token indices in [0, N) in random order."""
    g = _gen(seed)
    return torch.stack([torch.randperm(N, generator=g)[:R] for _ in range(M)]).to(torch.int32)


def gen_coarse_row(M: int, N: int, seed: int = 13, levels: int = 0) -> torch.Tensor:
    """bf16 [M, N] rows shaped like coarse logits (3 z, z ~ N(0, 1)); with levels > 0 the values
    are rounded to multiples of 1/levels first, so many entries tie (and both signed zeros occur)."""
    z = 3.0 * torch.randn(M, N, generator=_gen(seed), dtype=torch.float32)
    if levels > 0:
        z = torch.round(z * levels) / levels
    return z.to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (CPU copy), for the numpy side."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
