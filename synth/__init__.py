"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the storage dtypes.
It holds none of the loss or teacher-cache arithmetic: no logsumexp, no
softmax, no top-K selection, no gradient.  Both the CPU oracle and the HIP
library consume what it returns; neither side imports the other.

Recipes (the workloads of the fused top-K KD loss and its teacher cache):

* student head: h ~ N(0, 1) [T, d], W ~ N(0, 1/d) [V, d], both rounded to
  bf16 (round to nearest even).  N(mean, x) takes x as the variance, so
  W's rows give logits of roughly unit variance.
* teacher logits, Zipf-like: for each row an independent uniform random
  permutation pi of {0..V-1} and iid eps ~ N(0, 1);
  z(v) = -a * ln(1 + pi(v)) + s * eps(v), with a = 1.2, s = 0.3, float32.
* teacher head for the cache build: g ~ N(0, 1) [T, d] bf16,
  U ~ N(0, 1/d) [V, d] bf16, b ~ N(0, 0.1) [V] float32 (variance 0.1).

Every stream is keyed by (seed, stream id, block index) through numpy's
SeedSequence, so a block of rows can be regenerated on its own and the
result does not depend on how many worker processes produced it.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import torch

STREAM_H = 1
STREAM_W = 2
STREAM_TEACHER = 3
STREAM_G = 4
STREAM_U = 5
STREAM_B = 6
STREAM_TIES = 7
STREAM_LABELS = 8

# rows per independently seeded block
BLOCK = 256


def _rng(seed: int, stream: int, block: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(block)])


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy array -> bf16 CPU tensor, round to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU/GPU tensor (bf16, fp32, ...) to a float64 array."""
    return t.detach().to("cpu", torch.float64).numpy()


def _normal_block(args):
    seed, stream, block, rows, cols, std = args
    r = _rng(seed, stream, block)
    x = r.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _workers(n_blocks: int) -> int:
    if n_blocks < 4:
        return 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16, n_blocks))


def _map_blocks(fn, jobs):
    nw = _workers(len(jobs))
    if nw == 1:
        return [fn(j) for j in jobs]
    # spawned workers: they never inherit a parent's GPU runtime state
    with ProcessPoolExecutor(max_workers=nw, mp_context=multiprocessing.get_context("spawn")) as ex:
        return list(ex.map(fn, jobs))


def normal_f32(rows: int, cols: int, std: float, seed: int, stream: int) -> np.ndarray:
    """[rows, cols] float32 ~ N(0, std^2), generated in seeded row blocks."""
    jobs = []
    for b, r0 in enumerate(range(0, rows, BLOCK)):
        jobs.append((seed, stream, b, min(BLOCK, rows - r0), cols, std))
    if not jobs:
        return np.zeros((0, cols), np.float32)
    return np.concatenate(_map_blocks(_normal_block, jobs), axis=0)


def student_head(T: int, d: int, V: int, seed: int = 0):
    """(h bf16 [T, d] ~ N(0,1), W bf16 [V, d] ~ N(0, 1/d)) as CPU tensors."""
    h = to_bf16(normal_f32(T, d, 1.0, seed, STREAM_H))
    W = to_bf16(normal_f32(V, d, 1.0 / np.sqrt(d), seed, STREAM_W))
    return h, W


def teacher_head(T: int, d: int, V: int, seed: int = 0, bias_var: float = 0.1):
    """(g bf16 [T, d] ~ N(0,1), U bf16 [V, d] ~ N(0, 1/d), b fp32 [V] ~ N(0, bias_var))."""
    g = to_bf16(normal_f32(T, d, 1.0, seed, STREAM_G))
    U = to_bf16(normal_f32(V, d, 1.0 / np.sqrt(d), seed, STREAM_U))
    b = torch.from_numpy(normal_f32(1, V, float(np.sqrt(bias_var)), seed, STREAM_B)[0].copy())
    return g, U, b


def _zipf_block(args):
    seed, block, rows, V, expo, noise = args
    r = _rng(seed, STREAM_TEACHER, block)
    ranks = r.permuted(np.broadcast_to(np.arange(V, dtype=np.int64), (rows, V)), axis=1)
    eps = r.standard_normal((rows, V), dtype=np.float32)
    base = (-expo * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    return np.ascontiguousarray(base[ranks] + np.float32(noise) * eps)


def zipf_teacher_logits(T: int, V: int, seed: int = 0, exponent: float = 1.2,
                        noise: float = 0.3, first_block: int = 0, n_blocks: int | None = None) -> np.ndarray:
    """Zipf-like teacher logits, float32 [rows, V].

    Rows come in seeded blocks of BLOCK rows; ``first_block``/``n_blocks``
    regenerate a sub-range of blocks (rows first_block*BLOCK ...) without
    producing the rest.
    """
    total_blocks = (T + BLOCK - 1) // BLOCK
    if n_blocks is None:
        n_blocks = total_blocks - first_block
    jobs = []
    for b in range(first_block, first_block + n_blocks):
        r0 = b * BLOCK
        jobs.append((seed, b, min(BLOCK, T - r0), V, exponent, noise))
    if not jobs:
        return np.zeros((0, V), np.float32)
    return np.ascontiguousarray(np.concatenate(_map_blocks(_zipf_block, jobs), axis=0))


def zipf_teacher_logits_device(rows: int, V: int, seed: int, device, first_row: int = 0, exponent: float = 1.2,
                               noise: float = 0.3) -> torch.Tensor:
    """The Zipf-like teacher recipe above drawn on a GPU with torch's
    generator, float32 [rows, V] on ``device``: rows first_row .. are keyed by
    (seed, row block of BLOCK rows) so any row range regenerates alone.  The
    permutation of each row is the argsort of V iid float64 uniforms (a
    uniform random permutation; ties have probability ~V^2 2^-54).  Same
    distribution as zipf_teacher_logits, a different random stream: for
    large benchmark inputs, where the CPU generator would take minutes."""
    base = (-exponent * torch.log1p(torch.arange(V, dtype=torch.float64, device=device))).to(torch.float32)
    out = torch.empty((rows, V), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    r = 0
    while r < rows:
        row = first_row + r
        blk = row // BLOCK
        r1 = min(rows, (blk + 1) * BLOCK - first_row)
        gen.manual_seed(int(np.random.SeedSequence([int(seed), STREAM_TEACHER, int(blk)]).generate_state(1)[0]))
        keys = torch.rand((BLOCK, V), dtype=torch.float64, device=device, generator=gen)
        eps = torch.randn((BLOCK, V), dtype=torch.float32, device=device, generator=gen)
        perm = torch.argsort(keys, dim=1)
        blk_rows = base[perm] + noise * eps
        o0 = row - blk * BLOCK
        out[r:r1] = blk_rows[o0:o0 + (r1 - r)]
        del keys, eps, perm, blk_rows
        r = r1
    return out


def tie_heavy_logits(rows: int, V: int, seed: int = 0, step: float = 0.25,
                     span: float = 4.0) -> np.ndarray:
    """float32 logits rounded to multiples of ``step`` in [-span, span]: many exact ties."""
    r = _rng(seed, STREAM_TIES, 0)
    x = np.round(r.uniform(-span, span, size=(rows, V)) / step) * step
    return x.astype(np.float32)


def token_labels(T: int, V: int, seed: int = 0, unlabelled_every: int = 5) -> np.ndarray:
    """int32 data-token labels uniform in [0, V); every unlabelled_every-th
    token has none (-1)."""
    r = _rng(seed, STREAM_LABELS, 0)
    y = r.integers(0, V, size=T).astype(np.int32)
    if unlabelled_every > 0:
        y[::unlabelled_every] = -1
    return y
