"""Test inputs: seeded synthetic tensors (synth) and teacher caches built by
the CPU oracle.  Nothing here comes from the HIP path."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth


def _cache_block(args):
    T, V, K, seed, b = args
    zt = synth.zipf_teacher_logits(T, V, seed=seed, first_block=b, n_blocks=1)
    i, val, lse, m_q, _ = oracle.cache_from_logits(zt, K)
    return b, i.astype(np.int32), oracle.teacher_logp(val, lse).astype(np.float32), m_q.astype(np.float32)


def teacher_cache(T: int, V: int, K: int, seed: int = 0):
    """Zipf-like teacher rows -> oracle top-K cache: (idx int32, tlp fp32, m_q fp32) numpy.
    Row blocks are independent (seeded per block) and run in a process pool."""
    idx = np.zeros((T, K), np.int32)
    tlp = np.zeros((T, K), np.float32)
    mq = np.zeros(T, np.float32)
    nb = (T + synth.BLOCK - 1) // synth.BLOCK
    jobs = [(T, V, K, seed, b) for b in range(nb)]
    for b, i, tl, m in synth._map_blocks(_cache_block, jobs):
        r0 = b * synth.BLOCK
        idx[r0:r0 + len(i)] = i
        tlp[r0:r0 + len(i)] = tl
        mq[r0:r0 + len(i)] = m
    return idx, tlp, mq


def _gather_block(args):
    T, V, seed, b, idx_b = args
    zt = synth.zipf_teacher_logits(T, V, seed=seed, first_block=b, n_blocks=1).astype(np.float64)
    lt = np.stack([zt[r] - oracle.logsumexp(zt[r]) for r in range(zt.shape[0])])
    return b, np.take_along_axis(lt, idx_b.astype(np.int64), axis=1).astype(np.float32)


def student_topk_cache(h: torch.Tensor, W: torch.Tensor, K: int, T: int, V: int, seed: int = 0):
    """REVERSE support: the student's own top-K (oracle, fp64 logits) and the
    teacher log-probs gathered at those indices from the full Zipf rows."""
    h64 = synth.as_f64(h)
    W64 = synth.as_f64(W)
    idx = np.zeros((T, K), np.int32)
    tlp = np.zeros((T, K), np.float32)
    nb = (T + synth.BLOCK - 1) // synth.BLOCK
    for b in range(nb):
        r0 = b * synth.BLOCK
        r1 = min(T, r0 + synth.BLOCK)
        z = oracle.student_logits(h64[r0:r1], W64)
        i, _, _, _, _ = oracle.cache_from_logits(z, K)
        idx[r0:r1] = i
    jobs = [(T, V, seed, b, idx[b * synth.BLOCK:min(T, (b + 1) * synth.BLOCK)]) for b in range(nb)]
    for b, tl in synth._map_blocks(_gather_block, jobs):
        tlp[b * synth.BLOCK:b * synth.BLOCK + len(tl)] = tl
    return idx, tlp


def gather_teacher_logp(idx: np.ndarray, T: int, V: int, seed: int = 0) -> np.ndarray:
    """Teacher log-probabilities (oracle logsumexp of the full Zipf rows) at
    the given indices [T, K] (any selection, e.g. the student's top-K)."""
    out = np.zeros(idx.shape, np.float32)
    nb = (T + synth.BLOCK - 1) // synth.BLOCK
    jobs = [(T, V, seed, b, idx[b * synth.BLOCK:min(T, (b + 1) * synth.BLOCK)]) for b in range(nb)]
    for b, tl in synth._map_blocks(_gather_block, jobs):
        out[b * synth.BLOCK:b * synth.BLOCK + len(tl)] = tl
    return out


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def rel_err(a: float, b: float, floor: float = 1e-6) -> float:
    return abs(float(a) - float(b)) / max(abs(float(b)), floor)
