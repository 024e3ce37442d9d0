"""Sampled fp64 references at full size, composed from oracle functions.

The oracle's per-token math runs on every token (so the loss, lse, m_p for
every token and every sampled dW row see all T tokens); only the outputs are
sampled: dh at a few tokens, dW at a few vocabulary rows.  Token blocks are
independent, so they run on a thread pool (numpy releases the interpreter
lock inside BLAS and its elementwise loops); the per-block dW partials are
added in block order, so the result does not depend on the schedule."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def sampled_reference_modes(h64, W64, idx, tlp, mq, modes, tok_rows, vocab_rows, scale=None, block=256, log=None,
                            labels=None, ce_weight=0.0, tlp_labels=None, workers=None):
    """{mode: {loss, loss_tok, lse, m_p, dh (sampled tokens), dW (sampled rows)}}
    for several modes on the same inputs; z = h W^T is formed once per block."""
    T, d = h64.shape
    if scale is None:
        scale = 1.0 / T
    tok_rows = np.asarray(tok_rows)
    vocab_rows = np.asarray(vocab_rows)
    nb = (T + block - 1) // block

    def one(b):
        t0, t1 = b * block, min(T, (b + 1) * block)
        z = oracle.student_logits(h64[t0:t1], W64)
        res = {}
        for mode in modes:
            Lb, dz, lb, mb = oracle.loss_rows_from_logits(
                z, idx[t0:t1], tlp[t0:t1], None if mq is None else mq[t0:t1], mode,
                None if labels is None else labels[t0:t1], ce_weight,
                None if tlp_labels is None else tlp_labels[t0:t1])
            dWb = scale * (dz[:, vocab_rows].T @ h64[t0:t1])
            dhb = {j: scale * (dz[t - t0] @ W64) for j, t in enumerate(tok_rows) if t0 <= t < t1}
            res[mode] = (Lb, lb, mb, dWb, dhb)
        return b, res

    out = {m: {"loss_tok": np.zeros(T), "lse": np.zeros(T), "m_p": np.zeros(T),
               "dh": np.zeros((len(tok_rows), d)), "dW": np.zeros((len(vocab_rows), d))} for m in modes}
    nw = workers or _workers()
    parts = [None] * nb
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=max(1, _workers() // nw), user_api="blas")
    except Exception:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(max_workers=nw) as ex:
            for k, (b, res) in enumerate(ex.map(one, range(nb))):
                parts[b] = res
                if log is not None and k % 16 == 0:
                    log(f"oracle block {k + 1}/{nb}")
    finally:
        if limit is not None:
            limit.restore_original_limits()
    for b in range(nb):
        t0, t1 = b * block, min(T, (b + 1) * block)
        for mode in modes:
            Lb, lb, mb, dWb, dhb = parts[b][mode]
            o = out[mode]
            o["loss_tok"][t0:t1], o["lse"][t0:t1], o["m_p"][t0:t1] = Lb, lb, mb
            o["dW"] += dWb
            for j, v in dhb.items():
                o["dh"][j] = v
    for mode in modes:
        out[mode]["loss"] = scale * out[mode]["loss_tok"].sum()
    return out


def sampled_reference(h64, W64, idx, tlp, mq, mode, tok_rows, vocab_rows, scale=None, block=256, log=None,
                      labels=None, ce_weight=0.0, tlp_labels=None):
    return sampled_reference_modes(h64, W64, idx, tlp, mq, [mode], tok_rows, vocab_rows, scale, block, log,
                                   labels, ce_weight, tlp_labels)[mode]
