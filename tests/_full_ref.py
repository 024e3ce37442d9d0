"""Sampled fp64 references at full size, composed from oracle functions.

The oracle's per-token math runs on every token (so the loss, lse, m_p and
every dW row see all T tokens); only the outputs are sampled: dh at a few
tokens, dW at a few vocabulary rows."""
from __future__ import annotations

import numpy as np

import oracle


def sampled_reference(h64, W64, idx, tlp, mq, mode, tok_rows, vocab_rows, scale=None, block=256, log=None,
                      labels=None, ce_weight=0.0, tlp_labels=None):
    T, d = h64.shape
    if scale is None:
        scale = 1.0 / T
    L = np.zeros(T)
    lse = np.zeros(T)
    mp = np.zeros(T)
    tok_rows = np.asarray(tok_rows)
    vocab_rows = np.asarray(vocab_rows)
    dh = np.zeros((len(tok_rows), d))
    dW = np.zeros((len(vocab_rows), d))
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        z = oracle.student_logits(h64[t0:t1], W64)
        Lb, dz, lb, mb = oracle.loss_rows_from_logits(
            z, idx[t0:t1], tlp[t0:t1], None if mq is None else mq[t0:t1], mode,
            None if labels is None else labels[t0:t1], ce_weight,
            None if tlp_labels is None else tlp_labels[t0:t1])
        L[t0:t1], lse[t0:t1], mp[t0:t1] = Lb, lb, mb
        dW += scale * (dz[:, vocab_rows].T @ h64[t0:t1])
        for j, t in enumerate(tok_rows):
            if t0 <= t < t1:
                dh[j] = scale * (dz[t - t0] @ W64)
        if log is not None and (t0 // block) % 8 == 0:
            log(f"oracle block {t0 // block + 1}/{(T + block - 1) // block}")
    return {"loss": scale * L.sum(), "loss_tok": L, "lse": lse, "m_p": mp, "dh": dh, "dW": dW}
