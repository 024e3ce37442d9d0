"""float64 CPU oracle for the fused top-K KD loss and the teacher-cache build.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU-baseline leg, never by the product path.  Shares no code with the HIP
library.

Notation follows "The Gradient That Top-k Distillation Never Computes":
q is the teacher, p the student, S the retained index set (|S| = K),
z = W h the student logits, m_q the teacher's tail mass and m_p the
student's tail mass outside S.

Readings taken where the pages leave a step open are stated at the function
that takes them.
"""
from __future__ import annotations

import numpy as np

RENORM, TAIL, FULL, REVERSE, TAIL_REVERSE, REVERSE_TT = 0, 1, 2, 3, 4, 5
MODES = (RENORM, TAIL, FULL, REVERSE, TAIL_REVERSE)   # the modes that need no sampled token
MODE_NAMES = {RENORM: "renorm", TAIL: "tail", FULL: "full", REVERSE: "reverse", TAIL_REVERSE: "tail_reverse",
              REVERSE_TT: "reverse_tt"}

# Smallest normal float32: the floor for a student tail mass that rounds to 0
# while the teacher still has tail mass (the loss is then huge but finite).
_TINY = float(np.finfo(np.float32).tiny)


def logsumexp(x: np.ndarray) -> float:
    """log(sum(exp(x))) of a 1-D float64 vector, shifted by its max."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return -np.inf
    m = np.max(x)
    if not np.isfinite(m):
        return float(m)
    return float(m + np.log(np.sum(np.exp(x - m))))


def student_logits(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """z = h W^T for h [T, d], W [V, d]: the LM-head logits, float64."""
    return np.asarray(h, np.float64) @ np.asarray(W, np.float64).T


def _loss_row(z: np.ndarray, S: np.ndarray, tl: np.ndarray, m_q: float, mode: int):
    """Per-token loss L, logit gradient dz = dL/dz, lse and m_p for one row.

    z: [V] float64 logits; S: [k] distinct indices; tl: [k] teacher log-probs
    at S; m_q: teacher tail mass (used by TAIL only).
    """
    V = z.shape[0]
    lse = logsumexp(z)
    logp = z - lse
    p = np.exp(logp)
    in_s = np.zeros(V, dtype=bool)
    in_s[S] = True
    # Student tail mass: the direct sum over the tokens outside S.
    m_p = float(np.sum(p[~in_s]))
    q = np.exp(tl)
    Q = float(np.sum(q))
    dz = np.zeros(V)

    if mode == RENORM:
        # Renormalized top-k forward KL L_S = KL(q_hat || p_hat), both
        # renormalized over S ("The Gradient That Top-k Distillation Never
        # Computes", abstract and Figure 2).
        log_qh = tl - logsumexp(tl)
        log_ph = z[S] - logsumexp(z[S])
        qh = np.exp(log_qh)
        L = float(np.sum(qh * (log_qh - log_ph)))
        dz[S] = np.exp(log_ph) - qh
    elif mode == TAIL:
        # (K+1)-bin forward KL: teacher bins (q_S, m_q), student bins
        # (p_S, m_p), the extra bin carrying the tail mass ("Tail-Aware
        # Top-k On-Policy Distillation", abstract; taken in the forward
        # direction).  Gradient is the exact derivative of this L:
        #   dz_u = (Q + m_q) p_u - q_u [u in S] - (m_q / m_p) p_u [u not in S].
        L = float(np.sum(q * (tl - logp[S])))
        ratio = 0.0
        if m_q > 0.0:
            mp = max(m_p, _TINY)
            L += m_q * (np.log(m_q) - np.log(mp))
            ratio = m_q / mp
        dz = (Q + m_q) * p
        dz[S] -= q
        dz[~in_s] -= ratio * p[~in_s]
    elif mode == FULL:
        # Partial-mass forward KL against the unrenormalized top-K teacher
        # (p_v = 0 off S), identity (2) of the fused-chunked-loss paper:
        # H - C + M log Z with M = sum_S q.  Its gradient, Eq. (3), is the
        # dense M softmax(z) minus the sparse teacher term.
        L = float(np.sum(q * (tl - z[S]))) + Q * lse
        dz = Q * p
        dz[S] -= q
    elif mode == REVERSE:
        # Top-k reverse KL KL(p_hat || q_hat) over S ("Unbiased Top-k
        # Estimation for On-Policy Distillation", abstract).
        log_ph = z[S] - logsumexp(z[S])
        log_qh = tl - logsumexp(tl)
        ph = np.exp(log_ph)
        L = float(np.sum(ph * (log_ph - log_qh)))
        dz[S] = ph * (log_ph - log_qh - L)
    elif mode == TAIL_REVERSE:
        # Reverse KL over the top-k bins plus one tail token carrying the
        # tail mass: KL((p_S, m_p) || (q_S, m_q)) ("Tail-Aware Top-k
        # On-Policy Distillation", abstract).  With a_v = log(p_v / q_v) -
        # log(m_p / m_q) on S (the derivative of L in p_v, m_p = 1 - sum_S p),
        # dz_u = p_u (a_u [u in S] - sum_S p a).  Both tail masses are
        # floored at the smallest normal float32 inside the logarithms.
        mp = max(m_p, _TINY)
        mq = max(m_q, _TINY)
        tail_log = np.log(mp) - np.log(mq)
        L = float(np.sum(p[S] * (logp[S] - tl))) + m_p * tail_log
        a = (logp[S] - tl) - tail_log
        A = float(np.sum(p[S] * a))
        dz = -A * p
        dz[S] += p[S] * a
    elif mode == REVERSE_TT:
        # Top-k part of the tail-corrected reverse-KL gradient estimator
        # ("Unbiased Top-k Estimation for On-Policy Distillation", abstract and
        # Figure 1): L is the full-vocabulary reverse KL restricted to S,
        # sum_S p_v (log p_v - log q_v), and dz is the S-part of the full
        # reverse-KL gradient, sum_S a_v grad p_v with a = log p - log q held
        # fixed: dz_u = p_u (a_u [u in S] - sum_S p a).  It is not the
        # derivative of this L, which would add p_u ([u in S] - sum_S p) from
        # differentiating a.  The sampled-token correction is added by
        # _sampled_tail_term.
        a = logp[S] - tl
        L = float(np.sum(p[S] * a))
        dz = -L * p
        dz[S] += p[S] * a
    else:
        raise ValueError(f"unknown mode {mode}")
    return L, dz, lse, m_p


def _support(idx_row: np.ndarray, tlp_row: np.ndarray):
    """Entries with idx < 0 are padding and take no part in the loss."""
    keep = np.asarray(idx_row) >= 0
    return np.asarray(idx_row)[keep].astype(np.int64), np.asarray(tlp_row, np.float64)[keep]


def _label_term(z: np.ndarray, y: int, lse: float, ce_weight: float):
    """Hard-label cross-entropy term added to a distillation loss:
    ce_weight * (lse - z_y), gradient ce_weight * (softmax(z) - e_y).

    "The Gradient That Top-k Distillation Never Computes" (abstract) trains
    the top-k student with and without the cross-entropy term on the data
    token; the weight is not printed, so it is an argument here.  A label
    y < 0 means the token has no label (no term).
    """
    if y < 0 or ce_weight == 0.0:
        return 0.0, None
    p = np.exp(z - lse)
    g = ce_weight * p
    g[y] -= ce_weight
    return ce_weight * (lse - float(z[y])), g


def _sampled_tail_term(z: np.ndarray, y: int, tly: float, lse: float, S: np.ndarray):
    """Sampled-token tail correction of REVERSE_TT.

    The full reverse KL R = sum_v p_v l_v (l = log p - log q) has gradient
    sum_v l_v grad p_v; the part outside S equals E_{y ~ p}[1(y not in S)
    l_y grad log p_y].  With y the token the student sampled in its own
    rollout, 1(y not in S) l_y grad log p_y (l_y held fixed: the stop-gradient
    of "Unbiased Top-k Estimation for On-Policy Distillation", Figure 1) is
    an unbiased estimate of it, and 1(y not in S) l_y of the tail part of R.
    The paper's equation is not printed; this is the reading taken.
    Returns (loss term, gradient term) or (0, None).
    """
    if y < 0 or np.any(S == y):
        return 0.0, None
    ell = float(z[y] - lse) - float(tly)
    g = -ell * np.exp(z - lse)
    g[y] += ell
    return ell, g


def loss_rows_from_logits(z, idx, tlp, m_q, mode, labels=None, ce_weight=0.0, tlp_labels=None):
    """Per-token (L, dz, lse, m_p) for logits z [T, V].  Returns arrays.

    With labels [T] (int, -1 = none) and ce_weight, each labelled token also
    carries the hard-label cross-entropy term of _label_term.  For
    REVERSE_TT, labels are the sampled tokens and tlp_labels [T] the teacher
    log-probabilities at them (_sampled_tail_term)."""
    z = np.asarray(z, np.float64)
    T, V = z.shape
    L = np.zeros(T)
    dz = np.zeros((T, V))
    lse = np.zeros(T)
    m_p = np.zeros(T)
    mq = np.zeros(T) if m_q is None else np.asarray(m_q, np.float64)
    for t in range(T):
        S, tl = _support(idx[t], tlp[t])
        L[t], dz[t], lse[t], m_p[t] = _loss_row(z[t], S, tl, float(mq[t]), mode)
        if mode == REVERSE_TT and labels is not None:
            Ls, gs = _sampled_tail_term(z[t], int(labels[t]), float(tlp_labels[t]), lse[t], S)
            if gs is not None:
                L[t] += Ls
                dz[t] += gs
        elif labels is not None:
            Lc, gc = _label_term(z[t], int(labels[t]), lse[t], float(ce_weight))
            if gc is not None:
                L[t] += Lc
                dz[t] += gc
    return L, dz, lse, m_p


def loss_fwd_bwd(h, W, idx, tlp, m_q, mode, scale=None, block=256, labels=None, ce_weight=0.0, tlp_labels=None):
    """Fused LM head + top-K KD loss, forward and backward, as dense math.

    loss = scale * sum_t L_t; dh = scale * dz W; dW = scale * dz^T h,
    with z = h W^T in float64.  The mean over tokens (scale = 1/T) is the
    default reduction; the pages only define per-token losses.  labels and
    ce_weight add the hard-label cross-entropy term (_label_term).

    Returns a dict with loss, loss_tok [T], lse [T], m_p [T], dh [T, d],
    dW [V, d].
    """
    h = np.asarray(h, np.float64)
    W = np.asarray(W, np.float64)
    idx = np.asarray(idx)
    tlp = np.asarray(tlp, np.float64)
    T, d = h.shape
    V = W.shape[0]
    if scale is None:
        scale = 1.0 / max(T, 1)
    dh = np.zeros((T, d))
    dW = np.zeros((V, d))
    L = np.zeros(T)
    lse = np.zeros(T)
    m_p = np.zeros(T)
    mq = None if m_q is None else np.asarray(m_q, np.float64)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        z = h[t0:t1] @ W.T
        Lb, dz, lb, mb = loss_rows_from_logits(
            z, idx[t0:t1], tlp[t0:t1], None if mq is None else mq[t0:t1], mode,
            None if labels is None else labels[t0:t1], ce_weight,
            None if tlp_labels is None else tlp_labels[t0:t1])
        L[t0:t1], lse[t0:t1], m_p[t0:t1] = Lb, lb, mb
        dh[t0:t1] = scale * (dz @ W)
        dW += scale * (dz.T @ h[t0:t1])
    return {"loss": scale * float(np.sum(L)), "loss_tok": L, "lse": lse, "m_p": m_p,
            "dh": dh, "dW": dW}


def topk_row(z_row: np.ndarray, K: int):
    """Top-K of one logit row: indices ordered by (value desc, index asc).

    Ties go to the lower index; -0.0 and +0.0 compare equal.  The K-th
    largest value is found by a partition, then every strictly larger entry
    is kept together with the lowest-index entries equal to it.
    """
    z_row = np.asarray(z_row)
    V = z_row.shape[0]
    K = int(K)
    if K >= V:
        sel = np.arange(V)
    else:
        kth = np.partition(z_row, V - K)[V - K]
        above = np.flatnonzero(z_row > kth)
        equal = np.flatnonzero(z_row == kth)
        sel = np.concatenate([above, equal[:K - above.size]])
    order = np.lexsort((sel, -z_row[sel].astype(np.float64)))
    return sel[order]


def adaptive_k_row(z_row: np.ndarray, lse: float, rho: float) -> int:
    """k_rho = min{k : sum of the k largest teacher probabilities >= rho}.

    ("Sparse Teacher Support Cuts LLM Distillation Cost Without Losing
    Accuracy", definition of the retained rank k_rho.)  Probabilities are
    exp(z - lse) in float64, accumulated in descending order of value.
    Returns V if rounding keeps the total below rho.
    """
    z64 = np.asarray(z_row, np.float64)
    p_sorted = np.exp(np.sort(z64)[::-1] - lse)
    c = np.cumsum(p_sorted)
    hit = np.flatnonzero(c >= rho)
    return int(hit[0]) + 1 if hit.size else int(z64.shape[0])


def cache_from_logits(z, K, rho=()):
    """Teacher cache of logit rows z [T, V]: top-K, logsumexp, tail mass, k_rho.

    Returns (idx int64 [T, K], val [T, K] (the logits themselves, same dtype
    as z), lse float64 [T], m_q float64 [T], k_rho int64 [T, len(rho)]).
    m_q is the direct sum of exp(z - lse) over the tokens outside the top-K
    ("The Gradient That Top-k Distillation Never Computes", Figure 3: the
    mass a top-k cache discards).
    """
    z = np.asarray(z)
    T, V = z.shape
    K = int(K)
    idx = np.zeros((T, K), np.int64)
    val = np.zeros((T, K), z.dtype)
    lse = np.zeros(T)
    m_q = np.zeros(T)
    k_rho = np.zeros((T, len(rho)), np.int64)
    for t in range(T):
        row = z[t]
        sel = topk_row(row, K)
        idx[t] = sel
        val[t] = row[sel]
        z64 = row.astype(np.float64)
        lse[t] = logsumexp(z64)
        keep = np.ones(V, dtype=bool)
        keep[sel] = False
        m_q[t] = float(np.sum(np.exp(z64[keep] - lse[t])))
        for j, r in enumerate(rho):
            k_rho[t, j] = adaptive_k_row(z64, lse[t], float(r))
    return idx, val, lse, m_q, k_rho


def teacher_logp(val, lse):
    """Cached teacher log-probabilities at the retained indices: val - lse."""
    return np.asarray(val, np.float64) - np.asarray(lse, np.float64)[:, None]


def cache_build(g, U, b, K, rho=(), block=256):
    """Teacher-cache build from the teacher's final hidden state.

    z = U g + b per token ("The Gradient That Top-k Distillation Never
    Computes", Figure 3 bottom: the head reconstruction), then the top-K
    cache of each row.  b may be None (no bias, e.g. a student head).
    """
    g = np.asarray(g, np.float64)
    U = np.asarray(U, np.float64)
    T = g.shape[0]
    outs = []
    for t0 in range(0, T, block):
        z = g[t0:t0 + block] @ U.T
        if b is not None:
            z = z + np.asarray(b, np.float64)[None, :]
        outs.append(cache_from_logits(z, K, rho))
    return tuple(np.concatenate([o[i] for o in outs], axis=0) for i in range(5))


def quantize_hidden_int8(g):
    """Per-position symmetric int8 code of a hidden state: scale s = max|g| / 127
    and codes rint(g / s) in [-127, 127], both in float32 ("The Gradient That
    Top-k Distillation Never Computes", Table A2: the int8 hidden-state cache
    of d + 4 bytes per position; the quantizer itself is not printed, absmax
    with round-half-even is the reading taken).  A zero row has s = 0 and
    zero codes.  Returns (codes int8 [T, d], s float32 [T])."""
    g = np.asarray(g, np.float32)
    amax = np.max(np.abs(g), axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(g / safe[:, None]).astype(np.float32)
    q = np.clip(q, -127, 127)
    q[s == 0] = 0
    return q.astype(np.int8), s


def kl_hidden_fwd_bwd(h, W, g, U, b=None, scale=None, block=256, g_scale=None):
    """Exact full-vocabulary KL(q || p) with the teacher rebuilt from a cached
    hidden state: q = softmax(U g + b), p = softmax(W h).

    "The Gradient That Top-k Distillation Never Computes", Figure 3 (bottom):
    caching the teacher's final hidden state g instead of its top-k logits
    reconstructs the full teacher distribution exactly at 2dV FLOP per
    token.  Per token L = sum_v q_v (log q_v - log p_v), dL/dz = p - q;
    loss = scale * sum_t L (default scale 1/T), dh = scale * dz W,
    dW = scale * dz^T h.  With g_scale [T] (an int8 cache: g holds the
    codes), the teacher logits are g_scale_t * (U g_t) + b.  Returns a dict
    with loss, loss_tok, lse (student), lse_t (teacher), dh, dW.
    """
    h = np.asarray(h, np.float64)
    W = np.asarray(W, np.float64)
    g = np.asarray(g, np.float64)
    U = np.asarray(U, np.float64)
    T, d = h.shape
    V = W.shape[0]
    if scale is None:
        scale = 1.0 / max(T, 1)
    L = np.zeros(T)
    lse = np.zeros(T)
    lse_t = np.zeros(T)
    dh = np.zeros((T, d))
    dW = np.zeros((V, d))
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        z = h[t0:t1] @ W.T
        zt = g[t0:t1] @ U.T
        if g_scale is not None:
            zt = zt * np.asarray(g_scale, np.float64)[t0:t1, None]
        if b is not None:
            zt = zt + np.asarray(b, np.float64)[None, :]
        for r in range(t1 - t0):
            lse[t0 + r] = logsumexp(z[r])
            lse_t[t0 + r] = logsumexp(zt[r])
        logp = z - lse[t0:t1, None]
        logq = zt - lse_t[t0:t1, None]
        q = np.exp(logq)
        L[t0:t1] = np.sum(q * (logq - logp), axis=1)
        dz = np.exp(logp) - q
        dh[t0:t1] = scale * (dz @ W)
        dW += scale * (dz.T @ h[t0:t1])
    return {"loss": scale * float(np.sum(L)), "loss_tok": L, "lse": lse, "lse_t": lse_t, "dh": dh, "dW": dW}


def recover_teacher_hidden(idx, tlp, U, b=None):
    """Teacher hidden state and log-normalizer from k cached log-probabilities
    ("The Gradient That Top-k Distillation Never Computes", abstract and
    Table 1: the retained set determines the teacher's distribution once
    k >= d + 1).  Cached log q_v = U_v g + b_v - c on S, with c the teacher's
    logsumexp, is linear in (g, c): the least-squares solution of
    [U_S, -1] (g; c) = log q_S - b_S (numpy's lstsq, the minimum-norm one
    when k < d + 1, where it is not unique).  Returns (g_hat [T, d],
    c_hat [T]) in float64.
    """
    idx = np.asarray(idx)
    tlp = np.asarray(tlp, np.float64)
    U = np.asarray(U, np.float64)
    T, k = idx.shape
    d = U.shape[1]
    g_hat = np.zeros((T, d))
    c_hat = np.zeros(T)
    for t in range(T):
        S = idx[t].astype(np.int64)
        A = np.concatenate([U[S], -np.ones((k, 1))], axis=1)
        y = tlp[t] - (np.asarray(b, np.float64)[S] if b is not None else 0.0)
        x = np.linalg.lstsq(A, y, rcond=None)[0]
        g_hat[t], c_hat[t] = x[:d], x[d]
    return g_hat, c_hat
