"""Pins for the CPU oracle: printed values, closed forms, library routines,
finite differences and brute force.  CPU only.

Each test pins the oracle to something other than itself, chosen so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import RENORM, TAIL, FULL, REVERSE, TAIL_REVERSE, REVERSE_TT

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Worked example: "The Gradient That Top-k Distillation Never Computes", Fig. 2
# --------------------------------------------------------------------------

def _fig2_setup():
    g = json.load(open(os.path.join(GOLD, "worked_example_fig2.json")))
    V, k = g["vocab"], g["k"]
    m_q = g["student_tail_mass_before"]  # p equals the teacher
    head = np.array(g["renormalized_head"])
    q = np.concatenate([(1.0 - m_q) * head, np.full(V - k, m_q / (V - k))])
    # d = 2: h = (1, 0) gives the student p = q; h = (1, 1) lowers the
    # retained logits by ln 6 and gives p'.
    W = np.zeros((V, 2))
    W[:, 0] = np.log(q)
    W[:k, 1] = -np.log(6.0)
    h = np.array([[1.0, 0.0], [1.0, 1.0]])
    return g, q, W, h


@pytest.mark.parametrize("K_full", [False, True])
def test_fig2_printed_values(K_full):
    g, q, W, h = _fig2_setup()
    V, k = g["vocab"], g["k"]
    K = V if K_full else k
    idx = np.tile(np.arange(K), (2, 1))
    tlp = np.tile(np.log(q[:K]), (2, 1))
    m_q = np.full(2, 1.0 - q[:K].sum())
    tol = 0.5 * 10 ** -g["printed_decimals_full_vocab_kl"]

    z = oracle.student_logits(h, W)
    # renormalized heads of p and p' equal the printed teacher head
    for t in range(2):
        ph = np.exp(z[t, :k] - scipy.special.logsumexp(z[t, :k]))
        np.testing.assert_allclose(ph, g["renormalized_head"], atol=1e-12)

    if not K_full:
        r = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, RENORM, scale=1.0)
        assert abs(r["loss_tok"][0] - g["renormalized_loss_before"]) < 1e-12
        assert abs(r["loss_tok"][1] - g["renormalized_loss_after"]) < 1e-12
        np.testing.assert_allclose(r["m_p"], [g["student_tail_mass_before"],
                                              g["student_tail_mass_after"]], atol=1e-12)
        np.testing.assert_allclose(r["dh"], 0.0, atol=1e-12)
        # the tail loss sees what the renormalized one cannot
        rt = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, TAIL, scale=1.0)
        assert abs(rt["loss_tok"][0]) < 1e-12
        assert abs(rt["loss_tok"][1] - g["full_vocab_kl_after_nats"]) < tol
    else:
        r = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, FULL, scale=1.0)
        assert abs(r["loss_tok"][0] - g["full_vocab_kl_before_nats"]) < 1e-12
        assert abs(r["loss_tok"][1] - g["full_vocab_kl_after_nats"]) < tol


def test_fig2_closed_forms():
    """Exact values behind the printed 0.335 (derived by hand, not printed)."""
    g, q, W, h = _fig2_setup()
    k = g["k"]
    z = oracle.student_logits(h, W)
    idx = np.tile(np.arange(k), (2, 1))
    tlp = np.tile(np.log(q[:k]), (2, 1))
    m_q = np.full(2, 0.2)
    kl = 0.8 * math.log(2) - 0.2 * math.log(3)
    L, dz, lse, m_p = oracle.loss_rows_from_logits(z, idx, tlp, m_q, TAIL)
    assert abs(L[1] - kl) < 1e-12
    # dz(p') = p' - q: (-0.20, -0.10, -0.06, -0.04, +0.05 x 8)
    np.testing.assert_allclose(dz[1], [-0.2, -0.1, -0.06, -0.04] + [0.05] * 8, atol=1e-12)
    L, dz, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, FULL)
    assert abs(L[1] - 0.8 * math.log(2)) < 1e-12  # partial mass at K = 4
    np.testing.assert_allclose(dz[1], [-0.24, -0.12, -0.072, -0.048] + [0.06] * 8, atol=1e-12)
    L, dz, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, REVERSE)
    np.testing.assert_allclose(L, 0.0, atol=1e-12)
    np.testing.assert_allclose(dz, 0.0, atol=1e-12)


# --------------------------------------------------------------------------
# Small random problems
# --------------------------------------------------------------------------

def _problem(seed, T=3, d=8, V=24, K=5, consistent=True):
    r = np.random.default_rng(seed)
    h = r.standard_normal((T, d))
    W = r.standard_normal((V, d)) / np.sqrt(d)
    zt = r.standard_normal((T, V)) * 1.5
    idx = np.zeros((T, K), np.int64)
    tlp = np.zeros((T, K))
    m_q = np.zeros(T)
    for t in range(T):
        S = r.choice(V, size=K, replace=False)
        lq = zt[t] - scipy.special.logsumexp(zt[t])
        idx[t], tlp[t] = S, lq[S]
        m_q[t] = 1.0 - np.exp(lq[S]).sum()
        if not consistent:  # a cache whose bins do not sum to one
            tlp[t] += 0.05 * r.standard_normal(K)
            m_q[t] *= 1.1
    return h, W, idx, tlp, m_q


@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("consistent", [True, False])
def test_finite_differences(mode, consistent):
    h, W, idx, tlp, m_q = _problem(1 + mode, consistent=consistent)
    scale = 0.7
    r = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, mode, scale=scale)

    def f(hh, WW):
        return oracle.loss_fwd_bwd(hh, WW, idx, tlp, m_q, mode, scale=scale)["loss"]

    eps = 1e-6
    for name, X, G in (("h", h, r["dh"]), ("W", W, r["dW"])):
        num = np.zeros_like(X)
        for i in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[i] += eps
            Xm[i] -= eps
            num[i] = (f(Xp, W) - f(Xm, W)) / (2 * eps) if name == "h" else \
                     (f(h, Xp) - f(h, Xm)) / (2 * eps)
        err = np.linalg.norm(num - G) / max(np.linalg.norm(G), 1e-300)
        assert err < 1e-6, (name, err)


def _torch_loss(z_row, S, tl, m_q, mode):
    """The textbook divergence of each mode through torch's own KL routines."""
    from torch.distributions import Categorical, kl_divergence
    zt = torch.tensor(z_row, dtype=torch.float64, requires_grad=True)
    S_t = torch.tensor(S)
    tl_t = torch.tensor(tl, dtype=torch.float64)
    if mode == RENORM:
        L = kl_divergence(Categorical(logits=tl_t), Categorical(logits=zt[S_t]))
    elif mode == REVERSE:
        L = kl_divergence(Categorical(logits=zt[S_t]), Categorical(logits=tl_t))
    elif mode == FULL:
        target = torch.zeros_like(zt)
        target[S_t] = torch.exp(tl_t)
        L = torch.nn.functional.kl_div(torch.log_softmax(zt, 0), target, reduction="sum")
    else:  # TAIL / TAIL_REVERSE: KL between the two (K+1)-categoricals
        p = torch.softmax(zt, 0)
        mask = torch.ones_like(zt, dtype=torch.bool)
        mask[S_t] = False
        pt = torch.cat([p[S_t], p[mask].sum().reshape(1)])
        qt = torch.cat([torch.exp(tl_t), torch.tensor([m_q], dtype=torch.float64)])
        if mode == TAIL:
            L = torch.sum(qt * (torch.log(qt) - torch.log(pt)))
        else:
            L = torch.sum(pt * (torch.log(pt) - torch.log(qt)))
    L.backward()
    return float(L.detach()), zt.grad.numpy()


@pytest.mark.parametrize("mode", oracle.MODES)
def test_against_torch_textbook_forms(mode):
    h, W, idx, tlp, m_q = _problem(11 + mode, T=4, d=6, V=40, K=7)
    z = oracle.student_logits(h, W)
    L, dz, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, mode)
    for t in range(z.shape[0]):
        Lt, gt = _torch_loss(z[t], idx[t], tlp[t], m_q[t], mode)
        assert abs(L[t] - Lt) < 1e-12 * max(1.0, abs(Lt))
        np.testing.assert_allclose(dz[t], gt, atol=1e-13)


def test_k_equals_v_is_dense_kl():
    """At K = V the three forward modes all equal the dense KL(q || p)."""
    r = np.random.default_rng(5)
    T, d, V = 3, 5, 16
    h = r.standard_normal((T, d))
    W = r.standard_normal((V, d))
    zt = r.standard_normal((T, V))
    lq = zt - scipy.special.logsumexp(zt, axis=1, keepdims=True)
    perm = np.stack([r.permutation(V) for _ in range(T)])
    idx = perm
    tlp = np.take_along_axis(lq, perm, axis=1)
    m_q = np.zeros(T)
    z = h @ W.T
    p = scipy.special.softmax(z, axis=1)
    q = np.exp(lq)
    kl = scipy.special.rel_entr(q, p).sum(axis=1)
    for mode in (RENORM, TAIL, FULL):
        L, dz, _, m_p = oracle.loss_rows_from_logits(z, idx, tlp, m_q, mode)
        np.testing.assert_allclose(L, kl, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dz, p - q, atol=1e-13)
        np.testing.assert_allclose(m_p, 0.0, atol=0)


@pytest.mark.parametrize("mode", oracle.MODES)
def test_gradient_sums_to_zero(mode):
    for consistent in (True, False):
        h, W, idx, tlp, m_q = _problem(21 + mode, T=5, V=30, K=6, consistent=consistent)
        z = oracle.student_logits(h, W)
        _, dz, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, mode)
        np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-14)


@pytest.mark.parametrize("mode", [RENORM, REVERSE])
def test_renormalized_modes_blind_to_tail(mode):
    """Zero off S, invariant to shifting the retained logits, dh in the span
    of retained-row differences (Theorem 1 of the top-k gradient paper)."""
    h, W, idx, tlp, m_q = _problem(31 + mode, T=4, d=12, V=30, K=5)
    z = oracle.student_logits(h, W)
    L, dz, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, mode)
    for t in range(z.shape[0]):
        off = np.ones(z.shape[1], bool)
        off[idx[t]] = False
        assert np.all(dz[t, off] == 0.0)
    z2 = z.copy()
    for t in range(z.shape[0]):
        z2[t, idx[t]] += 0.37 * (t + 1)
    L2, dz2, _, m_p2 = oracle.loss_rows_from_logits(z2, idx, tlp, m_q, mode)
    np.testing.assert_allclose(L2, L, atol=1e-13)
    np.testing.assert_allclose(dz2, dz, atol=1e-13)
    r = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, mode, scale=1.0)
    for t in range(h.shape[0]):
        S = idx[t]
        A = (W[S[1:]] - W[S[0]]).T  # d x (K-1) basis of the span
        Qb, _ = np.linalg.qr(A)
        g = r["dh"][t]
        resid = g - Qb @ (Qb.T @ g)
        assert np.linalg.norm(resid) <= 1e-12 * max(np.linalg.norm(g), 1e-300)


def test_truncated_plus_residual_identity():
    """p - q = (1 - m_q)(p_hat - q_hat)|_S + r, with r = (m_q - m_p) p_hat on S
    and r = p - q off S: full gradient = truncated gradient + tail residual."""
    r_ = np.random.default_rng(41)
    T, d, V, K = 4, 6, 25, 5
    h = r_.standard_normal((T, d))
    W = r_.standard_normal((V, d))
    zt = r_.standard_normal((T, V)) * 2
    lq = zt - scipy.special.logsumexp(zt, axis=1, keepdims=True)
    z = h @ W.T
    full_idx = np.tile(np.arange(V), (T, 1))
    _, g_full, _, _ = oracle.loss_rows_from_logits(z, full_idx, lq, np.zeros(T), FULL)
    idx = np.stack([np.argsort(-lq[t])[:K] for t in range(T)])
    tlp = np.take_along_axis(lq, idx, axis=1)
    m_q = 1.0 - np.exp(tlp).sum(axis=1)
    _, g_trunc, _, m_p = oracle.loss_rows_from_logits(z, idx, tlp, m_q, RENORM)
    p = scipy.special.softmax(z, axis=1)
    for t in range(T):
        S = idx[t]
        off = np.ones(V, bool)
        off[S] = False
        ph = p[t, S] / p[t, S].sum()
        rhs = np.zeros(V)
        rhs[S] = (1 - m_q[t]) * g_trunc[t, S] + (m_q[t] - m_p[t]) * ph
        rhs[off] = p[t, off] - np.exp(lq[t, off])
        np.testing.assert_allclose(g_full[t], rhs, atol=1e-14)


def test_tail_mass_is_direct_tail_sum():
    h, W, idx, tlp, m_q = _problem(51, T=3, V=20, K=4)
    r = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, TAIL)
    z = h @ W.T
    for t in range(3):
        p = scipy.special.softmax(z[t])
        assert abs(r["m_p"][t] - (1.0 - p[idx[t]].sum())) < 1e-14
        assert abs(r["lse"][t] - scipy.special.logsumexp(z[t])) < 1e-13


def test_padding_entries_are_ignored():
    h, W, idx, tlp, m_q = _problem(61, T=3, V=20, K=4)
    pad_idx = np.concatenate([idx, -np.ones((3, 2), np.int64)], axis=1)
    pad_tlp = np.concatenate([tlp, np.full((3, 2), 123.0)], axis=1)
    for mode in oracle.MODES:
        a = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, mode)
        b = oracle.loss_fwd_bwd(h, W, pad_idx, pad_tlp, m_q, mode)
        assert a["loss"] == b["loss"]
        np.testing.assert_array_equal(a["dh"], b["dh"])


def test_zero_teacher_tail():
    """m_q = 0: the tail bin vanishes and TAIL reduces to the FULL form."""
    h, W, idx, tlp, m_q = _problem(71, T=3, V=20, K=4)
    z = h @ W.T
    m0 = np.zeros(3)
    Lt, dt, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m0, TAIL)
    Lf, df, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m0, FULL)
    np.testing.assert_allclose(Lt, Lf, atol=1e-13)
    np.testing.assert_allclose(dt, df, atol=1e-14)


# --------------------------------------------------------------------------
# Teacher cache: top-K, lse, m_q, k_rho
# --------------------------------------------------------------------------

def _brute_topk(row, K):
    keys = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))
    return np.array(keys[:K])


@pytest.mark.parametrize("K", [1, 3, 16, 64])
def test_topk_brute_force_with_ties(K):
    import synth
    z = synth.tie_heavy_logits(6, 97, seed=K)
    z[0, :] = 1.0                 # all equal
    z[1, ::3] = -0.0              # signed zeros mixed with +0.0
    z[1, 1::3] = 0.0
    z[2, 5:40] = -np.inf          # -inf entries
    for t in range(z.shape[0]):
        got = oracle.topk_row(z[t], K)
        np.testing.assert_array_equal(got, _brute_topk(z[t], K))


def test_topk_k_equals_v_and_values_bitwise():
    import synth
    z = synth.tie_heavy_logits(3, 33, seed=9)
    idx, val, lse, m_q, _ = oracle.cache_from_logits(z, 33)
    for t in range(3):
        np.testing.assert_array_equal(idx[t], _brute_topk(z[t], 33))
        assert val.dtype == np.float32
        np.testing.assert_array_equal(val[t].view(np.uint32), z[t, idx[t]].view(np.uint32))
    np.testing.assert_allclose(m_q, 0.0, atol=0)


def test_cache_lse_and_tail_mass():
    r = np.random.default_rng(81)
    z = (r.standard_normal((5, 300)) * 2).astype(np.float32)
    idx, val, lse, m_q, _ = oracle.cache_from_logits(z, 10)
    ref = scipy.special.logsumexp(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-13)
    # m_q from the discarded tail equals one minus the kept mass
    kept = np.exp(val.astype(np.float64) - lse[:, None]).sum(axis=1)
    np.testing.assert_allclose(m_q, 1.0 - kept, atol=1e-14)


def test_adaptive_k_exact_masses():
    """Rows with exactly representable masses: k_rho by hand."""
    probs = [Fraction(1, 2), Fraction(1, 4), Fraction(1, 8), Fraction(1, 16), Fraction(1, 16)]
    z = np.log(np.array([float(x) for x in probs]))[None, :]
    perm = np.array([3, 0, 4, 1, 2])
    z = z[:, perm]
    cases = {0.5: 1, 0.6: 2, 0.75: 2, 0.8: 3, 0.875: 3, 0.9: 4, 0.9375: 4, 0.95: 5, 0.99: 5}
    rho = tuple(cases)
    idx, val, lse, m_q, k = oracle.cache_from_logits(z, 2, rho)
    assert list(k[0]) == [cases[r] for r in rho]
    assert abs(m_q[0] - 0.25) < 1e-15
    assert list(idx[0]) == [1, 3]  # the two largest: values 1/2 and 1/4


def test_adaptive_k_against_exact_rational_sums():
    """k_rho on random rows, checked with exact rational cumulative sums of
    the float64 probabilities (rows with a near-tie at rho are skipped)."""
    r = np.random.default_rng(91)
    z = r.standard_normal((8, 60)) * 1.5
    rho = (0.5, 0.9, 0.95)
    _, _, lse, _, k = oracle.cache_from_logits(z, 4, rho)
    for t in range(z.shape[0]):
        p = sorted((float(np.exp(v - lse[t])) for v in z[t]), reverse=True)
        c = Fraction(0)
        cum = []
        for x in p:
            c += Fraction(x)
            cum.append(c)
        for j, rr in enumerate(rho):
            exact = next(i + 1 for i, cc in enumerate(cum) if cc >= Fraction(rr))
            if abs(float(cum[exact - 1]) - rr) < 1e-12:
                continue
            assert k[t, j] == exact


def test_cache_build_matches_head_reconstruction():
    """cache_build = top-K of U g + b (Figure 3 bottom of the top-k gradient paper)."""
    r = np.random.default_rng(101)
    T, d, V, K = 4, 8, 50, 6
    g = r.standard_normal((T, d))
    U = r.standard_normal((V, d))
    b = r.standard_normal(V) * 0.3
    idx, val, lse, m_q, k = oracle.cache_build(g, U, b, K, (0.9,))
    z = np.stack([U @ g[t] + b for t in range(T)])
    for t in range(T):
        np.testing.assert_array_equal(idx[t], _brute_topk(z[t], K))
        np.testing.assert_allclose(val[t], z[t, idx[t]], atol=1e-13)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), atol=1e-12)
    tl = oracle.teacher_logp(val, lse)
    np.testing.assert_allclose(np.exp(tl).sum(axis=1) + m_q, 1.0, atol=1e-13)


# --------------------------------------------------------------------------
# Hard-label cross-entropy term ("The Gradient That Top-k Distillation Never
# Computes", abstract: training with and without the CE term)
# --------------------------------------------------------------------------

def _labels(T, V, seed):
    r = np.random.default_rng(seed)
    y = r.integers(0, V, size=T)
    y[::3] = -1  # unlabelled tokens
    return y


@pytest.mark.parametrize("mode", oracle.MODES)
def test_label_term_against_torch_cross_entropy(mode):
    """The added term and its gradient equal torch's cross_entropy on the
    logits (fp64 autograd), on top of the distillation loss of the mode."""
    h, W, idx, tlp, m_q = _problem(31 + mode, T=6, d=5, V=30, K=6)
    y = _labels(6, 30, 7 + mode)
    y[1] = idx[1, 0]  # a label inside the retained set
    lam = 0.37
    z = oracle.student_logits(h, W)
    L0, dz0, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, mode)
    L1, dz1, _, _ = oracle.loss_rows_from_logits(z, idx, tlp, m_q, mode, labels=y, ce_weight=lam)
    for t in range(6):
        zt = torch.tensor(z[t], dtype=torch.float64, requires_grad=True)
        if y[t] >= 0:
            ce = torch.nn.functional.cross_entropy(zt[None], torch.tensor([int(y[t])]))
            (lam * ce).backward()
            extra, g = float(lam * ce.detach()), zt.grad.numpy()
        else:
            extra, g = 0.0, np.zeros(30)
        assert abs((L1[t] - L0[t]) - extra) < 1e-12
        np.testing.assert_allclose(dz1[t] - dz0[t], g, atol=1e-13)


@pytest.mark.parametrize("mode", [RENORM, TAIL])
def test_label_term_finite_differences(mode):
    h, W, idx, tlp, m_q = _problem(41 + mode, consistent=True)
    y = _labels(h.shape[0], W.shape[0], 3)
    r = oracle.loss_fwd_bwd(h, W, idx, tlp, m_q, mode, scale=0.6, labels=y, ce_weight=0.8)

    def f(hh, WW):
        return oracle.loss_fwd_bwd(hh, WW, idx, tlp, m_q, mode, scale=0.6, labels=y, ce_weight=0.8)["loss"]

    eps = 1e-6
    for name, X, G in (("h", h, r["dh"]), ("W", W, r["dW"])):
        num = np.zeros_like(X)
        for i in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[i] += eps
            Xm[i] -= eps
            num[i] = (f(Xp, W) - f(Xm, W)) / (2 * eps) if name == "h" else \
                     (f(h, Xp) - f(h, Xm)) / (2 * eps)
        err = np.linalg.norm(num - G) / max(np.linalg.norm(G), 1e-300)
        assert err < 1e-6, (name, err)


def test_label_term_alone_is_cross_entropy():
    """With every teacher entry padded out (empty support) the full-mode
    loss is zero and only the label term remains: the mean cross-entropy."""
    r = np.random.default_rng(5)
    T, d, V = 7, 4, 25
    h, W = r.standard_normal((T, d)), r.standard_normal((V, d))
    idx = np.full((T, 3), -1)
    tlp = np.zeros((T, 3))
    y = r.integers(0, V, size=T)
    out = oracle.loss_fwd_bwd(h, W, idx, tlp, None, FULL, labels=y, ce_weight=1.0)
    zt = torch.tensor(h @ W.T)
    ce = float(torch.nn.functional.cross_entropy(zt, torch.tensor(y)))
    assert abs(out["loss"] - ce) < 1e-12


# --------------------------------------------------------------------------
# Exact full-vocabulary KL from a hidden-state teacher cache ("The Gradient
# That Top-k Distillation Never Computes", Figure 3 bottom)
# --------------------------------------------------------------------------

def _hidden_problem(seed, T=5, d=6, dt=7, V=33):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, d)), r.standard_normal((V, d)) / np.sqrt(d),
            r.standard_normal((T, dt)), r.standard_normal((V, dt)) / np.sqrt(dt), 0.3 * r.standard_normal(V))


def test_kl_hidden_against_torch_kl_div():
    h, W, g, U, b = _hidden_problem(1)
    out = oracle.kl_hidden_fwd_bwd(h, W, g, U, b, scale=1.0)
    z = torch.tensor(h @ W.T, requires_grad=True)
    zt = torch.tensor(g @ U.T + b[None, :])
    kl = torch.nn.functional.kl_div(torch.log_softmax(z, 1), torch.log_softmax(zt, 1), log_target=True,
                                    reduction="none").sum(1)
    kl.sum().backward()
    np.testing.assert_allclose(out["loss_tok"], kl.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["dh"], z.grad.numpy() @ W, atol=1e-13)
    np.testing.assert_allclose(out["dW"], z.grad.numpy().T @ h, atol=1e-13)
    np.testing.assert_allclose(out["lse_t"], scipy.special.logsumexp(g @ U.T + b[None, :], axis=1), rtol=1e-14)


def test_kl_hidden_finite_differences():
    h, W, g, U, b = _hidden_problem(2, T=3, d=4, dt=5, V=11)
    out = oracle.kl_hidden_fwd_bwd(h, W, g, U, b, scale=0.5)

    def f(hh, WW):
        return oracle.kl_hidden_fwd_bwd(hh, WW, g, U, b, scale=0.5)["loss"]

    eps = 1e-6
    for name, X, G in (("h", h, out["dh"]), ("W", W, out["dW"])):
        num = np.zeros_like(X)
        for i in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[i] += eps
            Xm[i] -= eps
            num[i] = (f(Xp, W) - f(Xm, W)) / (2 * eps) if name == "h" else (f(h, Xp) - f(h, Xm)) / (2 * eps)
        assert np.linalg.norm(num - G) / np.linalg.norm(G) < 1e-6, name


def test_kl_hidden_self_distillation_is_zero():
    """Teacher = student (U = W, g = h, no bias): KL and every gradient vanish."""
    h, W, _, _, _ = _hidden_problem(3)
    out = oracle.kl_hidden_fwd_bwd(h, W, h, W, None)
    assert abs(out["loss"]) < 1e-14
    assert np.abs(out["dh"]).max() < 1e-14 and np.abs(out["dW"]).max() < 1e-14


def test_kl_hidden_equals_cached_full_support():
    """A top-K cache that keeps every index (K = V) of the same teacher gives
    the same loss and gradients through the full-vocabulary mode."""
    h, W, g, U, b = _hidden_problem(4)
    out = oracle.kl_hidden_fwd_bwd(h, W, g, U, b)
    zt = g @ U.T + b[None, :]
    V = zt.shape[1]
    idx = np.tile(np.arange(V), (zt.shape[0], 1))
    tlp = zt - scipy.special.logsumexp(zt, axis=1)[:, None]
    ref = oracle.loss_fwd_bwd(h, W, idx, tlp, None, FULL)
    assert abs(out["loss"] - ref["loss"]) < 1e-12
    np.testing.assert_allclose(out["dh"], ref["dh"], atol=1e-13)
    np.testing.assert_allclose(out["dW"], ref["dW"], atol=1e-13)


def test_tail_reverse_at_full_support_is_dense_reverse_kl():
    """K = V: no tail on either side, and the tail-token reverse KL is the
    dense KL(p || q) with gradient p (log p - log q - KL)."""
    from torch.distributions import Categorical, kl_divergence
    r = np.random.default_rng(21)
    T, d, V = 4, 5, 17
    h, W = r.standard_normal((T, d)), r.standard_normal((V, d))
    zt_teacher = r.standard_normal((T, V))
    tlp = zt_teacher - scipy.special.logsumexp(zt_teacher, axis=1)[:, None]
    idx = np.tile(np.arange(V), (T, 1))
    z = oracle.student_logits(h, W)
    L, dz, _, m_p = oracle.loss_rows_from_logits(z, idx, tlp, np.zeros(T), TAIL_REVERSE)
    assert np.abs(m_p).max() < 1e-15
    for t in range(T):
        zt = torch.tensor(z[t], requires_grad=True)
        kl = kl_divergence(Categorical(logits=zt), Categorical(logits=torch.tensor(tlp[t])))
        kl.backward()
        assert abs(L[t] - float(kl.detach())) < 1e-12
        np.testing.assert_allclose(dz[t], zt.grad.numpy(), atol=1e-13)


# --------------------------------------------------------------------------
# Tail-corrected top-k reverse KL ("Unbiased Top-k Estimation for On-Policy
# Distillation", abstract and Figure 1)
# --------------------------------------------------------------------------

def _reverse_kl_torch(z_row, logq_row):
    from torch.distributions import Categorical, kl_divergence
    zt = torch.tensor(z_row, requires_grad=True)
    kl = kl_divergence(Categorical(logits=zt), Categorical(logits=torch.tensor(logq_row)))
    kl.backward()
    return float(kl.detach()), zt.grad.numpy()


def test_reverse_tt_is_unbiased_over_the_sampled_token():
    """Averaged over the sampled token y ~ p (every y enumerated, weighted by
    the student's probability), the loss estimate is the full reverse KL
    KL(p || q) and the logit gradient is its exact gradient."""
    r = np.random.default_rng(17)
    V, K = 23, 5
    z = r.standard_normal(V) * 1.3
    zt = r.standard_normal(V) * 1.1
    logq = zt - scipy.special.logsumexp(zt)
    S = r.choice(V, size=K, replace=False)
    p = scipy.special.softmax(z)
    Lbar, gbar = 0.0, np.zeros(V)
    for y in range(V):
        L, dz, _, _ = oracle.loss_rows_from_logits(z[None], S[None], logq[S][None], None, REVERSE_TT,
                                                   labels=np.array([y]), tlp_labels=np.array([logq[y]]))
        Lbar += p[y] * L[0]
        gbar += p[y] * dz[0]
    kl, grad = _reverse_kl_torch(z, logq)
    assert abs(Lbar - kl) < 1e-12
    np.testing.assert_allclose(gbar, grad, atol=1e-13)


def test_reverse_tt_sample_inside_support_or_absent_adds_nothing():
    r = np.random.default_rng(18)
    V, K = 19, 4
    z = r.standard_normal((3, V))
    logq = r.standard_normal((3, V))
    logq -= scipy.special.logsumexp(logq, axis=1)[:, None]
    S = np.stack([r.choice(V, size=K, replace=False) for _ in range(3)])
    tl = np.take_along_axis(logq, S, 1)
    y = np.array([S[0, 2], -1, S[2, 0]])
    L0, d0, _, _ = oracle.loss_rows_from_logits(z, S, tl, None, REVERSE_TT)
    L1, d1, _, _ = oracle.loss_rows_from_logits(z, S, tl, None, REVERSE_TT, labels=y,
                                                tlp_labels=np.array([logq[0, y[0]], 0.0, logq[2, y[2]]]))
    np.testing.assert_array_equal(L0, L1)
    np.testing.assert_array_equal(d0, d1)
    # full support: the top-k part alone is the dense reverse KL
    Sfull = np.tile(np.arange(V), (3, 1))
    Lf, df, _, _ = oracle.loss_rows_from_logits(z, Sfull, logq, None, REVERSE_TT)
    for t in range(3):
        kl, grad = _reverse_kl_torch(z[t], logq[t])
        assert abs(Lf[t] - kl) < 1e-12
        np.testing.assert_allclose(df[t], grad, atol=1e-13)


def test_int8_hidden_cache_codes():
    """Codes within [-127, 127], the largest magnitude hits 127, every value
    is reconstructed within half a step, and zero rows stay zero."""
    r = np.random.default_rng(31)
    g = (r.standard_normal((9, 70)) * np.array([0.1, 1, 5, 30, 1e-3, 2, 2, 2, 2])[:, None]).astype(np.float32)
    g[3, 5] = -g[3].__abs__().max() * 1.5  # a negative extreme
    g[8] = 0.0
    q, s = oracle.quantize_hidden_int8(g)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert s[8] == 0 and np.all(q[8] == 0)
    for t in range(8):
        assert np.abs(q[t].astype(np.int32)).max() == 127
        err = np.abs(g[t].astype(np.float64) - s[t] * q[t].astype(np.float64))
        assert err.max() <= 0.5 * s[t] * (1 + 1e-6)


def test_kl_hidden_int8_equals_dequantized_teacher():
    """The int8 path (codes + per-position scale) is the float path on the
    dequantized hidden states s * codes."""
    h, W, g, U, b = _hidden_problem(8, T=6, d=5, dt=9, V=29)
    q, s = oracle.quantize_hidden_int8(g)
    a = oracle.kl_hidden_fwd_bwd(h, W, q.astype(np.float64), U, b, g_scale=s)
    ref = oracle.kl_hidden_fwd_bwd(h, W, q.astype(np.float64) * s.astype(np.float64)[:, None], U, b)
    assert abs(a["loss"] - ref["loss"]) < 1e-13
    np.testing.assert_allclose(a["dh"], ref["dh"], atol=1e-14)
    np.testing.assert_allclose(a["lse_t"], ref["lse_t"], atol=1e-13)


# --------------------------------------------------------------------------
# Teacher recovery from k cached log-probabilities ("The Gradient That Top-k
# Distillation Never Computes", abstract and Table 1: exact from k = d + 1)
# --------------------------------------------------------------------------

def test_teacher_recovery_transition_at_d_plus_1():
    r = np.random.default_rng(41)
    T, d, V = 4, 12, 200
    U = r.standard_normal((V, d)) / np.sqrt(d)
    b = 0.3 * r.standard_normal(V)
    g = r.standard_normal((T, d))
    z = g @ U.T + b[None, :]
    logq = z - scipy.special.logsumexp(z, axis=1)[:, None]
    order = np.argsort(-z, axis=1)
    for k, exact in ((d - 1, False), (d, False), (d + 1, True), (3 * d, True)):
        idx = order[:, :k]
        tl = np.take_along_axis(logq, idx, 1)
        gh, ch = oracle.recover_teacher_hidden(idx, tl, U, b)
        zh = gh @ U.T + b[None, :]
        logqh = zh - scipy.special.logsumexp(zh, axis=1)[:, None]
        kl = np.sum(np.exp(logq) * (logq - logqh), axis=1)
        if exact:
            np.testing.assert_allclose(gh, g, atol=1e-9)
            np.testing.assert_allclose(ch, scipy.special.logsumexp(z, axis=1), atol=1e-9)
            assert kl.max() < 1e-15
        else:
            # below d + 1 the retained set does not determine the teacher
            assert kl.min() > 1e-6, (k, kl)
