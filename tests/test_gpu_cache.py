"""GPU parity of the teacher-cache build (kd_topk_rows, kd_topk_cache_build)
against the fp64 CPU oracle.

Top-K on identical fp32 logits must match bit-exactly (indices and value
bits; ties to the lower index).  lse and m_q: absolute 1e-5.  k_rho: the
GPU's k is accepted when the oracle's fp64 cumulative mass satisfies
C(k) >= rho - 1e-5 and C(k-1) < rho + 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_kd_loss_amd as kd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RHO = (0.9, 0.95)


def _krho_ok(z_row64, lse, rho, k):
    p = np.sort(np.exp(z_row64 - lse))[::-1]
    c = np.cumsum(p)
    ck = c[k - 1]
    ckm1 = c[k - 2] if k >= 2 else 0.0
    return ck >= rho - 1e-5 and ckm1 < rho + 1e-5


def _check_logp(glp, rv, rlse, rows_ok):
    """teacher_logp = val - lse against the oracle's fp64 difference: within
    one fp32 ulp of the value plus 1e-6 (the GPU logsumexp's own rounding)."""
    ref = oracle.teacher_logp(rv, rlse)[rows_ok]
    g = glp[rows_ok].astype(np.float64)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(g[~fin], ref[~fin])
    ulp = np.spacing(np.abs(ref[fin]).astype(np.float32)).astype(np.float64)
    err = np.abs(g[fin] - ref[fin])
    assert np.all(err <= ulp + 1e-6), float((err - ulp).max())
    return float((err / ulp).max()) if err.size else 0.0


def _check_rows(z, K, rho=RHO):
    zt = torch.from_numpy(z).to(DEV)
    o = kd.topk_rows(zt, K, rho)
    torch.cuda.synchronize()
    gi, gv = o.idx.cpu().numpy(), o.val.cpu().numpy()
    glse, gmq, gk = o.lse.cpu().numpy(), o.m_q.cpu().numpy(), o.k_rho.cpu().numpy()
    ri, rv, rlse, rmq, rk = oracle.cache_from_logits(z, K, rho)
    np.testing.assert_array_equal(gi, ri)
    np.testing.assert_array_equal(gv.view(np.uint32), rv.view(np.uint32))
    fin = np.isfinite(rlse)
    # lse within 1e-5, or within one fp32 ulp of it for |lse| >= 128 (the
    # fp32 result's own rounding)
    tol = np.maximum(1e-5, np.spacing(np.abs(rlse[fin]).astype(np.float32)).astype(np.float64))
    assert np.all(np.abs(glse[fin].astype(np.float64) - rlse[fin]) <= tol), \
        float(np.max(np.abs(glse[fin].astype(np.float64) - rlse[fin]) - tol))
    np.testing.assert_allclose(gmq[fin], rmq[fin], atol=1e-5, rtol=0)
    _check_logp(o.teacher_logp.cpu().numpy(), rv, rlse, fin)
    exact = 0
    for t in range(z.shape[0]):
        if not fin[t]:
            continue
        z64 = z[t].astype(np.float64)
        for j, r in enumerate(rho):
            assert _krho_ok(z64, rlse[t], r, int(gk[t, j])), (t, r, int(gk[t, j]), int(rk[t, j]))
            exact += int(gk[t, j] == rk[t, j])
    return exact / max(1, z.shape[0] * len(rho))


@pytest.mark.parametrize("K", [1, 8, 64, 256, 1024])
def test_rows_zipf_bit_exact(K):
    z = synth.zipf_teacher_logits(40, 5000, seed=K)
    frac = _check_rows(z, K)
    print(f"K={K} k_rho exact-match fraction {frac:.3f}")


@pytest.mark.parametrize("shift,scale", [(300.0, 1.1), (150.0, 30.0), (-400.0, 30.0)])
def test_rows_large_magnitude_logits(shift, scale):
    """Logits far from zero (a softmax is shift invariant, so these are valid
    teacher rows).  A narrow row near 300 stays in the single-read path; a
    spread of 30 puts the K-th value about 40 below the row maximum, so the
    rows reach the exact kernel, with maxima near 270 (where its first digit's
    bins are 64 wide) or with every logit negative."""
    r = np.random.default_rng(int(abs(shift)) + int(scale))
    z = (r.standard_normal((64, 20000)) * scale + shift).astype(np.float32)
    _check_rows(z, 64)


def test_rows_vocab_above_2_18_exact_kernel_only():
    """V >= 2^18 does not fit the fast kernel's 18-bit bin counts: every row
    takes the exact radix-digit kernel (its maximum read, three digits, the
    k_rho refinement), here with rows near zero and far from it."""
    r = np.random.default_rng(44)
    z = (r.standard_normal((12, 300_001)) * 1.1).astype(np.float32)
    z[4:8] += np.float32(170.0)
    z[8:] = (r.standard_normal((4, 300_001)) * 25.0 - 300.0).astype(np.float32)
    _check_rows(z, 64)


def test_cache_build_vocab_above_2_18():
    T, d, V, K = 20, 64, 270_000, 32
    g, U, b = synth.teacher_head(T, d, V, seed=6)
    o = kd.cache_build(g.to(DEV), U.to(DEV), b.to(DEV), K, RHO)
    torch.cuda.synchronize()
    z = synth.as_f64(g) @ synth.as_f64(U).T + b.double().numpy()[None, :]
    _, _, rlse, rmq, _ = oracle.cache_from_logits(z, K, RHO)
    gi = o.idx.cpu().numpy()
    np.testing.assert_allclose(o.lse.cpu().numpy(), rlse, atol=1e-4)
    np.testing.assert_allclose(o.m_q.cpu().numpy(), rmq, atol=1e-5)
    for t in range(T):
        kth = np.sort(z[t])[::-1][K - 1]
        assert np.all(z[t, gi[t]] >= kth - 2e-4) and len(set(gi[t].tolist())) == K
        for j, rr in enumerate(RHO):
            assert _krho_ok(z[t], rlse[t], rr, int(o.k_rho.cpu().numpy()[t, j]))


def test_rows_ties_signed_zero_neg_inf():
    z = synth.tie_heavy_logits(24, 3001, seed=1, step=0.25, span=2.0)
    z[0, :] = 0.5                      # one big tie: lowest indices win
    z[1, ::2] = -0.0
    z[1, 1::2] = 0.0
    z[2, 100:2000] = -np.inf
    z[3, :] = -np.inf
    z[3, 17] = 1.0
    for K in (1, 7, 100, 1024):
        zz = z.copy()
        if K > 1:
            zz[3] = z[3]
            zz[3, :K] = 0.25           # keep row 3 with at least K finite values
        _check_rows(zz, K, rho=(0.5,))


@pytest.mark.timeout(300)
def test_rows_full_vocab_width_256_rows():
    """256 rows as wide as the Qwen vocabulary (V = 151,936), K = 256 and both
    k_rho targets: 128 Zipf-like teacher rows and 128 Gaussian rows
    N(0, 1.1) (the cache-build workload's logit statistics)."""
    r = np.random.default_rng(3)
    zg = (r.standard_normal((128, 151936)) * np.sqrt(1.1)).astype(np.float32)
    zz = synth.zipf_teacher_logits(128, 151936, seed=3)
    for name, z in (("gaussian", zg), ("zipf", zz)):
        frac = _check_rows(z, 256)
        print(f"{name}: 128 rows bit-exact; k_rho exact-match fraction {frac:.3f}")


def test_rows_k_equals_v_and_ragged():
    z = synth.tie_heavy_logits(5, 77, seed=4)
    _check_rows(z, 77, rho=(0.9,))
    z = synth.zipf_teacher_logits(9, 1023, seed=4)
    _check_rows(z, 513)


def test_cache_build_small_with_bias():
    T, d, V, K = 300, 128, 5000, 37
    g, U, b = synth.teacher_head(T, d, V, seed=2)
    o = kd.cache_build(g.to(DEV), U.to(DEV), b.to(DEV), K, RHO)
    torch.cuda.synchronize()
    z = synth.as_f64(g) @ synth.as_f64(U).T + b.double().numpy()[None, :]
    ri, rv, rlse, rmq, rk = oracle.cache_from_logits(z, K, RHO)
    gi, gv = o.idx.cpu().numpy(), o.val.cpu().numpy()
    np.testing.assert_allclose(o.lse.cpu().numpy(), rlse, atol=1e-4)
    np.testing.assert_allclose(o.m_q.cpu().numpy(), rmq, atol=1e-5)
    # values are the logits at the returned indices (fp32 accumulation)
    np.testing.assert_allclose(gv, np.take_along_axis(z, gi.astype(np.int64), 1), atol=1e-4)
    # the returned set is a valid top-K of the fp64 logits up to fp32 rounding
    for t in range(T):
        kth = np.sort(z[t])[::-1][K - 1]
        assert np.all(z[t, gi[t]] >= kth - 2e-4)
        assert len(set(gi[t].tolist())) == K
    agree = np.mean([len(set(gi[t]) & set(ri[t])) / K for t in range(T)])
    assert agree > 0.99, agree
    # teacher_logp: the fp64 log-probabilities at the returned entries, up to
    # the fp32 accumulation of the logits
    tl = o.teacher_logp.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(tl, np.take_along_axis(z, gi.astype(np.int64), 1) - rlse[:, None], atol=2e-4)
    gk = o.k_rho.cpu().numpy()
    for t in range(0, T, 7):
        for j, r in enumerate(RHO):
            assert _krho_ok(z[t], rlse[t], r, int(gk[t, j]))


def test_cache_build_ragged_last_token_block():
    """T = 2 * 2048 + 300: the cache build works in blocks of 2048 tokens
    (one GEMM and one row pass per block); the last block is partial.  Every
    row against the oracle."""
    T, d, V, K = 2 * 2048 + 300, 64, 3000, 16
    g, U, b = synth.teacher_head(T, d, V, seed=12)
    o = kd.cache_build(g.to(DEV), U.to(DEV), b.to(DEV), K, RHO)
    torch.cuda.synchronize()
    z = synth.as_f64(g) @ synth.as_f64(U).T + b.double().numpy()[None, :]
    _, _, rlse, rmq, _ = oracle.cache_from_logits(z, K, RHO)
    gi, gv, gk = o.idx.cpu().numpy(), o.val.cpu().numpy(), o.k_rho.cpu().numpy()
    np.testing.assert_allclose(o.lse.cpu().numpy(), rlse, atol=1e-4)
    np.testing.assert_allclose(o.m_q.cpu().numpy(), rmq, atol=1e-5)
    np.testing.assert_allclose(gv, np.take_along_axis(z, gi.astype(np.int64), 1), atol=1e-4)
    kth = -np.sort(-z, axis=1)[:, K - 1]
    assert np.all(np.take_along_axis(z, gi.astype(np.int64), 1) >= kth[:, None] - 2e-4)
    assert all(len(set(gi[t].tolist())) == K for t in range(T))
    for t in range(0, T, 97):
        for j, r in enumerate(RHO):
            assert _krho_ok(z[t], rlse[t], r, int(gk[t, j])), (t, r)


@pytest.mark.parametrize("T,d,V,K", [(1, 64, 1000, 8), (50, 64, 7, 7), (33, 128, 100, 3)])
def test_cache_build_single_token_and_tiny_vocab(T, d, V, K):
    """One token; a vocabulary of 7 with K = V and one of 100 (a single
    partial 256-row tile of the GEMM, one partial row of the row pass)."""
    g, U, b = synth.teacher_head(T, d, V, seed=13)
    o = kd.cache_build(g.to(DEV), U.to(DEV), b.to(DEV), K, RHO)
    torch.cuda.synchronize()
    z = synth.as_f64(g) @ synth.as_f64(U).T + b.double().numpy()[None, :]
    _, _, rlse, rmq, _ = oracle.cache_from_logits(z, K, RHO)
    gi, gv, gk = o.idx.cpu().numpy(), o.val.cpu().numpy(), o.k_rho.cpu().numpy()
    np.testing.assert_allclose(o.lse.cpu().numpy(), rlse, atol=1e-4)
    np.testing.assert_allclose(o.m_q.cpu().numpy(), rmq, atol=1e-5)
    np.testing.assert_allclose(gv, np.take_along_axis(z, gi.astype(np.int64), 1), atol=1e-4)
    kth = -np.sort(-z, axis=1)[:, K - 1]
    assert np.all(np.take_along_axis(z, gi.astype(np.int64), 1) >= kth[:, None] - 2e-4)
    assert all(len(set(gi[t].tolist())) == K for t in range(T))
    for t in range(T):
        for j, r in enumerate(RHO):
            assert _krho_ok(z[t], rlse[t], r, int(gk[t, j])), (t, r)


def test_cache_build_student_head_no_bias():
    T, d, V, K = 64, 64, 1024, 16
    h, W = synth.student_head(T, d, V, seed=9)
    o = kd.cache_build(h.to(DEV), W.to(DEV), None, K)
    torch.cuda.synchronize()
    z = synth.as_f64(h) @ synth.as_f64(W).T
    _, _, rlse, rmq, _ = oracle.cache_from_logits(z, K)
    np.testing.assert_allclose(o.lse.cpu().numpy(), rlse, atol=1e-4)
    np.testing.assert_allclose(o.m_q.cpu().numpy(), rmq, atol=1e-5)
    assert o.k_rho.shape == (T, 0)


def test_rows_huge_tie_takes_lowest_indices():
    """More equal keys than the candidate buffer holds: the ordered pass
    must still return the lowest indices."""
    z = np.full((3, 10000), 0.7, np.float32)
    z[1, 5000:] = -0.0
    z[1, :5000] = 0.0
    z[2, 9000:] = 3.0
    _check_rows(z, 1024, rho=(0.5, 0.9))


def test_rows_fine_ties_wide_rows():
    """Many small groups of equal values spread over a wide row: candidate
    bins hold ties that must resolve to the lower indices."""
    z = synth.tie_heavy_logits(12, 40000, seed=7, step=1.0 / 64.0, span=3.0)
    for K in (5, 256, 1000):
        _check_rows(z, K, rho=(0.3, 0.9, 0.95))


def test_rows_bitwise_deterministic():
    r = np.random.default_rng(11)
    z = torch.from_numpy((r.standard_normal((64, 151936)) * 1.05).astype(np.float32)).to(DEV)
    a = kd.topk_rows(z, 256, RHO)
    b = kd.topk_rows(z, 256, RHO)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y)


def test_rows_single_pass_collection_no_rho():
    """Without k_rho targets the candidates are collected during the
    histogram pass above a bound from the threads' maxima (K <= 512) or by
    the separate pass (K > 512); ties, signed zeros, -inf and a tie larger
    than the candidate buffer go through both."""
    z = synth.tie_heavy_logits(12, 40000, seed=7, step=1.0 / 64.0, span=3.0)
    for K in (1, 5, 256, 512, 513, 1000):
        _check_rows(z, K, rho=())
    h = np.full((3, 10000), 0.7, np.float32)
    h[1, 5000:] = -0.0
    h[1, :5000] = 0.0
    h[2, 9000:] = 3.0
    h[2, :100] = -np.inf
    for K in (1, 300, 1024):
        _check_rows(h, K, rho=())


@pytest.mark.parametrize("d", [64, 192, 320])
@pytest.mark.parametrize("rho", [(), RHO])
def test_cache_build_integer_logits_bit_exact(rho, d):
    """Small-integer hidden states and head rows make every logit an exact
    integer in fp32 (|z| < 2^24), so the cache build's top-K (through the
    GEMM's per-tile maxima) must equal the oracle's bit for bit, with heavy
    ties resolved to the lower index.  d = 64, 192, 320 runs the GEMM's k-loop
    over 1, 3 and 5 slices of 64 (the odd counts end on the other register
    set)."""
    T, V = 50, 5000
    r = np.random.default_rng(31 + d)
    g = r.integers(-2, 3, size=(T, d)).astype(np.float32)
    U = r.integers(-2, 3, size=(V, d)).astype(np.float32)
    b = r.integers(-3, 4, size=V).astype(np.float32)
    z = g.astype(np.float64) @ U.astype(np.float64).T + b[None, :]
    for K in (1, 16, 300):
        o = kd.cache_build(torch.from_numpy(g).to(torch.bfloat16).to(DEV),
                           torch.from_numpy(U).to(torch.bfloat16).to(DEV), torch.from_numpy(b).to(DEV), K, rho)
        torch.cuda.synchronize()
        ri, rv, rlse, rmq, rk = oracle.cache_from_logits(z.astype(np.float32), K, rho)
        np.testing.assert_array_equal(o.idx.cpu().numpy(), ri)
        np.testing.assert_array_equal(o.val.cpu().numpy().view(np.uint32), rv.view(np.uint32))
        np.testing.assert_allclose(o.lse.cpu().numpy(), rlse, atol=1e-5, rtol=0)
        np.testing.assert_allclose(o.m_q.cpu().numpy(), rmq, atol=1e-5, rtol=0)


def test_rows_single_pass_degenerate_bounds():
    """Single-read path with a bound of -inf (fewer finite partial maxima
    than K): K = V on short rows, and wide rows that are mostly -inf (the
    collection overflows and the exact kernel takes the row)."""
    r = np.random.default_rng(43)
    z = r.standard_normal((6, 300)).astype(np.float32)
    _check_rows(z, 300, rho=())
    _check_rows(z, 100, rho=())
    w = np.full((4, 40000), -np.inf, np.float32)
    for t in range(4):
        pos = r.choice(40000, 300 + 400 * t, replace=False)
        w[t, pos] = r.standard_normal(len(pos)).astype(np.float32)
    for K in (50, 300, 450):
        _check_rows(w, K, rho=())


@pytest.mark.timeout(300)
def test_rows_deferred_crossing_bins_match_in_kernel_pass():
    """512 rows of N(0, 1.1) logits over V = 151,936 with both k_rho targets:
    about 5% of them have a crossing bin whose count and mass leave k_rho
    open, which kd_topk_rows hands to its separate collecting launch and
    kd_topk_rows_noalloc reads again in the row's own workgroup.  Every
    output is bitwise equal between the two, and lse and k_rho match the
    oracle's fp64 logsumexp and cumulative mass on 48 sampled rows (which
    rows were deferred is not visible through the ABI)."""
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((512, 151936)) * np.sqrt(1.1)).astype(np.float32)
    zt = torch.from_numpy(z).to(DEV)
    a = kd.topk_rows(zt, 256, RHO)
    b = kd.topk_rows_noalloc(zt, 256, RHO)
    torch.cuda.synchronize()
    for name, x, y in zip(a._fields, a, b):
        xx = x.view(torch.int32) if x.dtype == torch.float32 else x
        yy = y.view(torch.int32) if y.dtype == torch.float32 else y
        assert torch.equal(xx, yy), name
    gk, glse = a.k_rho.cpu().numpy(), a.lse.cpu().numpy()
    rows = rng.choice(512, 48, replace=False)
    for t in rows:
        z64 = z[t].astype(np.float64)
        lse = float(np.logaddexp.reduce(z64))
        assert abs(glse[t] - lse) <= 1e-5
        for j, r in enumerate(RHO):
            assert _krho_ok(z64, lse, r, int(gk[t, j])), (t, r, int(gk[t, j]))
