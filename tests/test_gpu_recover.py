"""GPU parity of kd_teacher_recover (teacher hidden state from k >= d + 1
cached log-probabilities) against the fp64 CPU oracle on the same fp32
cache: the recovered state and logsumexp agree to 1e-5 relative, and both
match the generating teacher to the precision the fp32 cache allows."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
import top_kd_loss_amd as kd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _teacher(T, d, V, seed):
    g, U, b = synth.teacher_head(T, d, V, seed=seed)
    z = synth.as_f64(g) @ synth.as_f64(U).T + b.double().numpy()[None, :]
    logq = z - scipy.special.logsumexp(z, axis=1)[:, None]
    return g, U, b, z, logq


@pytest.mark.parametrize("d,k", [(64, 65), (64, 130), (96, 160), (127, 128)])
def test_recover_matches_oracle(d, k):
    T, V = 24, 3000
    g, U, b, z, logq = _teacher(T, d, V, seed=d + k)
    idx = np.argsort(-z, axis=1)[:, :k].astype(np.int32)
    tlp = np.take_along_axis(logq, idx.astype(np.int64), 1).astype(np.float32)
    gh, ch = kd.teacher_recover(torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV), U.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    gh, ch = gh.cpu().numpy(), ch.cpu().numpy()
    rg, rc = oracle.recover_teacher_hidden(idx, tlp, synth.as_f64(U), b.double().numpy())
    np.testing.assert_allclose(gh, rg, rtol=1e-5, atol=1e-5 * np.abs(rg).max())
    np.testing.assert_allclose(ch, rc, rtol=1e-5, atol=1e-5)
    # the full teacher distribution comes back (fp32 cache rounding aside)
    zh = gh.astype(np.float64) @ synth.as_f64(U).T + b.double().numpy()[None, :]
    logqh = zh - scipy.special.logsumexp(zh, axis=1)[:, None]
    kl = np.sum(np.exp(logq) * (logq - logqh), axis=1)
    print(f"d={d} k={k}: max KL(q || q_hat) = {kl.max():.2e}")
    assert kl.max() < 1e-6


@pytest.mark.parametrize("d,k", [(64, 65), (64, 130), (96, 160), (127, 128)])
def test_multi_workgroup_solver_matches_lds_solver(d, k):
    """Both fp64 Householder solvers on the same small systems."""
    T, V = 24, 3000
    g, U, b, z, logq = _teacher(T, d, V, seed=d + k)
    idx = np.argsort(-z, axis=1)[:, :k].astype(np.int32)
    tlp = np.take_along_axis(logq, idx.astype(np.int64), 1).astype(np.float32)
    args = (torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV), U.to(DEV), b.to(DEV))
    a = kd.teacher_recover(*args, multi_workgroup=False)
    m = kd.teacher_recover(*args, multi_workgroup=True)
    torch.cuda.synchronize()
    for x, y in zip(a, m):
        x, y = x.cpu().numpy(), y.cpu().numpy()
        np.testing.assert_allclose(y, x, rtol=1e-6, atol=1e-6 * np.abs(x).max())


@pytest.mark.timeout(600)
def test_recover_qwen_width_transition_at_d_plus_1():
    """A teacher head of real width (d = 2048; V = 8192 rows of U ~ N(0, 1/d),
    b ~ N(0, 0.1)), its top-k fp32 log-probabilities cached: with k = d + 1
    and k = 3000 the multi-workgroup least-squares solution matches the
    oracle's and gives back the full distribution; with k = d (one
    equation short) the system is underdetermined, the minimum-norm
    solution matches the oracle's and KL(q || q_hat) > 0."""
    T, d, V = 3, 2048, 8192
    g, U, b, z, logq = _teacher(T, d, V, seed=41)
    Ud, bd = U.to(DEV), b.to(DEV)
    U64, b64 = synth.as_f64(U), b.double().numpy()
    kls = {}
    for k in (d + 1, 3000, d):
        idx = np.argsort(-z, axis=1)[:, :k].astype(np.int32)
        tlp = np.take_along_axis(logq, idx.astype(np.int64), 1).astype(np.float32)
        gh, ch = kd.teacher_recover(torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV), Ud, bd)
        torch.cuda.synchronize()
        gh, ch = gh.cpu().numpy(), ch.cpu().numpy()
        rg, rc = oracle.recover_teacher_hidden(idx, tlp, U64, b64)
        np.testing.assert_allclose(gh, rg, rtol=1e-5, atol=1e-5 * np.abs(rg).max())
        np.testing.assert_allclose(ch, rc, rtol=1e-5, atol=1e-5)
        zh = gh.astype(np.float64) @ U64.T + b64[None, :]
        logqh = zh - scipy.special.logsumexp(zh, axis=1)[:, None]
        kls[k] = np.sum(np.exp(logq) * (logq - logqh), axis=1)
        print(f"d={d} k={k}: KL(q || q_hat) per position {kls[k]}")
    assert kls[d + 1].max() < 1e-4 and kls[3000].max() < 1e-4
    assert kls[d].min() > 100 * max(kls[d + 1].max(), kls[3000].max(), 1e-12), kls


def test_recover_rejects_k_below_d_plus_1_and_flags_bad_indices():
    T, d, V = 4, 64, 500
    g, U, b, z, logq = _teacher(T, d, V, seed=3)
    idx = np.argsort(-z, axis=1)[:, :d].astype(np.int32)
    tlp = np.take_along_axis(logq, idx.astype(np.int64), 1).astype(np.float32)
    with pytest.raises(kd.KDError):
        kd.teacher_recover(torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV), U.to(DEV), b.to(DEV),
                           multi_workgroup=False)
    idx = np.argsort(-z, axis=1)[:, :d + 8].astype(np.int32)
    tlp = np.take_along_axis(logq, idx.astype(np.int64), 1).astype(np.float32)
    idx[2, 3] = V  # out of range
    for mw in (False, True):
        gh, ch = kd.teacher_recover(torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV), U.to(DEV),
                                    b.to(DEV), multi_workgroup=mw)
        torch.cuda.synchronize()
        assert np.isnan(ch.cpu().numpy()[2]) and np.isfinite(ch.cpu().numpy()[[0, 1, 3]]).all()
