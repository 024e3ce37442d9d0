"""GPU parity of the token-block option (kd_topk_loss_fwd_bwd_tokblock)
against the fp64 CPU oracle.

The dense modes keep each block's logits (bf16 exp(z - m)) instead of
recomputing them in the backward.  Bar as for the chunked call: loss
relative error <= 1e-3, dh and dW relative Frobenius error <= 1e-2.  The
forward outputs (loss, per-token loss, lse, m_p) must equal the chunked
call's bitwise (same tiles, same order)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_kd_loss_amd as kd
from _inputs import rel_err, rel_fro, teacher_cache

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DENSE = [kd.TAIL, kd.FULL, kd.TAIL_REVERSE, kd.REVERSE_TT]


def _run(h, W, idx, tlp, mq, mode, token_block=0, chunk=8192):
    out = kd.loss_fwd_bwd(h.to(DEV), W.to(DEV), torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV),
                          torch.from_numpy(mq).to(DEV), mode=mode, chunk=chunk, token_block=token_block)
    torch.cuda.synchronize()
    return {k: getattr(out, k).cpu().numpy() for k in out._fields}


def _compare(g, r, tag):
    assert np.isfinite(g["dh"]).all() and np.isfinite(g["dW"]).all(), tag
    assert rel_err(g["loss"], r["loss"]) <= 1e-3, (tag, float(g["loss"]), r["loss"])
    np.testing.assert_allclose(g["lse"], r["lse"], atol=2e-4, rtol=0, err_msg=tag)
    np.testing.assert_allclose(g["m_p"], r["m_p"], atol=2e-4, rtol=0, err_msg=tag)
    e_dh, e_dw = rel_fro(g["dh"], r["dh"]), rel_fro(g["dW"], r["dW"])
    print(f"{tag}: loss={float(g['loss']):.6f} ref={r['loss']:.6f} dh={e_dh:.2e} dW={e_dw:.2e}")
    assert e_dh <= 1e-2 and e_dw <= 1e-2, (tag, e_dh, e_dw)


@pytest.mark.parametrize("mode", DENSE + [kd.RENORM])
def test_tiny_single_block(mode):
    T, d, V, K = 64, 64, 1024, 8
    h, W = synth.student_head(T, d, V, seed=0)
    idx, tlp, mq = teacher_cache(T, V, K, seed=0)
    g = _run(h, W, idx, tlp, mq, mode, token_block=256)
    r = oracle.loss_fwd_bwd(synth.as_f64(h), synth.as_f64(W), idx, tlp, mq, mode)
    _compare(g, r, f"tiny token-block mode={oracle.MODE_NAMES[mode]}")


@pytest.mark.parametrize("mode", DENSE)
def test_ragged_several_blocks(mode):
    """Three token blocks (256, 256, 188 tokens: dW accumulated over them),
    a vocabulary that is not a multiple of the tile, padding slots."""
    T, d, V, K = 700, 128, 2500, 13
    h, W = synth.student_head(T, d, V, seed=3)
    idx, tlp, mq = teacher_cache(T, V, K, seed=3)
    idx[5, 3:] = -1
    g = _run(h, W, idx, tlp, mq, mode, token_block=200)  # rounded up to 256
    r = oracle.loss_fwd_bwd(synth.as_f64(h), synth.as_f64(W), idx, tlp, mq, mode)
    _compare(g, r, f"ragged token-block mode={oracle.MODE_NAMES[mode]}")
    c = _run(h, W, idx, tlp, mq, mode, chunk=700)
    for key in ("loss", "loss_tok", "lse", "m_p"):
        assert np.array_equal(g[key].view(np.uint32), c[key].view(np.uint32)), key


@pytest.mark.parametrize("mode", DENSE)
def test_odd_slice_counts_two_blocks(mode):
    """d = 192 (forward k-loop of 3 slices of 64) and V = 2454 (the dh k-loop
    over the whole vocabulary rounded to 64: 39 slices), two token blocks
    (256 and 144 tokens)."""
    T, d, V, K = 400, 192, 2454, 13
    h, W = synth.student_head(T, d, V, seed=8)
    idx, tlp, mq = teacher_cache(T, V, K, seed=8)
    g = _run(h, W, idx, tlp, mq, mode, token_block=256)
    r = oracle.loss_fwd_bwd(synth.as_f64(h), synth.as_f64(W), idx, tlp, mq, mode)
    _compare(g, r, f"odd-slice token-block mode={oracle.MODE_NAMES[mode]}")


def test_peaked_student_tail():
    """The peaked-student case (m_p ~ 1e-11, m_q = 0.3) through the token-block
    path: the off-S factor A e^(m - B) with B = lse_off stays bounded."""
    T, d, V, K = 64, 64, 1024, 8
    rng = np.random.default_rng(23)
    S = np.array([5, 300, 517, 700, 701, 900, 1020, 1023], np.int32)
    W = rng.standard_normal((V, d)).astype(np.float32) / 8.0
    W[:, 0] = 0.0
    W[S, 0] = 1.875
    h = rng.standard_normal((T, d)).astype(np.float32)
    h[:, 0] = 16.0
    hb, Wb = synth.to_bf16(h), synth.to_bf16(W)
    idx = np.tile(S, (T, 1))
    mq = np.full(T, 0.3, np.float32)
    head = rng.standard_normal((T, K))
    head = np.exp(head) / np.exp(head).sum(1, keepdims=True)
    tlp = np.log(0.7 * head).astype(np.float32)
    for mode in (kd.TAIL, kd.FULL, kd.TAIL_REVERSE):
        g = _run(hb, Wb, idx, tlp, mq, mode, token_block=256)
        r = oracle.loss_fwd_bwd(synth.as_f64(hb), synth.as_f64(Wb), idx, tlp, mq, mode)
        _compare(g, r, f"peaked student token-block mode={oracle.MODE_NAMES[mode]}")


def test_k_equals_v_and_bitwise_deterministic():
    """S covering the vocabulary (no entry off S: the dense factor is 0) and
    two identical calls giving identical bits."""
    T, d, V = 40, 64, 256
    h, W = synth.student_head(T, d, V, seed=7)
    zt = synth.zipf_teacher_logits(T, V, seed=7).astype(np.float64)
    lq = np.stack([zt[t] - oracle.logsumexp(zt[t]) for t in range(T)])
    perm = np.stack([np.random.default_rng(t).permutation(V) for t in range(T)]).astype(np.int32)
    tlp = np.take_along_axis(lq, perm, axis=1).astype(np.float32)
    mq = np.zeros(T, np.float32)
    for mode in (kd.TAIL, kd.FULL):
        g = _run(h, W, perm, tlp, mq, mode, token_block=256)
        r = oracle.loss_fwd_bwd(synth.as_f64(h), synth.as_f64(W), perm, tlp, mq, mode)
        _compare(g, r, f"K=V token-block mode={oracle.MODE_NAMES[mode]}")
        g2 = _run(h, W, perm, tlp, mq, mode, token_block=256)
        for key in g:
            assert np.array_equal(np.asarray(g[key]).view(np.uint32), np.asarray(g2[key]).view(np.uint32)), key


def test_argument_errors():
    L = kd.lib()
    assert L.kd_topk_loss_tokblock_workspace(4096, 2048, 151936, 15, kd.TAIL, 0) == 0
    # 16,384 x 151,936 bf16 logits reach 4 GiB: refused
    assert L.kd_topk_loss_tokblock_workspace(32768, 2560, 151936, 64, kd.TAIL, 16384) == 0
    assert L.kd_topk_loss_tokblock_workspace(32768, 2560, 151936, 64, kd.TAIL, 8192) > 8192 * 151936 * 2
    h = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((8, 4), dtype=torch.int32, device=DEV)
    tlp = torch.zeros((8, 4), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        kd.loss_fwd_bwd(h, W, idx, tlp, None, mode=kd.FULL, token_block=256,
                        labels=torch.zeros(8, dtype=torch.int32, device=DEV), ce_weight=0.5)
