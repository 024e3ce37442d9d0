"""GPU parity of kd_kl_hidden_fwd_bwd (exact full-vocabulary KL with the
teacher rebuilt from a cached hidden state) against the fp64 CPU oracle.

Bar as for the top-K loss: loss relative error <= 1e-3; dh and dW relative
Frobenius error <= 1e-2; lse and lse_t within 2e-4 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_kd_loss_amd as kd
from _inputs import rel_err, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(T, d, dt, V, seed, bias=True):
    h, W = synth.student_head(T, d, V, seed=seed)
    g, U, b = synth.teacher_head(T, dt, V, seed=seed + 100)
    return h, W, g, U, (b if bias else None)


def _gpu(h, W, g, U, b, chunk):
    o = kd.kl_hidden_fwd_bwd(h.to(DEV), W.to(DEV), g.to(DEV), U.to(DEV), None if b is None else b.to(DEV),
                             chunk=chunk)
    torch.cuda.synchronize()
    return {k: getattr(o, k).cpu().numpy() for k in o._fields}


def _check(gout, r, tag):
    assert rel_err(gout["loss"], r["loss"]) <= 1e-3, (tag, float(gout["loss"]), r["loss"])
    np.testing.assert_allclose(gout["lse"], r["lse"], atol=2e-4, rtol=0, err_msg=tag)
    np.testing.assert_allclose(gout["lse_t"], r["lse_t"], atol=2e-4, rtol=0, err_msg=tag)
    lt = np.abs(gout["loss_tok"] - r["loss_tok"]) / np.maximum(np.abs(r["loss_tok"]), 1e-3)
    assert lt.max() <= 5e-3, (tag, float(lt.max()))
    e_dh, e_dw = rel_fro(gout["dh"], r["dh"]), rel_fro(gout["dW"], r["dW"])
    assert e_dh <= 1e-2 and e_dw <= 1e-2, (tag, e_dh, e_dw)
    return e_dh, e_dw


# "odd": k-loops over 3 (d = 192) and 5 (d_t = 320) slices of 64, and a last
# 150-row chunk whose dh loop has 3
SHAPES = {"tiny": (64, 64, 128, 1024, 8192, 0), "ragged": (300, 128, 64, 2500, 700, 3),
          "odd": (200, 192, 320, 2454, 700, 5)}


@pytest.mark.parametrize("shape", ["tiny", "ragged", "odd"])
def test_kl_hidden_matches_oracle(shape):
    T, d, dt, V, chunk, seed = SHAPES[shape]
    h, W, g, U, b = _inputs(T, d, dt, V, seed)
    gout = _gpu(h, W, g, U, b, chunk)
    r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), synth.as_f64(g), synth.as_f64(U),
                                 b.double().numpy())
    e = _check(gout, r, shape)
    print(f"kl_hidden {shape}: loss={float(gout['loss']):.6f} ref={r['loss']:.6f} dh={e[0]:.2e} dW={e[1]:.2e}")


def test_kl_hidden_no_bias_and_self_distillation():
    T, d, V = 96, 64, 1500
    h, W, g, U, _ = _inputs(T, d, 64, V, 5, bias=False)
    gout = _gpu(h, W, g, U, None, 512)
    r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), synth.as_f64(g), synth.as_f64(U), None)
    _check(gout, r, "no bias")
    # teacher = student: the KL is zero and p - q vanishes exactly
    s = _gpu(h, W, h, W, None, 512)
    assert abs(float(s["loss"])) < 1e-5
    assert np.abs(s["dh"]).max() == 0.0 and np.abs(s["dW"]).max() == 0.0


def test_kl_hidden_empty_tokens_and_errors():
    d, dt, V = 64, 64, 300
    W = torch.zeros((V, d), dtype=torch.bfloat16, device=DEV)
    U = torch.zeros((V, dt), dtype=torch.bfloat16, device=DEV)
    h = torch.zeros((0, d), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((0, dt), dtype=torch.bfloat16, device=DEV)
    o = kd.kl_hidden_fwd_bwd(h, W, g, U)
    torch.cuda.synchronize()
    assert float(o.loss) == 0.0 and float(o.dW.abs().max()) == 0.0
    with pytest.raises(kd.KDError):
        kd.kl_hidden_fwd_bwd(torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV),
                             torch.zeros((V, 48), dtype=torch.bfloat16, device=DEV),
                             torch.zeros((4, dt), dtype=torch.bfloat16, device=DEV), U)


def test_kl_hidden_full_width_qwen3_8b_teacher_1p7b_student():
    """Full vocabulary and head widths (V = 151,936, student d = 2048,
    teacher d = 4096), 128 tokens: 19 vocabulary chunks of 8192 rows."""
    T, d, dt, V = 128, 2048, 4096, 151936
    h, W, g, U, b = _inputs(T, d, dt, V, 7)
    gout = _gpu(h, W, g, U, b, 8192)
    r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), synth.as_f64(g), synth.as_f64(U),
                                 b.double().numpy(), block=32)
    e = _check(gout, r, "full width")
    print(f"kl_hidden full width: loss={float(gout['loss']):.6f} ref={r['loss']:.6f} dh={e[0]:.2e} dW={e[1]:.2e}")


def test_kl_hidden_bench_size_every_output():
    """The benchmarked workload itself: T = 4096 tokens, student d = 2048,
    teacher d = 4096, V = 151,936, chunk 8192 (16 token tiles x 19 chunks),
    every output against the fp64 oracle (about 13 TFLOP on the host)."""
    T, d, dt, V = 4096, 2048, 4096, 151936
    h, W = synth.student_head(T, d, V, seed=0)
    g, U, b = synth.teacher_head(T, dt, V, seed=1)
    gout = _gpu(h, W, g, U, b, 8192)
    r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), synth.as_f64(g), synth.as_f64(U),
                                 b.double().numpy())
    e = _check(gout, r, "bench size")
    print(f"kl_hidden bench size: loss={float(gout['loss']):.6f} ref={r['loss']:.6f} dh={e[0]:.2e} dW={e[1]:.2e}")


def test_int8_quantize_codes_bit_exact():
    """GPU codes and scales equal the oracle's on identical bf16 inputs
    (fp32 decisions on both sides), including a zero row and ties at .5."""
    T, dt = 37, 320
    g, _, _ = synth.teacher_head(T, dt, 64, seed=11)
    g = g.clone()
    g[3] = 0
    g[5, :8] = torch.tensor([127.0, 0.5, 1.5, -2.5, 63.5, -63.5, 3.0, -126.5], dtype=torch.bfloat16)
    codes, sc = kd.hidden_quantize_int8(g.to(DEV))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_hidden_int8(g.float().numpy())
    np.testing.assert_array_equal(codes.cpu().numpy(), rq)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("shape", ["tiny", "ragged", "odd"])
def test_kl_hidden_int8_cache(shape):
    T, d, dt, V, chunk, seed = SHAPES[shape]
    h, W, g, U, b = _inputs(T, d, dt, V, seed)
    # the cache comes from the oracle's quantizer (the GPU's is checked bit-exactly above)
    rq, rs = oracle.quantize_hidden_int8(g.float().numpy())
    o = kd.kl_hidden_fwd_bwd(h.to(DEV), W.to(DEV), torch.from_numpy(rq).to(DEV), U.to(DEV), b.to(DEV), chunk=chunk,
                             g_scale=torch.from_numpy(rs).to(DEV))
    torch.cuda.synchronize()
    gout = {k: getattr(o, k).cpu().numpy() for k in o._fields}
    r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), rq.astype(np.float64), synth.as_f64(U),
                                 b.double().numpy(), g_scale=rs)
    e = _check(gout, r, "int8 " + shape)
    print(f"kl_hidden int8 {shape}: loss={float(gout['loss']):.6f} ref={r['loss']:.6f} dh={e[0]:.2e} dW={e[1]:.2e}")


# --------------------------------------------------------------------------
# Cached teacher logsumexp (kd_kl_hidden_cached_lse_fwd_bwd)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", ["tiny", "ragged", "ragged_int8"])
def test_kl_hidden_cached_lse_matches_oracle(shape):
    """The teacher's logsumexp given as an input (the oracle's, in fp32):
    same bar as the recomputing call."""
    if shape == "tiny":
        T, d, dt, V, chunk, seed = 64, 64, 128, 1024, 8192, 0
    else:
        T, d, dt, V, chunk, seed = 300, 128, 64, 2500, 700, 3
    h, W, g, U, b = _inputs(T, d, dt, V, seed)
    if shape.endswith("int8"):
        rq, rs = oracle.quantize_hidden_int8(g.float().numpy())
        r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), rq.astype(np.float64), synth.as_f64(U),
                                     b.double().numpy(), g_scale=rs)
        gq, gs = torch.from_numpy(rq).to(DEV), torch.from_numpy(rs).to(DEV)
    else:
        r = oracle.kl_hidden_fwd_bwd(synth.as_f64(h), synth.as_f64(W), synth.as_f64(g), synth.as_f64(U),
                                     b.double().numpy())
        gq, gs = g.to(DEV), None
    lse_t = torch.from_numpy(r["lse_t"].astype(np.float32)).to(DEV)
    o = kd.kl_hidden_fwd_bwd(h.to(DEV), W.to(DEV), gq, U.to(DEV), b.to(DEV), chunk=chunk, g_scale=gs,
                             teacher_lse=lse_t)
    torch.cuda.synchronize()
    gout = {k: getattr(o, k).cpu().numpy() for k in o._fields}
    e = _check(gout, r, "cached lse " + shape)
    print(f"kl_hidden cached lse {shape}: loss={float(gout['loss']):.6f} ref={r['loss']:.6f} "
          f"dh={e[0]:.2e} dW={e[1]:.2e}")


def test_kl_hidden_cached_lse_reuses_the_recomputed_normalizer():
    """Feeding back the lse_t of a recomputing call: q is formed from the same
    fp32 normalizer, so dh and dW are bitwise those of that call; the loss
    (entropy from per-tile sums instead of the online partials) agrees to
    fp32 rounding."""
    T, d, dt, V, chunk = 300, 128, 64, 2500, 700
    h, W, g, U, b = _inputs(T, d, dt, V, 9)
    args = (h.to(DEV), W.to(DEV), g.to(DEV), U.to(DEV), b.to(DEV))
    full = kd.kl_hidden_fwd_bwd(*args, chunk=chunk)
    cached = kd.kl_hidden_fwd_bwd(*args, chunk=chunk, teacher_lse=full.lse_t.clone())
    torch.cuda.synchronize()
    assert torch.equal(full.dh, cached.dh) and torch.equal(full.dW, cached.dW)
    assert torch.equal(full.lse, cached.lse) and torch.equal(full.lse_t, cached.lse_t)
    assert rel_err(float(cached.loss), float(full.loss)) <= 1e-5
    np.testing.assert_allclose(cached.loss_tok.cpu().numpy(), full.loss_tok.cpu().numpy(), atol=2e-5, rtol=0)


def test_kl_hidden_cached_lse_argument_errors():
    import ctypes
    T, d, dt, V = 8, 64, 64, 300
    z = lambda *s, dt_=torch.bfloat16: torch.zeros(s, dtype=dt_, device=DEV)
    h, W, g, U = z(T, d), z(V, d), z(T, dt), z(V, dt)
    codes, gs = z(T, dt, dt_=torch.int8), z(T, dt_=torch.float32)
    f32 = lambda *s: z(*s, dt_=torch.float32)
    loss, dh, dW, lse_t = f32(), f32(T, d), f32(V, d), f32(T)
    L = kd.lib()
    ws = torch.empty(int(L.kd_kl_hidden_int8_workspace(T, d, dt, V, 512)), dtype=torch.uint8, device=DEV)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(g_, codes_, gs_, lse_):
        return L.kd_kl_hidden_cached_lse_fwd_bwd(p(h), p(W), p(g_), p(codes_), p(gs_), p(U), None, p(lse_), T, d, dt,
                                                 V, 512, 1.0 / T, p(loss), None, None, None, p(dh), p(dW), p(ws),
                                                 ws.numel(), s)

    assert call(g, None, None, None) == 1 and b"teacher_lse" in L.kd_last_error()
    assert call(g, codes, gs, lse_t) == 1 and b"not both" in L.kd_last_error()
    assert call(None, codes, None, lse_t) == 1
    assert call(g, None, None, lse_t) == 0
    torch.cuda.synchronize()
