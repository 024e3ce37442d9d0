"""CPU-only checks of the C-ABI library: it loads, exports every function
include/kdtopk.h declares, sizes workspaces, and rejects bad arguments on
the host before any GPU work."""
import ctypes
import os
import re

import pytest

import top_kd_loss_amd as kd

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kdtopk.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_two_calls():
    names = _declared()
    for n in ("kd_topk_loss_fwd_bwd", "kd_topk_cache_build", "kd_topk_loss_workspace",
              "kd_topk_cache_build_workspace", "kd_topk_rows", "kd_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = kd.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert set(_declared()) == set(kd.EXPORTS)
    assert "gfx950" in kd.version()


def test_workspace_is_linear_in_tokens():
    L = kd.lib()
    for mode in (kd.RENORM, kd.TAIL):
        w = [L.kd_topk_loss_workspace(T, 2560, 151936, 64, mode, 8192) for T in (4096, 8192, 16384, 32768)]
        assert all(x > 0 for x in w)
        d1, d2, d3 = w[1] - w[0], w[2] - w[1], w[3] - w[2]
        # exactly linear up to 256-byte alignment of the sub-buffers
        assert abs(2 * d1 - d2) < 64 * 256 and abs(2 * d2 - d3) < 64 * 256
    # the dense-mode scratch is bounded by the chunk, not by V
    a = L.kd_topk_loss_workspace(4096, 2048, 151936, 15, kd.TAIL, 8192)
    b = L.kd_topk_loss_workspace(4096, 2048, 151936, 15, kd.TAIL, 16384)
    assert b > a


@pytest.mark.parametrize("args", [
    (0, 64, 100, 0, 0, 8192),      # K = 0
    (8, 64, 100, 101, 0, 8192),    # K > V
    (8, 60, 100, 4, 0, 8192),      # d % 64
    (8, 64, 100, 4, 7, 8192),      # mode
    (8, 64, 100, 4, 0, 0),         # chunk
    (8, 64, 5000, 1025, 0, 8192),  # K > 1024
])
def test_invalid_sizes_rejected(args):
    L = kd.lib()
    assert L.kd_topk_loss_workspace(*args) == 0
    T, d, V, K, mode, chunk = args
    st = L.kd_topk_loss_fwd_bwd(None, None, None, None, None, T, d, V, K, mode, chunk, 1.0,
                                None, None, None, None, None, None, None, 0, None)
    assert st == 1  # KD_EINVAL
    assert L.kd_last_error()


def test_workspace_too_small_is_reported_before_launch():
    L = kd.lib()
    buf = ctypes.create_string_buffer(16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    st = L.kd_topk_loss_fwd_bwd(p, p, p, p, p, 8, 64, 100, 4, kd.TAIL, 8192, 1.0,
                                p, None, None, None, p, p, p, 16, None)
    assert st == 3  # KD_ENOWS
    assert b"workspace too small" in L.kd_last_error()


def test_cache_argument_errors():
    L = kd.lib()
    assert L.kd_topk_cache_build_workspace(16, 64, 1000, 8, 2) > 0
    assert L.kd_topk_cache_build_workspace(16, 64, 1000, 8, 9) == 0
    rho = (ctypes.c_float * 1)(1.5)
    st = L.kd_topk_rows(None, 4, 100, 4, rho, 1, None, None, None, None, None, None, None, 0, None)
    assert st == 1 and b"rho" in L.kd_last_error()


def _host_ptrs(n, size=4096):
    """Host buffers standing in for device arrays in calls that must be
    rejected on the host before any launch."""
    bufs = [ctypes.create_string_buffer(size + 16) for _ in range(n)]
    return bufs, [ctypes.c_void_p((ctypes.addressof(b) + 15) & ~15) for b in bufs]


def test_selected_entry_argument_errors():
    L = kd.lib()
    _, (h, W, idx, tlp, sl, sz, y, loss, dh, dW, ws) = _host_ptrs(11)
    # the student's logsumexp and logits at idx come together
    st = L.kd_topk_loss_fwd_bwd_selected(h, W, idx, tlp, None, sl, None, None, None, 8, 64, 100, 4, kd.REVERSE,
                                         8192, 1.0, loss, None, None, None, dh, dW, ws, 1 << 40, None)
    assert st == 1 and b"student_lse" in L.kd_last_error()
    # sampled tokens only with the tail-corrected reverse mode
    st = L.kd_topk_loss_fwd_bwd_selected(h, W, idx, tlp, None, sl, sz, y, None, 8, 64, 100, 4, kd.REVERSE,
                                         8192, 1.0, loss, None, None, None, dh, dW, ws, 1 << 40, None)
    assert st == 1 and b"KD_REVERSE_TT" in L.kd_last_error()


def test_cached_lse_entry_argument_errors():
    L = kd.lib()
    _, (h, W, g, codes, gs, U, loss, dh, dW, ws) = _host_ptrs(10)
    st = L.kd_kl_hidden_cached_lse_fwd_bwd(h, W, g, None, None, U, None, None, 8, 64, 64, 300, 512, 1.0, loss, None,
                                           None, None, dh, dW, ws, 1 << 40, None)
    assert st == 1 and b"teacher_lse" in L.kd_last_error()
    _, (tl,) = _host_ptrs(1)
    st = L.kd_kl_hidden_cached_lse_fwd_bwd(h, W, g, codes, gs, U, None, tl, 8, 64, 64, 300, 512, 1.0, loss, None,
                                           None, None, dh, dW, ws, 1 << 40, None)
    assert st == 1 and b"not both" in L.kd_last_error()


def test_misaligned_matrix_rejected_before_launch():
    L = kd.lib()
    _, (h, W, idx, tlp, loss, dh, dW, ws) = _host_ptrs(8)
    W_off = ctypes.c_void_p(W.value + 8)
    st = L.kd_topk_loss_fwd_bwd(h, W_off, idx, tlp, None, 8, 64, 100, 4, kd.RENORM, 8192, 1.0,
                                loss, None, None, None, dh, dW, ws, 1 << 40, None)
    assert st == 1 and b"16-byte aligned" in L.kd_last_error()


def test_row_pass_workspace_holds_flags_and_deferred_crossing_bins():
    """kd_topk_rows_workspace: 4 bytes per row rounded to 256, and with k_rho
    targets a 240-byte record per row (rounded to 256) plus 512 eight-byte
    candidate slots per row and target; rows of V >= 2^18 (the exact
    kernel only) need the flags alone."""
    L = kd.lib()
    r256 = lambda x: (x + 255) // 256 * 256
    for T, n_rho in ((2048, 0), (2048, 2), (777, 1), (1, 8)):
        want = r256(T * 4) + (r256(T * 240) + T * n_rho * 512 * 8 if n_rho else 0)
        assert L.kd_topk_rows_workspace(T, 151936, 256, n_rho) == want, (T, n_rho)
    assert L.kd_topk_rows_workspace(100, 1 << 18, 16, 2) == r256(100 * 4)


def test_row_pass_refuses_small_or_misaligned_workspace_before_launch():
    L = kd.lib()
    bufs, (z, idx, val, lse, mq, krho, logp, ws) = _host_ptrs(8)
    rho = (ctypes.c_float * 2)(0.9, 0.95)
    need = L.kd_topk_rows_workspace(4, 1000, 8, 2)
    st = L.kd_topk_rows(z, 4, 1000, 8, rho, 2, idx, val, lse, mq, krho, logp, ws, need - 1, None)
    assert st == 3 and b"workspace too small" in L.kd_last_error()
    ws_off = ctypes.c_void_p(ws.value + 8)
    st = L.kd_topk_rows(z, 4, 1000, 8, rho, 2, idx, val, lse, mq, krho, logp, ws_off, need, None)
    assert st == 1 and b"16-byte aligned" in L.kd_last_error()


def test_missing_library_fails_loudly(monkeypatch):
    """No CPU fallback: without the built library every call raises."""
    monkeypatch.setattr(kd, "_lib", None)
    monkeypatch.setattr(kd, "LIB_PATH", "/nonexistent/libkdtopk.so")
    with pytest.raises(kd.KDError, match="not built"):
        kd.lib()


def test_cpu_tensors_are_refused():
    import torch
    h = torch.zeros((4, 64), dtype=torch.bfloat16)
    W = torch.zeros((100, 64), dtype=torch.bfloat16)
    idx = torch.zeros((4, 2), dtype=torch.int32)
    tlp = torch.zeros((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="no CPU path"):
        kd.loss_fwd_bwd(h, W, idx, tlp, None, mode=kd.RENORM)
    with pytest.raises(ValueError, match="no CPU path"):
        kd.cache_build(h, W, None, 2)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
