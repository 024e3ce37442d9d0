"""Python binding of libkdtopk.so: the fused top-K KD loss and the teacher
cache build on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
library behind the C ABI declared in include/kdtopk.h.  PyTorch provides
device memory and the current stream.  There is no CPU fallback: the calls
raise if the library is not built or the tensors are not on a GPU.

    out = loss_fwd_bwd(h, W, idx, teacher_logp, m_q, mode=TAIL, chunk=8192)
    out.loss, out.dh, out.dW, out.loss_tok, out.lse, out.m_p
    idx, val, lse, m_q, k_rho = cache_build(g, U, b, K, rho=(0.9, 0.95))
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence

import torch

RENORM, TAIL, FULL, REVERSE, TAIL_REVERSE, REVERSE_TT = 0, 1, 2, 3, 4, 5
MODE_BY_NAME = {"renorm": RENORM, "tail": TAIL, "full": FULL, "reverse": REVERSE, "tail_reverse": TAIL_REVERSE,
                "reverse_tt": REVERSE_TT}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdtopk.so")
_lib = None

_i64, _i32, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "kd_topk_loss_workspace": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32]),
    "kd_topk_loss_fwd_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _f32,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_topk_loss_ce_workspace": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32, _f32]),
    "kd_topk_loss_tokblock_workspace": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32]),
    "kd_topk_loss_fwd_bwd_tokblock": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                                     _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_topk_loss_fwd_bwd_ce": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _i64, _i64, _i64, _i32, _i32,
                                               _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_kl_hidden_workspace": (_sz, [_i64, _i64, _i64, _i64, _i32]),
    "kd_kl_hidden_fwd_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _f32,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_topk_loss_fwd_bwd_tt": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _f32,
                                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_topk_loss_fwd_bwd_selected": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                                     _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                                     _vp]),
    "kd_hidden_quantize_int8": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "kd_kl_hidden_int8_workspace": (_sz, [_i64, _i64, _i64, _i64, _i32]),
    "kd_kl_hidden_int8_fwd_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _f32,
                                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_kl_hidden_cached_lse_fwd_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                       _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_teacher_recover": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "kd_teacher_recover_workspace": (_sz, [_i64, _i64, _i32]),
    "kd_teacher_recover_ws": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp]),
    "kd_topk_cache_build_workspace": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "kd_topk_cache_build": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _i32,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_topk_rows_workspace": (_sz, [_i64, _i64, _i32, _i32]),
    "kd_topk_rows": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                    _vp]),
    "kd_topk_rows_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kd_last_error": (ctypes.c_char_p, []),
    "kd_version": (ctypes.c_char_p, []),
    "kd_profile_begin": (ctypes.c_int, []),
    "kd_profile_end": (_i32, [_i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_f32), ctypes.POINTER(_i32)]),
}
EXPORTS = tuple(_SIGS)


class KDError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libkdtopk.so (torch's HIP runtime is already in the process)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KDError(f"{LIB_PATH} is not built; run `python -m top_kd_loss_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().kd_last_error().decode(errors="replace")
        raise KDError(f"{what} failed with status {status}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device: torch.device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class LossOut(NamedTuple):
    loss: torch.Tensor      # [] fp32
    dh: torch.Tensor        # [T, d] fp32
    dW: torch.Tensor        # [V, d] fp32
    loss_tok: torch.Tensor  # [T] fp32
    lse: torch.Tensor       # [T] fp32
    m_p: torch.Tensor       # [T] fp32


def loss_workspace_bytes(T: int, d: int, V: int, K: int, mode: int, chunk: int, ce_weight: float = 0.0,
                         token_block: int = 0) -> int:
    if token_block:
        return int(lib().kd_topk_loss_tokblock_workspace(T, d, V, K, mode, token_block))
    if ce_weight:
        return int(lib().kd_topk_loss_ce_workspace(T, d, V, K, mode, chunk, ce_weight))
    return int(lib().kd_topk_loss_workspace(T, d, V, K, mode, chunk))


def loss_fwd_bwd(h: torch.Tensor, W: torch.Tensor, idx: torch.Tensor, teacher_logp: torch.Tensor,
                 m_q: Optional[torch.Tensor] = None, mode: int = TAIL, chunk: int = 8192,
                 scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                 out: Optional[LossOut] = None, labels: Optional[torch.Tensor] = None,
                 ce_weight: float = 0.0, labels_teacher_logp: Optional[torch.Tensor] = None,
                 student_lse: Optional[torch.Tensor] = None,
                 student_logits: Optional[torch.Tensor] = None, token_block: int = 0) -> LossOut:
    """Fused LM head + top-K KD loss, forward and backward (kd_topk_loss_fwd_bwd;
    with labels [T] int32 (-1 = none) and ce_weight > 0, kd_topk_loss_fwd_bwd_ce
    adds the weighted hard-label cross-entropy term; with mode REVERSE_TT,
    labels are the sampled tokens and labels_teacher_logp [T] the teacher's
    log-probabilities at them, kd_topk_loss_fwd_bwd_tt).  student_lse [T] and
    student_logits [T, K] (e.g. lse and val of cache_build(h, W, None, K), the
    selection of idx) skip the forward pass (kd_topk_loss_fwd_bwd_selected).
    token_block > 0 takes the token-block path (kd_topk_loss_fwd_bwd_tokblock):
    the dense modes keep each block's [token_block, V] logits (bf16) instead
    of recomputing them in the backward; chunk is then unused."""
    if isinstance(mode, str):
        mode = MODE_BY_NAME[mode]
    dev = h.device
    T, d = h.shape
    V = W.shape[0]
    K = idx.shape[1]
    _need(h, "h", torch.bfloat16, (T, d), dev)
    _need(W, "W", torch.bfloat16, (V, d), dev)
    _need(idx, "idx", torch.int32, (T, K), dev)
    _need(teacher_logp, "teacher_logp", torch.float32, (T, K), dev)
    if m_q is not None:
        _need(m_q, "m_q", torch.float32, (T,), dev)
    if labels is not None:
        _need(labels, "labels", torch.int32, (T,), dev)
    if labels_teacher_logp is not None:
        _need(labels_teacher_logp, "labels_teacher_logp", torch.float32, (T,), dev)
    sel = student_lse is not None or student_logits is not None
    if sel:
        if student_lse is None or student_logits is None:
            raise ValueError("student_lse and student_logits come together")
        if ce_weight != 0.0:
            raise ValueError("the cross-entropy term is not available with given student logits")
        _need(student_lse, "student_lse", torch.float32, (T,), dev)
        _need(student_logits, "student_logits", torch.float32, (T, K), dev)
    ce = ce_weight != 0.0
    tt = mode == REVERSE_TT and labels is not None
    if token_block and (sel or ce or labels is not None):
        raise ValueError("the token-block path takes no labels, sampled tokens or given student logits")
    if scale is None:
        scale = 1.0 / max(T, 1)
    L = lib()
    ws_bytes = loss_workspace_bytes(T, d, V, K, mode, chunk, ce_weight, token_block)
    if ws_bytes == 0 and token_block:
        _check(L.kd_topk_loss_fwd_bwd_tokblock(None, None, None, None, None, T, d, V, K, mode, token_block, scale,
                                               None, None, None, None, None, None, None, 0, None),
               "kd_topk_loss_fwd_bwd_tokblock")
    if ws_bytes == 0:
        _check(L.kd_topk_loss_fwd_bwd_ce(None, None, None, None, None, None, ce_weight, T, d, V, K, mode, chunk,
                                         scale, None, None, None, None, None, None, None, 0, None),
               "kd_topk_loss_fwd_bwd_ce")
    with torch.cuda.device(dev):
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if out is None:
            f32 = dict(dtype=torch.float32, device=dev)
            out = LossOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                          torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
        if token_block:
            st = L.kd_topk_loss_fwd_bwd_tokblock(_ptr(h), _ptr(W), _ptr(idx), _ptr(teacher_logp), _ptr(m_q),
                                                 T, d, V, K, mode, token_block, scale,
                                                 _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse), _ptr(out.m_p),
                                                 _ptr(out.dh), _ptr(out.dW), _ptr(workspace), workspace.numel(),
                                                 _stream(dev))
        elif sel:
            st = L.kd_topk_loss_fwd_bwd_selected(_ptr(h), _ptr(W), _ptr(idx), _ptr(teacher_logp), _ptr(m_q),
                                                 _ptr(student_lse), _ptr(student_logits),
                                                 _ptr(labels) if tt else None,
                                                 _ptr(labels_teacher_logp) if tt else None, T, d, V, K, mode, chunk,
                                                 scale, _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse),
                                                 _ptr(out.m_p), _ptr(out.dh), _ptr(out.dW), _ptr(workspace),
                                                 workspace.numel(), _stream(dev))
        elif tt:
            st = L.kd_topk_loss_fwd_bwd_tt(_ptr(h), _ptr(W), _ptr(idx), _ptr(teacher_logp), _ptr(labels),
                                           _ptr(labels_teacher_logp), T, d, V, K, chunk, scale,
                                           _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse), _ptr(out.m_p),
                                           _ptr(out.dh), _ptr(out.dW), _ptr(workspace), workspace.numel(),
                                           _stream(dev))
        elif ce:
            st = L.kd_topk_loss_fwd_bwd_ce(_ptr(h), _ptr(W), _ptr(idx), _ptr(teacher_logp), _ptr(m_q),
                                           _ptr(labels), ce_weight, T, d, V, K, mode, chunk, scale,
                                           _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse), _ptr(out.m_p),
                                           _ptr(out.dh), _ptr(out.dW), _ptr(workspace), workspace.numel(),
                                           _stream(dev))
        else:
            st = L.kd_topk_loss_fwd_bwd(_ptr(h), _ptr(W), _ptr(idx), _ptr(teacher_logp), _ptr(m_q),
                                        T, d, V, K, mode, chunk, scale,
                                        _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse), _ptr(out.m_p),
                                        _ptr(out.dh), _ptr(out.dW), _ptr(workspace), workspace.numel(),
                                        _stream(dev))
    _check(st, "kd_topk_loss_fwd_bwd_tokblock" if token_block else "kd_topk_loss_fwd_bwd_selected" if sel
           else "kd_topk_loss_fwd_bwd_tt" if tt
           else "kd_topk_loss_fwd_bwd_ce" if ce else "kd_topk_loss_fwd_bwd")
    return out


class KlOut(NamedTuple):
    loss: torch.Tensor
    dh: torch.Tensor
    dW: torch.Tensor
    loss_tok: torch.Tensor
    lse: torch.Tensor
    lse_t: torch.Tensor


def hidden_quantize_int8(g: torch.Tensor):
    """int8 hidden-state cache of g [T, d] bf16: (codes int8 [T, d], scale fp32 [T])
    (kd_hidden_quantize_int8)."""
    T, d = g.shape
    _need(g, "g", torch.bfloat16, (T, d), g.device)
    codes = torch.empty((T, d), dtype=torch.int8, device=g.device)
    sc = torch.empty(T, dtype=torch.float32, device=g.device)
    with torch.cuda.device(g.device):
        _check(lib().kd_hidden_quantize_int8(_ptr(g), T, d, _ptr(codes), _ptr(sc), _stream(g.device)),
               "kd_hidden_quantize_int8")
    return codes, sc


def kl_hidden_fwd_bwd(h: torch.Tensor, W: torch.Tensor, g: torch.Tensor, U: torch.Tensor,
                      b: Optional[torch.Tensor] = None, chunk: int = 8192, scale: Optional[float] = None,
                      workspace: Optional[torch.Tensor] = None, out: Optional[KlOut] = None,
                      g_scale: Optional[torch.Tensor] = None,
                      teacher_lse: Optional[torch.Tensor] = None) -> KlOut:
    """Exact full-vocabulary KL(softmax(U g + b) || softmax(W h)), forward and
    backward, with the teacher rebuilt from its cached hidden state g
    (kd_kl_hidden_fwd_bwd); g int8 codes with g_scale [T] take the int8 cache
    (kd_kl_hidden_int8_fwd_bwd).  teacher_lse [T] (the lse_t output of an
    earlier call on the same cache) skips the teacher's logsumexp pass
    (kd_kl_hidden_cached_lse_fwd_bwd)."""
    dev = h.device
    T, d = h.shape
    V = W.shape[0]
    dt = g.shape[1]
    int8 = g.dtype == torch.int8
    _need(h, "h", torch.bfloat16, (T, d), dev)
    _need(W, "W", torch.bfloat16, (V, d), dev)
    _need(g, "g", torch.int8 if int8 else torch.bfloat16, (T, dt), dev)
    _need(U, "U", torch.bfloat16, (V, dt), dev)
    if int8:
        if g_scale is None:
            raise ValueError("int8 hidden states need g_scale")
        _need(g_scale, "g_scale", torch.float32, (T,), dev)
    if b is not None:
        _need(b, "b", torch.float32, (V,), dev)
    if teacher_lse is not None:
        _need(teacher_lse, "teacher_lse", torch.float32, (T,), dev)
    if scale is None:
        scale = 1.0 / max(T, 1)
    L = lib()
    ws_bytes = int((L.kd_kl_hidden_int8_workspace if int8 else L.kd_kl_hidden_workspace)(T, d, dt, V, chunk))
    if ws_bytes == 0:
        _check(L.kd_kl_hidden_fwd_bwd(None, None, None, None, None, T, d, dt, V, chunk, scale,
                                      None, None, None, None, None, None, None, 0, None), "kd_kl_hidden_fwd_bwd")
    with torch.cuda.device(dev):
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if out is None:
            f32 = dict(dtype=torch.float32, device=dev)
            out = KlOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                        torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
        if teacher_lse is not None:
            st = L.kd_kl_hidden_cached_lse_fwd_bwd(_ptr(h), _ptr(W), None if int8 else _ptr(g), _ptr(g) if int8 else None,
                                                   _ptr(g_scale) if int8 else None, _ptr(U), _ptr(b), _ptr(teacher_lse),
                                                   T, d, dt, V, chunk, scale, _ptr(out.loss), _ptr(out.loss_tok),
                                                   _ptr(out.lse), _ptr(out.lse_t), _ptr(out.dh), _ptr(out.dW),
                                                   _ptr(workspace), workspace.numel(), _stream(dev))
        elif int8:
            st = L.kd_kl_hidden_int8_fwd_bwd(_ptr(h), _ptr(W), _ptr(g), _ptr(g_scale), _ptr(U), _ptr(b), T, d, dt,
                                             V, chunk, scale, _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse),
                                             _ptr(out.lse_t), _ptr(out.dh), _ptr(out.dW), _ptr(workspace),
                                             workspace.numel(), _stream(dev))
        else:
            st = L.kd_kl_hidden_fwd_bwd(_ptr(h), _ptr(W), _ptr(g), _ptr(U), _ptr(b), T, d, dt, V, chunk, scale,
                                        _ptr(out.loss), _ptr(out.loss_tok), _ptr(out.lse), _ptr(out.lse_t),
                                        _ptr(out.dh), _ptr(out.dW), _ptr(workspace), workspace.numel(),
                                        _stream(dev))
    _check(st, "kd_kl_hidden_cached_lse_fwd_bwd" if teacher_lse is not None
           else "kd_kl_hidden_int8_fwd_bwd" if int8 else "kd_kl_hidden_fwd_bwd")
    return out


def teacher_recover(idx: torch.Tensor, teacher_logp: torch.Tensor, U: torch.Tensor,
                    b: Optional[torch.Tensor] = None, multi_workgroup: Optional[bool] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Teacher hidden state and logsumexp from k cached log-probs: returns
    (g_hat [T, d] fp32, c_hat [T] fp32).  The one-workgroup solver in LDS
    (kd_teacher_recover) serves small systems with k >= d + 1; wide heads,
    and k <= d (the minimum-norm solution), take the multi-workgroup one
    (kd_teacher_recover_ws).  multi_workgroup forces the choice."""
    dev = idx.device
    T, k = idx.shape
    V, d = U.shape
    _need(idx, "idx", torch.int32, (T, k), dev)
    _need(teacher_logp, "teacher_logp", torch.float32, (T, k), dev)
    _need(U, "U", torch.bfloat16, (V, d), dev)
    if b is not None:
        _need(b, "b", torch.float32, (V,), dev)
    g_hat = torch.empty((T, d), dtype=torch.float32, device=dev)
    c_hat = torch.empty(T, dtype=torch.float32, device=dev)
    kp = k + 1 if k % 2 == 0 else k
    if multi_workgroup is None:
        multi_workgroup = k < d + 1 or (d + 2) * kp > 19968
    with torch.cuda.device(dev):
        if multi_workgroup:
            L = lib()
            nb = int(L.kd_teacher_recover_workspace(T, d, k))
            if workspace is None or workspace.numel() < nb:
                workspace = torch.empty(max(nb, 8), dtype=torch.uint8, device=dev)
            _check(L.kd_teacher_recover_ws(_ptr(idx), _ptr(teacher_logp), _ptr(U), _ptr(b), T, d, V, k,
                                           _ptr(g_hat), _ptr(c_hat), _ptr(workspace), workspace.numel(),
                                           _stream(dev)), "kd_teacher_recover_ws")
        else:
            _check(lib().kd_teacher_recover(_ptr(idx), _ptr(teacher_logp), _ptr(U), _ptr(b), T, d, V, k,
                                            _ptr(g_hat), _ptr(c_hat), _stream(dev)), "kd_teacher_recover")
    return g_hat, c_hat


class CacheOut(NamedTuple):
    idx: torch.Tensor           # [T, K] int32
    val: torch.Tensor           # [T, K] fp32
    lse: torch.Tensor           # [T] fp32
    m_q: torch.Tensor           # [T] fp32
    k_rho: torch.Tensor         # [T, n_rho] int32
    teacher_logp: torch.Tensor  # [T, K] fp32: val - lse, the loss's teacher_logp input


def _rho_arr(rho: Sequence[float]):
    n = len(rho)
    arr = (ctypes.c_float * max(n, 1))(*[float(r) for r in rho])
    return arr, n


def _cache_out(T: int, K: int, n: int, dev) -> CacheOut:
    return CacheOut(torch.empty((T, K), dtype=torch.int32, device=dev),
                    torch.empty((T, K), dtype=torch.float32, device=dev),
                    torch.empty(T, dtype=torch.float32, device=dev),
                    torch.empty(T, dtype=torch.float32, device=dev),
                    torch.empty((T, n), dtype=torch.int32, device=dev),
                    torch.empty((T, K), dtype=torch.float32, device=dev))


def cache_build(g: torch.Tensor, U: torch.Tensor, b: Optional[torch.Tensor], K: int,
                rho: Sequence[float] = (), workspace: Optional[torch.Tensor] = None) -> CacheOut:
    """Teacher cache: top-K of z = U g + b per token, lse, m_q, k_rho and the
    teacher log-probabilities val - lse (kd_topk_cache_build)."""
    dev = g.device
    T, d = g.shape
    V = U.shape[0]
    _need(g, "g", torch.bfloat16, (T, d), dev)
    _need(U, "U", torch.bfloat16, (V, d), dev)
    if b is not None:
        _need(b, "b", torch.float32, (V,), dev)
    L = lib()
    arr, n = _rho_arr(rho)
    ws_bytes = int(L.kd_topk_cache_build_workspace(T, d, V, K, n))
    with torch.cuda.device(dev):
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        o = _cache_out(T, K, n, dev)
        st = L.kd_topk_cache_build(_ptr(g), _ptr(U), _ptr(b), T, d, V, K, arr, n,
                                   _ptr(o.idx), _ptr(o.val), _ptr(o.lse), _ptr(o.m_q),
                                   _ptr(o.k_rho) if n else None, _ptr(o.teacher_logp), _ptr(workspace),
                                   workspace.numel(), _stream(dev))
    _check(st, "kd_topk_cache_build")
    return o


def topk_rows(z: torch.Tensor, K: int, rho: Sequence[float] = (),
              workspace: Optional[torch.Tensor] = None) -> CacheOut:
    """Row pass on fp32 logits z [T, V]: top-K, lse, tail mass, k_rho and
    val - lse (kd_topk_rows)."""
    dev = z.device
    T, V = z.shape
    _need(z, "z", torch.float32, (T, V), dev)
    L = lib()
    arr, n = _rho_arr(rho)
    ws_bytes = int(L.kd_topk_rows_workspace(T, V, K, n))
    with torch.cuda.device(dev):
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        o = _cache_out(T, K, n, dev)
        st = L.kd_topk_rows(_ptr(z), T, V, K, arr, n, _ptr(o.idx), _ptr(o.val), _ptr(o.lse), _ptr(o.m_q),
                            _ptr(o.k_rho) if n else None, _ptr(o.teacher_logp), _ptr(workspace),
                            workspace.numel(), _stream(dev))
    _check(st, "kd_topk_rows")
    return o


def topk_rows_noalloc(z: torch.Tensor, K: int, rho: Sequence[float] = (), out: Optional[CacheOut] = None) -> CacheOut:
    """kd_topk_rows_noalloc: the row pass with the library's static device
    scratch instead of a workspace (at most 1,048,576 rows; calls on one
    device must not overlap).  `out` (a CacheOut of the right shapes) lets
    the caller allocate nothing either."""
    dev = z.device
    T, V = z.shape
    _need(z, "z", torch.float32, (T, V), dev)
    arr, n = _rho_arr(rho)
    with torch.cuda.device(dev):
        o = out if out is not None else _cache_out(T, K, n, dev)
        st = lib().kd_topk_rows_noalloc(_ptr(z), T, V, K, arr, n, _ptr(o.idx), _ptr(o.val), _ptr(o.lse), _ptr(o.m_q),
                                        _ptr(o.k_rho) if n else None, _ptr(o.teacher_logp), _stream(dev))
    _check(st, "kd_topk_rows_noalloc")
    return o


def profile_begin() -> None:
    """Start bracketing every library kernel launch with HIP events."""
    _check(lib().kd_profile_begin(), "kd_profile_begin")


def profile_end() -> dict:
    """Stop recording; {kernel name: (total ms, launches)} of the recorded launches."""
    n = 64
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    k = lib().kd_profile_end(n, names, ms, cnt)
    return {names[i].decode(): (float(ms[i]), int(cnt[i])) for i in range(min(k, n))}


def version() -> str:
    return lib().kd_version().decode()
