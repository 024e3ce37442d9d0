"""kd_topk_rows_noalloc (the row pass with the library's static device
scratch, for callers that cannot allocate) against kd_topk_rows, through
the C ABI: every output bitwise equal, on two calls in a row, the second
with fewer rows; rows that take the exact kernel through the fallback flags
(non-finite maxima, a tie larger than the candidate pool) included."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import top_kd_loss_amd as kd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rows(T, V, seed):
    z = synth.zipf_teacher_logits(T, V, seed=seed)
    z[1, :] = -np.inf                  # no finite value: flagged, exact kernel
    z[1, 7] = 2.0
    z[2, :] = 0.5                      # one tie over the whole row
    z[3, ::3] = -np.inf
    return torch.from_numpy(z).to(DEV)


def _same(a, b):
    for name, x, y in zip(a._fields, a, b):
        xx = x.view(torch.int32) if x.dtype == torch.float32 else x
        yy = y.view(torch.int32) if y.dtype == torch.float32 else y
        assert torch.equal(xx, yy), name


@pytest.mark.parametrize("rho", [(), (0.9, 0.95)])
def test_noalloc_matches_workspace_call_twice(rho):
    for T, V, K, seed in ((300, 5000, 64, 1), (77, 3001, 256, 2)):
        z = _rows(T, V, seed)
        ref = kd.topk_rows(z, K, rho)
        got = kd.topk_rows_noalloc(z, K, rho)
        torch.cuda.synchronize()
        _same(got, ref)


def test_noalloc_refuses_too_many_rows():
    L = kd.lib()
    rho = (ctypes.c_float * 1)(0.9)
    st = L.kd_topk_rows_noalloc(None, (1 << 20) + 1, 100, 4, rho, 0, None, None, None, None, None, None, None)
    assert st == 2 and b"at most" in L.kd_last_error()
