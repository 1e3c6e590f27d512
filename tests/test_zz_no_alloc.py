"""stq_gemv_noalloc, the GEMV entry point for callers that cannot allocate
(graph capture, tight serving loops, harnesses that forbid allocation),
called through the C ABI against stq_gemv on the same inputs: both take the
same plan, so their outputs must agree bit for bit.  Two calls in a row, the
second on a smaller batch, check that the library's fixed scratch keeps no
state a later call depends on."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import stq_oracle as O
import synth_inputs as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stq():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import sparse_ternary_bit_amd as m
    return m


def _table(seed, n_experts, n, k):
    rb = O.row_bytes(k)
    stride = (n * rb + 15) // 16 * 16
    t = np.zeros(n_experts * stride, dtype=np.uint8)
    for e in range(n_experts):
        t[e * stride: e * stride + n * rb] = O.quantize_rows(S.gaussian_weights(seed + e, n, k), None)
    return torch.from_numpy(t).cuda(), stride


def _noalloc(stq, table, stride, E, n, k, x, pe, pt, y):
    L = stq.lib()
    f = L.stq_gemv_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    st = f(table.data_ptr(), stride, E, n, k, x.data_ptr(), 1, x.shape[1], x.shape[0], pe.data_ptr(),
           pt.data_ptr(), pe.numel(), y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.stq_last_error().decode()


@pytest.mark.parametrize("plan", [None, "4,2"])
def test_noalloc_matches_gemv_twice_second_smaller(stq, monkeypatch, plan):
    """Through the C ABI (ctypes) and through the binding, against stq_gemv."""
    if plan:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    else:
        monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    n, k, E = 1024, 2048, 12
    table, stride = _table(300, E, n, k)
    for T, seed in ((24, 301), (3, 302)):                 # the second call is smaller
        pe_np, pt_np = S.uniform_topk_pairs(seed, T, E, 4)
        pe, pt = torch.from_numpy(pe_np).cuda(), torch.from_numpy(pt_np).cuda()
        x = S.torch_bf16_normal(seed, (T, k))
        assert stq.gemv_plan(E, n, k, pe.numel())[2] > 0  # the call uses the scratch
        y_ref = stq.gemv(table, stride, E, n, k, x, pe, pt)
        y = torch.full((pe.numel(), n), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc(stq, table, stride, E, n, k, x, pe, pt, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), (T, plan)
        y2 = torch.full_like(y, float("nan"))
        stq.gemv_noalloc(table, stride, E, n, k, x, pe, pt, y2)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref), (T, plan)
        # and both meet the oracle's tolerance on a few pairs
        xf = x.float().cpu().numpy()
        yc = y.cpu().numpy()
        for i in (0, pe.numel() - 1):
            raw = table[int(pe_np[i]) * stride: int(pe_np[i]) * stride + n * O.row_bytes(k)].cpu().numpy()
            ref = O.gemv(raw, n, k, xf[pt_np[i]])
            A = O.tolerance_scale(raw, n, k, xf[pt_np[i]])[0]
            assert np.all(np.abs(yc[i] - ref) <= 1e-3 * A)
