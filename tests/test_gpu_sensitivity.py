"""GPU parity of the layer-sensitivity entry points against the oracle,
through the C ABI.

stq_q2_roundtrip is compared bit for bit.  stq_layer_errors is compared
row by row within the oracle's fp64 bound (layer_errors_tolerance: two fp64
evaluations that differ only in summation order); exact cases (w_hat = w)
must give exactly zero.  The full-size case runs the benchmark's shape
(4096 x 7168 weights, 512 calibration rows) and checks sampled rows one by
one; the study case runs the whole allocation through the GPU and must pick
the same layers as the oracle.
"""
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
    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def check_errors(full, diag, w, w_hat, x, what=""):
    f_ref, d_ref = O.layer_errors(w, w_hat, x)
    b_full, b_diag = O.layer_errors_tolerance(w, w_hat, x)
    ef = np.abs(full - f_ref)
    ed = np.abs(diag - d_ref)
    assert np.all(ef <= b_full), f"{what}: full off by {np.max(ef / np.maximum(b_full, 1e-300))} bounds"
    assert np.all(ed <= b_diag), f"{what}: diag off by {np.max(ed / np.maximum(b_diag, 1e-300))} bounds"


# ---------------------------------------------------------------------------
# 2-bit stand-in
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_rows,k,seed", [(1, 256, 1), (7, 1024, 2), (65, 512, 3), (3, 7168, 4)])
def test_q2_roundtrip_bit_exact(stq, n_rows, k, seed):
    w = S.gaussian_weights(seed, n_rows, k)
    got = host(stq.q2_roundtrip(dev(w)))
    assert np.array_equal(got.view(np.uint32), O.q2_roundtrip(w).view(np.uint32))


def test_q2_roundtrip_special_blocks(stq):
    rng = np.random.default_rng(9)
    w = np.zeros((1, 256 * 6), dtype=np.float32)
    w[0, 256:512] = -0.0                                            # block of -0.0: ss = 0, s = 0, sign kept
    w[0, 512:768] = rng.normal(0, 1e5, 256)                         # rms/2 far above 65504: clamped scale
    w[0, 768:1024] = rng.normal(0, 1e-6, 256)                       # fp16 subnormal scale
    w[0, 1024:1280] = np.where(rng.random(256) < 0.5, 1.0, -3.0)    # weights on and between the levels
    w[0, 1280:1536] = rng.standard_t(2, 256) * 0.02                 # heavy tails
    got = host(stq.q2_roundtrip(dev(w)))
    assert np.array_equal(got.view(np.uint32), O.q2_roundtrip(w).view(np.uint32))


# ---------------------------------------------------------------------------
# full-Hessian and diagonal error
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_rows,k,n_cal,seed", [
    (1, 256, 1, 11), (63, 512, 65, 12), (64, 256, 64, 13), (65, 1280, 200, 14), (130, 768, 63, 15),
])
def test_layer_errors_match_oracle(stq, n_rows, k, n_cal, seed):
    w = S.gaussian_weights(seed, n_rows, k)
    rng = np.random.default_rng(seed + 100)
    x = (rng.normal(0, 1, (n_cal, k)) * rng.uniform(0.1, 10, k)).astype(np.float32)
    for w_hat in (O.dequantize_rows(O.quantize_rows(w, S.imatrix_from_calibration(x)), n_rows, k),
                  O.q2_roundtrip(w)):
        full, diag = stq.layer_errors(dev(w), dev(w_hat), dev(x))
        check_errors(host(full), host(diag), w, w_hat, x, f"{n_rows}x{k} N={n_cal}")


def test_layer_errors_paired_columns(stq):
    # strongly correlated columns: the full score differs from the diagonal one
    w, x = S.paired_channel_layer(21, 96, 1024, 130, sign=-1.0, coupling=0.9)
    w_hat = O.q2_roundtrip(w)
    full, diag = stq.layer_errors(dev(w), dev(w_hat), dev(x))
    full, diag = host(full), host(diag)
    check_errors(full, diag, w, w_hat, x, "paired")
    assert full.sum() < 0.5 * diag.sum()


def test_layer_errors_exact_zero_and_repeatable(stq):
    w = S.gaussian_weights(31, 70, 512)
    x = np.random.default_rng(32).normal(0, 1, (90, 512)).astype(np.float32)
    wd, xd = dev(w), dev(x)
    full, diag = stq.layer_errors(wd, wd, xd)
    assert torch.count_nonzero(full).item() == 0 and torch.count_nonzero(diag).item() == 0
    w_hat = dev(O.q2_roundtrip(w))
    a = stq.layer_errors(wd, w_hat, xd)
    b = stq.layer_errors(wd, w_hat, xd)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_layer_errors_full_size_sampled_rows(stq):
    """4096 x 7168 weights (one expert's gate/up matrix) with 512 calibration
    rows, the benchmark's shape, encoded on the GPU with the calibration
    imatrix; the oracle encodes sampled rows itself and scores them.  The
    2-bit stand-in of the same weights is checked on the sampled rows."""
    n, k, n_cal = 4096, 7168, 512
    w = S.gaussian_weights(41, n, k)
    x = S.paired_channel_layer(42, 1, k, n_cal, sign=1.0, coupling=0.5)[1]
    q = S.imatrix_from_calibration(x)
    wd = dev(w)
    w_hat = stq.dequantize_rows(stq.quantize_rows(wd, dev(q)), n, k)
    full, diag = stq.layer_errors(wd, w_hat, dev(x))
    full, diag = host(full), host(diag)
    rows = np.array([0, 1, 63, 64, 1000, 2047, 3333, 4095])
    ws = w[rows]
    ws_hat = O.dequantize_rows(O.quantize_rows(ws, q), len(rows), k)
    check_errors(full[rows], diag[rows], ws, ws_hat, x, "full size")
    assert np.all(np.isfinite(full)) and np.all(full > 0) and np.all(diag > 0)
    # the 2-bit stand-in at the same size, sampled rows bit for bit
    q2 = host(stq.q2_roundtrip(wd))
    assert np.array_equal(q2[rows].view(np.uint32), O.q2_roundtrip(ws).view(np.uint32))


def test_allocation_study_matches_oracle(stq):
    """Twelve synthetic layers scored on the GPU (encode, decode, 2-bit
    stand-in, both error measures), allocated by full-Hessian gain per
    byte: the same layers as the oracle picks from its own scores."""
    rng = np.random.default_rng(5)
    gains_gpu, gains_ref = [], []
    for l in range(12):
        w, x = S.paired_channel_layer(300 + l, 64, 1024, 96, sign=float(rng.choice([-1.0, 1.0])),
                                      coupling=float(rng.uniform(0.0, 0.95)))
        q = S.imatrix_from_calibration(x)
        wd, xd = dev(w), dev(x)
        stq_hat = stq.dequantize_rows(stq.quantize_rows(wd, dev(q)), 64, 1024)
        f_s, _ = stq.layer_errors(wd, stq_hat, xd)
        f_q, _ = stq.layer_errors(wd, stq.q2_roundtrip(wd), xd)
        gains_gpu.append(float(host(f_s).sum() - host(f_q).sum()))
        r_s, _ = O.layer_errors(w, O.dequantize_rows(O.quantize_rows(w, q), 64, 1024), x)
        r_q, _ = O.layer_errors(w, O.q2_roundtrip(w), x)
        gains_ref.append(float(r_s.sum() - r_q.sum()))
    np.testing.assert_allclose(gains_gpu, gains_ref, rtol=1e-9)
    extra = np.full(12, float((O.Q2_BLOCK_BYTES - O.BLOCK_BYTES) * 64 * 4))
    budget = extra.sum() / 2
    assert np.array_equal(stq.greedy_allocation(gains_gpu, extra, budget),
                          O.greedy_allocation(gains_ref, extra, budget))
