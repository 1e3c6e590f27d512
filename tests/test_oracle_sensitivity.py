"""Pins of the oracle's layer-sensitivity tools (full-Hessian and diagonal
reconstruction error, the stand-in 2-bit format, greedy per-byte allocation,
Spearman correlation), and the study the pages describe: with correlated
calibration activations the full-Hessian ranking of layers differs from the
diagonal one, and allocating by it leaves less full-Hessian error."""
import numpy as np
import pytest

from oracle import stq_oracle as O
import synth_inputs as S


def test_full_equals_diagonal_when_the_hessian_is_diagonal():
    rng = np.random.default_rng(0)
    w = rng.normal(0, 0.02, (5, 256)).astype(np.float32)
    w_hat = O.q2_roundtrip(w)
    sigma = rng.uniform(0.5, 3.0, 256)
    x = np.diag(sigma)                               # calibration rows sigma_k e_k: X^T X diagonal
    full, diag = O.layer_errors(w, w_hat, x)
    np.testing.assert_allclose(full, diag, rtol=1e-12)


def test_full_error_by_brute_force():
    rng = np.random.default_rng(1)
    w = rng.normal(0, 1, (3, 7))
    w_hat = rng.normal(0, 1, (3, 7))
    x = rng.normal(0, 1, (4, 7))
    full, diag = O.layer_errors(w, w_hat, x)
    for r in range(3):
        f = sum(sum((w[r, k] - w_hat[r, k]) * x[i, k] for k in range(7)) ** 2 for i in range(4))
        d = sum(sum(x[i, k] ** 2 for i in range(4)) * (w[r, k] - w_hat[r, k]) ** 2 for k in range(7))
        assert abs(full[r] - f) <= 1e-12 * f and abs(diag[r] - d) <= 1e-12 * d


def test_tolerance_covers_an_exactly_rounded_evaluation():
    """math.fsum gives each dot product and each final sum correctly rounded;
    the oracle's numpy evaluation stays within the stated bound of it, and
    the bound is tiny against the errors themselves."""
    import math
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, (6, 512)).astype(np.float32)
    w_hat = O.q2_roundtrip(w)
    x = (rng.normal(0, 1, (40, 512)) * rng.uniform(0.1, 10, 512)).astype(np.float32)
    full, diag = O.layer_errors(w, w_hat, x)
    b_full, b_diag = O.layer_errors_tolerance(w, w_hat, x)
    d = w.astype(np.float64) - w_hat.astype(np.float64)
    xd = x.astype(np.float64)
    hd = [math.fsum(xd[:, c] ** 2) for c in range(512)]
    for r in range(6):
        p = [math.fsum(d[r] * xd[i]) for i in range(40)]
        f = math.fsum(v * v for v in p)
        g = math.fsum(hd[c] * d[r, c] ** 2 for c in range(512))
        assert abs(full[r] - f) <= b_full[r] and abs(diag[r] - g) <= b_diag[r]
    assert np.all(b_full < 1e-9 * full) and np.all(b_diag < 1e-12 * diag)


def test_q2_hand_block():
    # 192 weights of 0.6 and 64 of -1.8: mean square 1.08, rms 1.0392..., s = rms/2 -> fp16 0.51953125;
    # 0.6 < 2s = 1.0390625 takes s, 1.8 takes 3s
    w = np.concatenate([np.full(192, 0.6), np.full(64, -1.8)]).astype(np.float32)[None, :]
    rec = O.q2_roundtrip(w)[0]
    assert np.all(rec[:192] == np.float32(0.51953125))
    assert np.all(rec[192:] == np.float32(-3 * 0.51953125))


def test_q2_beats_stq_on_gaussian_rows():
    w = S.gaussian_weights(3, 64, 1024)
    q2 = O.weighted_error(w, O.q2_roundtrip(w))
    stq = O.weighted_error(w, O.dequantize_rows(O.quantize_rows(w), 64, 1024))
    assert q2 < 0.6 * stq
    assert O.Q2_BLOCK_BYTES * 8 / 256 == 2.0625 and O.BLOCK_BYTES * 8 / 256 == 1.3125


def test_greedy_allocation_hand_case():
    # ratios 2, 3, 2, 1: take 1 (2 bytes), skip 0 (would need 7), take 2 (5), take 3 (6)
    chosen = O.greedy_allocation([10, 6, 6, 1], [5, 2, 3, 1], 6)
    assert chosen.tolist() == [False, True, True, True]
    assert not O.greedy_allocation([1, 2], [3, 3], 2).any()


def test_spearman_against_scipy():
    from scipy.stats import spearmanr
    rng = np.random.default_rng(4)
    a = rng.integers(0, 6, 40).astype(float)
    b = a + rng.normal(0, 2, 40)
    assert abs(O.spearman(a, b) - spearmanr(a, b).statistic) < 1e-12


@pytest.fixture(scope="module")
def layers():
    """12 synthetic layers (64 x 1024 rows) with paired, correlated columns;
    per layer a weight scale, a pair sign and a coupling drawn at random, so
    that the off-diagonal Hessian terms raise or cancel the error by a
    layer-dependent factor.  Per layer: summed full and diagonal error of the
    STQ1_0 encoding (with the diagonal imatrix) and of the 2-bit stand-in."""
    rng = np.random.default_rng(5)
    out = []
    for l in range(12):
        w, x = S.paired_channel_layer(100 + l, 64, 1024, 256, sign=float(rng.choice([-1.0, 1.0])),
                                      coupling=float(rng.uniform(0.0, 0.95)))
        w = (w * rng.uniform(0.7, 1.4)).astype(np.float32)
        stq = O.dequantize_rows(O.quantize_rows(w, S.imatrix_from_calibration(x)), 64, 1024)
        q2 = O.q2_roundtrip(w)
        f_s, d_s = O.layer_errors(w, stq, x)
        f_q, d_q = O.layer_errors(w, q2, x)
        out.append((f_s.sum(), d_s.sum(), f_q.sum(), d_q.sum()))
    return np.array(out)


def test_paired_columns_scale_the_full_error():
    # exact mirror (sign -1) with identical activations (coupling 1): the pair's
    # contributions cancel in w x, so the full error is ~0 while the diagonal
    # estimate is not; sign +1 doubles it
    w, x = S.paired_channel_layer(7, 8, 512, 32, sign=-1.0, coupling=1.0)
    full, diag = O.layer_errors(w, O.q2_roundtrip(w), x)
    assert np.all(full < 1e-6 * diag)
    w, x = S.paired_channel_layer(7, 8, 512, 256, sign=1.0, coupling=1.0)
    full, diag = O.layer_errors(w, O.q2_roundtrip(w), x)
    assert abs(full.sum() / diag.sum() - 2.0) < 0.1


def test_full_and_diagonal_rankings_differ(layers):
    gain_full = layers[:, 0] - layers[:, 2]
    gain_diag = layers[:, 1] - layers[:, 3]
    assert np.all(gain_full > 0) and np.all(gain_diag > 0)
    assert O.spearman(gain_full, gain_diag) < 0.9


def test_allocating_by_full_hessian_leaves_less_full_error(layers):
    extra = np.full(len(layers), (O.Q2_BLOCK_BYTES - O.BLOCK_BYTES) * 64 * 4)
    budget = extra.sum() / 2
    by_full = O.greedy_allocation(layers[:, 0] - layers[:, 2], extra, budget)
    by_diag = O.greedy_allocation(layers[:, 1] - layers[:, 3], extra, budget)
    err = lambda chosen: float(np.where(chosen, layers[:, 2], layers[:, 0]).sum())
    assert by_full.sum() == by_diag.sum() == len(layers) // 2
    assert err(by_full) <= err(by_diag)
