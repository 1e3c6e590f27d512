"""Pins of the oracle's routed-expert FFN (gate/up GEMV, SiLU(gate) * up,
down GEMV, routing-weighted combine) against values fixed by mathematics and
a hand-built expert, independent of the oracle's own code paths."""
import math

import numpy as np
import pytest

from oracle import stq_oracle as O


def test_silu_reference_values():
    # logistic(1) = 0.7310585786300049 (tabulated); silu(v) = v * logistic(v)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-16
    assert abs(O.silu(np.array([-1.0]))[0] + 0.2689414213699951) < 1e-16
    big = O.silu(np.array([50.0, -50.0]))
    assert abs(big[0] - 50.0) < 1e-12 and abs(big[1]) < 1e-18


def test_silu_odd_even_identity():
    # silu(v) - silu(-v) = v (logistic(v) + logistic(-v) = 1)
    v = np.random.default_rng(0).normal(0, 8, 2000)
    np.testing.assert_allclose(O.silu(v) - O.silu(-v), v, rtol=1e-13, atol=1e-13)


def test_silu_lipschitz_constant():
    v = np.linspace(-30, 30, 600001)
    slope = np.abs(np.diff(O.silu(v)) / np.diff(v))
    assert slope.max() <= O.SILU_LIPSCHITZ
    assert slope.max() > 1.09   # the constant is tight (max |silu'| = 1.0998...)


def _blocks(codes_per_row, d_bits, nb):
    """Packed matrix of len(codes_per_row) rows, every block with the same
    64 codes and scale bits."""
    n = len(codes_per_row)
    blocks = np.zeros((n, nb, O.BLOCK_BYTES), dtype=np.uint8)
    for r, codes in enumerate(codes_per_row):
        one = O.pack_blocks(np.array([d_bits[r]], dtype=np.uint16), np.asarray(codes, dtype=np.uint8)[None, :])
        blocks[r, :] = one[0]
    return O.pack_matrix(blocks)


def _hand_expert(d_model=256, d_ff=256):
    # gate rows: group 0 code 9 = (-1, 0, +1, +1), other groups code 0 = (0, +1, +1, +1), d = 1
    # up rows:   group 0 code 8 = (+1, 0, +1, +1), d = 2
    # down rows: all groups code 0, d = 1
    assert O.pattern_of_code(9) == (-1, 0, 1, 1) and O.pattern_of_code(8) == (1, 0, 1, 1)
    assert O.pattern_of_code(0) == (0, 1, 1, 1)
    gate = [9] + [0] * 63
    up = [8] + [0] * 63
    gu = _blocks([gate] * d_ff + [up] * d_ff, [0x3C00] * d_ff + [0x4000] * d_ff, d_model // 256)
    dn = _blocks([[0] * 64] * d_model, [0x3C00] * d_model, d_ff // 256)
    return gu, dn


def test_hand_built_expert():
    d_model = d_ff = 256
    gu, dn = _hand_expert()
    x = np.zeros((2, d_model))
    x[0, 0] = 1.0                      # token 0: unit vector, g = -1, u = 2; token 1: zeros
    pe = np.array([0, 1, 0, 1])
    pw = np.array([0.25, 0.75, 0.5, 0.5])
    y = O.moe_ffn_decode({0: gu, 1: gu}, {0: dn, 1: dn}, d_model, d_ff, x, pe, pw, 2)
    # h = silu(-1) * 2 = -0.5378828427399902; each down row adds lanes 1..3 of 64 groups: 192 h
    expect = 192 * 2 * -0.2689414213699951
    np.testing.assert_allclose(y[0], np.full(d_model, expect), rtol=1e-14)
    assert np.all(y[1] == 0.0)
    # gate and up swapped would give 192 * silu(2) * (-1): a different value
    assert abs(192 * (2 / (1 + math.exp(-2))) * -1 - expect) > 1.0


def test_linear_in_routing_weights():
    rng = np.random.default_rng(3)
    d_model, d_ff, E = 512, 256, 3
    gu = {e: O.quantize_rows(rng.normal(0, 0.05, (2 * d_ff, d_model)).astype(np.float32)) for e in range(E)}
    dn = {e: O.quantize_rows(rng.normal(0, 0.05, (d_model, d_ff)).astype(np.float32)) for e in range(E)}
    x = rng.normal(0, 1, (2, d_model))
    pe = np.array([0, 2, 1, 0])
    w1, w2 = rng.random(4), rng.random(4)
    y1 = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, w1, 2)
    y2 = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, w2, 2)
    y12 = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, w1 + w2, 2)
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-12, atol=1e-12 * np.abs(y12).max())


def test_unknown_expert_poisons_only_its_token():
    gu, dn = _hand_expert()
    x = np.ones((2, 256))
    y = O.moe_ffn_decode({0: gu}, {0: dn}, 256, 256, x, np.array([0, 7, 0, 0]), np.ones(4), 2)
    assert np.all(np.isnan(y[0])) and np.all(np.isfinite(y[1]))


@pytest.mark.parametrize("tol", [0.0, 1e-3])
def test_tolerance_is_nonnegative_and_grows_with_tol(tol):
    gu, dn = _hand_expert()
    x = np.random.default_rng(5).normal(0, 1, (1, 256))
    b0 = O.moe_ffn_tolerance({0: gu}, {0: dn}, 256, 256, x, np.array([0]), np.array([1.0]), 1, tol=0.0)
    b = O.moe_ffn_tolerance({0: gu}, {0: dn}, 256, 256, x, np.array([0]), np.array([1.0]), 1, tol=tol)
    assert np.all(b >= b0) and np.all(b0 >= 0) and np.all(np.isfinite(b))
