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


def _sgn(v):
    return np.where(np.asarray(v) < 0, -1.0, 1.0)


def _adversarial_ffn(gu, dn, d_model, d_ff, x, pe, pw, top_k, r_star, tol=0.0, eps_act=0.0, fp32=False):
    """A worst-case GPU of the routed-expert FFN, built independently of
    moe_ffn_tolerance: every GEMV output (gate, up, down) is moved by its
    full allowance tol * A, and the activation by eps_act * |h|, with signs
    chosen so that all moves add up at output column r_star[t] of token t.
    With fp32, SiLU(gate) * up is evaluated in fp32 and the routing combine
    is a chain of fp32 fused multiply-adds (else both are exact fp64).

    g' = g + dg*s, u' = u + du*s' with the signs of silu'(g)*u and silu(g)
    times the wanted sign of dh, so both first-order terms of
    h' - h = (silu(g') - silu(g)) u' + silu(g) (u' - u) push the same way;
    the wanted sign of dh_c is sign(w_k) * sign(W_down[r_star, c]), so
    W_down (h' - h) at r_star adds |W_down[r_star, c]| |dh_c| over c."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, d_model)
    y = np.zeros((x.shape[0], d_model), dtype=np.float64)
    for t in range(x.shape[0]):
        acc = np.zeros(d_model, dtype=np.float32 if fp32 else np.float64)
        for k in range(top_k):
            p = t * top_k + k
            e = int(pe[p])
            gu_e = O.gemv(gu[e], 2 * d_ff, d_model, x[t])
            g, u = gu_e[:d_ff], gu_e[d_ff:]
            a_gu = O.tolerance_scale(gu[e], 2 * d_ff, d_model, x[t])[0]
            dg, du = tol * a_gu[:d_ff], tol * a_gu[d_ff:]
            w_dn = O.dequantize_rows(dn[e], d_model, d_ff).astype(np.float64)
            want = _sgn(pw[p]) * _sgn(w_dn[r_star[t]])
            sig = 1.0 / (1.0 + np.exp(-g))
            dsilu = sig * (1.0 + g * (1.0 - sig))           # silu'(g)
            g2 = g + dg * want * _sgn(dsilu * u)
            u2 = u + du * want * _sgn(O.silu(g))
            if fp32:
                g32, u32 = g2.astype(np.float32), u2.astype(np.float32)
                h = ((g32 / (np.float32(1.0) + np.exp(-g32))) * u32).astype(np.float64)
            else:
                h = O.silu(g2) * u2
            h = h + eps_act * np.abs(h) * want
            h_exact = O.silu(g) * u
            lin = w_dn @ (h - h_exact)
            a_dn = O.tolerance_scale(dn[e], d_model, d_ff, np.abs(h))[0]
            z = w_dn @ h_exact + lin + tol * a_dn * _sgn(lin)   # the allowance adds to |lin|
            if fp32:   # w32 * z32 is exact in fp64: one rounding per step, as an fma
                acc = (acc.astype(np.float64) + np.float64(np.float32(pw[p])) * z.astype(np.float32)).astype(np.float32)
            else:
                acc = acc + np.float64(pw[p]) * z
        y[t] = acc
    return y


def _ffn_case(kind, seed, d_model, d_ff, E=3, T=3, top_k=2):
    """Experts, tokens and routing for the tolerance pins.  'random': N(0, 0.02)
    weights and N(0, 1) tokens (the gate's error term L*dg*|u| dominates);
    'gate_exact': gate rows of one all-positive pattern and positive tokens, so
    the gate sum has no cancellation and |silu(g)|*du dominates; 'no_cancel':
    gate and up rows of that pattern, so h is large against its error and the
    down projection's own allowance tol*A_down is a large share."""
    rng = np.random.default_rng(seed)
    def rand(n, k):
        return O.quantize_rows(rng.normal(0, 0.02, (n, k)).astype(np.float32))
    def positive(n, k, d_bits):
        # every group code 0 = (0, +1, +1, +1), scale d_bits
        blocks = np.zeros((n, k // 256, O.BLOCK_BYTES), dtype=np.uint8)
        one = O.pack_blocks(np.array([d_bits], dtype=np.uint16), np.zeros((1, 64), dtype=np.uint8))
        blocks[:, :] = one[0]
        return O.pack_matrix(blocks)
    gu, dn = {}, {}
    for e in range(E):
        dn[e] = rand(d_model, d_ff)
        if kind == "random":
            gu[e] = rand(2 * d_ff, d_model)
        else:
            g_rows = O.unpack_matrix(positive(d_ff, d_model, 0x2000 + 0x40 * e), d_ff, d_model // 256)
            u_src = positive(d_ff, d_model, 0x2400) if kind == "no_cancel" else rand(d_ff, d_model)
            u_rows = O.unpack_matrix(u_src, d_ff, d_model // 256)
            gu[e] = O.pack_matrix(np.concatenate([g_rows, u_rows]))
    if kind == "random":
        x = rng.normal(0, 1, (T, d_model))
    else:
        x = rng.uniform(0.5, 1.5, (T, d_model))
    x = x.astype(np.float32).astype(np.float64)
    pe = np.stack([rng.choice(E, top_k, replace=top_k > E) for _ in range(T)]).reshape(-1)
    pw = rng.random(T * top_k).astype(np.float32)
    pw[1] = -pw[1]                                        # a negative routing weight too
    r_star = rng.integers(0, d_model, T)
    return gu, dn, x, pe, pw, r_star


# (case, the share of the bound the adversary must reach at its columns)
GEMV_TERM_CASES = [("random", 0.5), ("gate_exact", 0.8), ("no_cancel", 0.8)]


@pytest.mark.parametrize("kind,reach", GEMV_TERM_CASES)
def test_tolerance_gemv_terms_cover_worst_case_and_are_tight(kind, reach):
    """The GEMV part of moe_ffn_tolerance (eps_act = eps_sum = 0) holds for
    every FFN whose three GEMVs stay inside |err| <= 1e-3 * A, and is not
    loose: at the aimed columns the deviation reaches `reach` of the bound.
    A dropped term fails the first check in the case it dominates (|W_down|
    dh in 'random', |silu(g)| du in 'gate_exact', tol * A_down in
    'no_cancel'); an inflated one (a wrong Lipschitz factor, A_down on a
    wrong vector, a scaled bound) fails the second."""
    d_model, d_ff, top_k, tol = 512, 256, 2, 1e-3
    gu, dn, x, pe, pw, r_star = _ffn_case(kind, 11, d_model, d_ff, top_k=top_k)
    T = x.shape[0]
    y = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    bound = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, x, pe, pw, top_k, tol=tol, eps_act=0.0, eps_sum=0.0)
    dev = np.abs(_adversarial_ffn(gu, dn, d_model, d_ff, x, pe, pw, top_k, r_star, tol=tol) - y)
    assert np.all(dev <= bound * (1 + 1e-9)), float(np.max(dev / bound))
    aimed = dev[np.arange(T), r_star] / bound[np.arange(T), r_star]
    assert np.all(aimed >= reach), aimed


def test_tolerance_activation_term_is_exact():
    """With tol = 0 and no combine term, the bound is the activation allowance
    eps_act*|h| carried through |W_down| and the routing weights: an
    activation moved by exactly that much, aimed at one column, reaches it."""
    d_model, d_ff, top_k = 512, 256, 2
    gu, dn, x, pe, pw, r_star = _ffn_case("random", 12, d_model, d_ff, top_k=top_k)
    T = x.shape[0]
    y = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    bound = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, x, pe, pw, top_k, tol=0.0, eps_act=1e-6, eps_sum=0.0)
    dev = np.abs(_adversarial_ffn(gu, dn, d_model, d_ff, x, pe, pw, top_k, r_star, eps_act=1e-6) - y)
    assert np.all(dev <= bound * (1 + 1e-6))
    aimed = dev[np.arange(T), r_star] / bound[np.arange(T), r_star]
    np.testing.assert_allclose(aimed, 1.0, rtol=1e-3)


def test_tolerance_combine_term_covers_fp32_rounding():
    """With tol = 0 and eps_act = 0 the bound is the fp32 combine's rounding
    allowance alone: an exact FFN combined in fp32 stays inside it, and with
    eight routed pairs the rounding reaches a visible share of it."""
    d_model, d_ff, top_k = 256, 256, 8
    gu, dn, x, pe, pw, r_star = _ffn_case("random", 13, d_model, d_ff, E=8, T=4, top_k=top_k)
    y = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    bound = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, x, pe, pw, top_k, tol=0.0, eps_act=0.0)
    x = np.asarray(x)
    # exact pair outputs, combined by the fp32 fma chain only
    acc = np.zeros((x.shape[0], d_model), dtype=np.float32)
    for k in range(top_k):
        z = np.stack([O._ffn_pair(gu[int(pe[t * top_k + k])], dn[int(pe[t * top_k + k])], d_model, d_ff, x[t], d_model)[3]
                      for t in range(x.shape[0])])
        w = np.array([np.float32(pw[t * top_k + k]) for t in range(x.shape[0])], dtype=np.float64)[:, None]
        acc = (acc.astype(np.float64) + w * z.astype(np.float32)).astype(np.float32)
    dev = np.abs(acc.astype(np.float64) - y)
    assert np.all(dev <= bound)
    assert np.max(dev / bound) >= 0.05


@pytest.mark.parametrize("seed,d_model,d_ff,top_k", [(11, 512, 256, 2), (12, 256, 512, 4)])
def test_tolerance_holds_for_an_fp32_gpu(seed, d_model, d_ff, top_k):
    """All terms at once: GEMVs at their full allowance, fp32 SiLU * up and an
    fp32 combine stay inside the bound with its default constants."""
    rng_kind = "random"
    gu, dn, x, pe, pw, r_star = _ffn_case(rng_kind, seed, d_model, d_ff, top_k=top_k)
    y = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    bound = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    for tol in (1e-3, 0.0):
        dev = np.abs(_adversarial_ffn(gu, dn, d_model, d_ff, x, pe, pw, top_k, r_star, tol=tol, fp32=True) - y)
        assert np.all(dev <= bound), float(np.max(dev / bound))


def test_down_row_subset_gives_those_rows():
    """Rows of the down projection are independent: an FFN whose down
    matrices hold only rows R gives the full FFN's columns R, value and bound."""
    d_model, d_ff, top_k = 512, 256, 2
    gu, dn, x, pe, pw, _ = _ffn_case("random", 14, d_model, d_ff, top_k=top_k)
    R = np.array([0, 7, 300, 511])
    dn_r = {e: O.pack_matrix(O.unpack_matrix(m, d_model, d_ff // 256)[R]) for e, m in dn.items()}
    y = O.moe_ffn_decode(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    b = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, x, pe, pw, top_k)
    y_r = O.moe_ffn_decode(gu, dn_r, d_model, d_ff, x, pe, pw, top_k, n_out=len(R))
    b_r = O.moe_ffn_tolerance(gu, dn_r, d_model, d_ff, x, pe, pw, top_k, n_out=len(R))
    np.testing.assert_allclose(y_r, y[:, R], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(b_r, b[:, R], rtol=1e-14, atol=1e-18)
