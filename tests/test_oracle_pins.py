"""Pins of the CPU oracle against things fixed outside of it.

Each test checks the oracle against enumeration, exact rational arithmetic,
closed forms, brute force or hand-derived values -- never against a copy of
its own formula.  These run on the CPU (no GPU marker).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import stq_oracle as O
import synth_inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stq1_0_layout_examples.json")


# ---------------------------------------------------------------------------
# P1 codebook: the 32 codes are exactly the one-zero ternary patterns
# (lemmy post 66506, "Four weights, five bits"; alphasignal "How STQ1_0 works")
# ---------------------------------------------------------------------------
def test_codebook_is_exactly_the_one_zero_patterns():
    want = {t for t in itertools.product((-1, 0, 1), repeat=4) if t.count(0) == 1}
    assert len(want) == 32 == 4 * 8                      # 4 zero positions x 8 sign choices
    got = [tuple(int(v) for v in row) for row in O.CODEBOOK]
    assert len(set(got)) == 32                           # injective
    assert set(got) == want                              # onto
    assert 2 ** 5 == 32                                  # five bits


def test_code_inverse_and_zero_lane_sign_ignored():
    for c in range(32):
        t = O.CODEBOOK[c]
        z = int(np.flatnonzero(t == 0)[0])
        neg = t < 0
        assert O.codes_from_pattern(np.array(z), neg) == c
        neg2 = neg.copy()
        neg2[z] = not neg2[z]                            # flipping the zero lane's sign flag changes nothing
        assert O.codes_from_pattern(np.array(z), neg2) == c


def test_table_select_bit_marks_zero_in_upper_pair():
    for c in range(32):
        z = int(np.flatnonzero(O.CODEBOOK[c] == 0)[0])
        assert (c >> 4) == (z >> 1)


def test_hand_derived_patterns():
    gold = json.load(open(GOLDEN))["patterns"]
    for c, t in gold.items():
        assert list(O.CODEBOOK[int(c)]) == t, c


# ---------------------------------------------------------------------------
# P2 sizes (lemmy "Four weights, five bits"; alphasignal "How STQ1_0 works")
# ---------------------------------------------------------------------------
def test_sizes():
    assert O.BLOCK_BYTES == 2 + 32 + 8 == 42
    assert Fraction(O.BLOCK_BYTES * 8, O.QK) == Fraction(13125, 10000)    # 1.3125 bpw
    assert Fraction(5, 4) == Fraction(125, 100)                          # codes alone: 1.25 bpw
    assert O.row_bytes(1024) == 168 and O.row_bytes(7168) == 1176
    assert 256 * O.row_bytes(1024) == 43008
    assert 4096 * O.row_bytes(7168) == 4816896
    assert 256 * 4096 * O.row_bytes(7168) == 1233125376
    with pytest.raises(ValueError):
        O.row_bytes(1000)


# ---------------------------------------------------------------------------
# O2 layout: hand-derived bytes, bijectivity of the bit map
# ---------------------------------------------------------------------------
def test_pack_matches_hand_derived_bytes():
    gold = json.load(open(GOLDEN))["blocks"]
    for ex in gold:
        codes = np.zeros((1, 64), dtype=np.uint8)
        for g, c in ex["codes"].items():
            codes[0, int(g)] = c
        raw = O.pack_blocks(np.array([int(ex["d_bits"], 16)], dtype=np.uint16), codes)[0]
        want = np.zeros(42, dtype=np.uint8)
        for pos, v in ex["bytes"].items():
            want[int(pos)] = int(v, 16)
        assert raw.tolist() == want.tolist(), ex


def test_matrix_layout_matches_hand_derived_offsets():
    gold = json.load(open(GOLDEN))["matrix_offsets"]
    n, nb = gold["n_rows"], gold["nb"]
    for r, b, off in gold["offsets"]:
        assert O.block_offset(r, b, n, nb) == off, (r, b)
    # every block has its own 42 bytes and the matrix is exactly n*nb*42 bytes
    offs = sorted(O.block_offset(r, b, n, nb) for r in range(n) for b in range(nb))
    assert offs == list(range(0, n * nb * 42, 42))
    blocks = np.random.default_rng(2).integers(0, 256, size=(n, nb, 42)).astype(np.uint8)
    flat = O.pack_matrix(blocks)
    assert np.array_equal(O.unpack_matrix(flat, n, nb), blocks)
    for r, b, off in gold["offsets"]:
        assert np.array_equal(flat[off:off + 42], blocks[r, b])


def test_every_code_bit_has_its_own_position():
    seen = {}
    for g in range(64):
        byte, shift = O.qs_position(g)
        for b in range(4):
            key = (byte, shift + b)
            assert key not in seen
            seen[key] = (g, b)
        byte, bit = O.qh_position(g)
        assert (byte, bit) not in seen
        seen[(byte, bit)] = (g, 4)
    assert len(seen) == 320                              # 40 bytes of codes, every bit used once
    assert {k[0] for k in seen} == set(range(2, 42))


def test_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 32, size=(50, 64)).astype(np.uint8)
    d16 = rng.integers(0, 65536, size=50).astype(np.uint16)
    raw = O.pack_blocks(d16, codes)
    d2, c2 = O.unpack_blocks(raw)
    assert np.array_equal(d2, d16) and np.array_equal(c2, codes)


# ---------------------------------------------------------------------------
# O3 decode
# ---------------------------------------------------------------------------
def test_decode_values_and_signed_zero():
    gold = json.load(open(GOLDEN))["patterns"]
    for d_bits, d_val in [(0x3800, 0.5), (0xBC00, -1.0), (0x8000, -0.0), (0x0001, 2.0 ** -24)]:
        codes = np.zeros((1, 64), dtype=np.uint8)
        for i, c in enumerate(gold):
            codes[0, i] = int(c)
        raw = O.pack_blocks(np.array([d_bits], dtype=np.uint16), codes)
        w = O.dequantize_rows(raw, 1, 256)[0]
        for i, (c, t) in enumerate(gold.items()):
            for j in range(4):
                v = w[4 * i + j]
                if t[j] == 0:
                    assert v == 0.0 and not math.copysign(1.0, v) < 0       # +0.0 in the zero lane
                else:
                    want = np.float32(d_val) if t[j] > 0 else -np.float32(d_val)
                    assert np.float32(v).tobytes() == np.float32(want).tobytes()


# ---------------------------------------------------------------------------
# P3 round trips and special blocks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("encoder", ["wls", "amax"])
def test_quantize_of_decoded_valid_blocks_is_identity(encoder):
    rng = np.random.default_rng(5)
    nb = 40
    codes = rng.integers(0, 32, size=(nb, 64)).astype(np.uint8)
    # random positive *normal* fp16 scales
    exp = rng.integers(1, 31, size=nb)
    man = rng.integers(0, 1024, size=nb)
    d16 = ((exp << 10) | man).astype(np.uint16)
    raw = O.pack_matrix(O.pack_blocks(d16, codes).reshape(4, 10, 42))   # 4 rows x 10 blocks
    w = O.dequantize_rows(raw, 4, 2560)
    q = rng.uniform(0.05, 3.0, size=2560).astype(np.float32)
    again = O.quantize_rows(w, q, encoder=encoder, rounds=3)
    assert np.array_equal(again, raw)


@pytest.mark.parametrize("encoder", ["wls", "amax"])
def test_all_zero_block_packs_to_zero_bytes(encoder):
    for w0 in (0.0, -0.0):
        w = np.full((2, 256), w0, dtype=np.float32)
        assert not O.quantize_rows(w, None, encoder=encoder).any()


def test_constant_block():
    a = np.float32(0.375)                                 # exactly representable in fp16
    w = np.full((1, 256), a, dtype=np.float32)
    for enc in ("wls", "amax"):
        raw = O.quantize_rows(w, None, encoder=enc)
        d16, codes = O.unpack_blocks(raw)
        assert not codes.any()                            # zero in lane 0, all +
        assert O.fp16_bits_to_f32(d16)[0] == a
        w_hat = O.dequantize_rows(raw, 1, 256)
        assert O.weighted_error(w, w_hat) == 64 * float(a) ** 2


def test_rounds_zero_is_single_fit_of_amax_pattern():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(3, 512)).astype(np.float32)
    q = rng.uniform(0.1, 2, size=512).astype(np.float32)
    tr = O.encode_trace(w, q, rounds=0)
    assert len(tr["z"]) == 1 and len(tr["d"]) == 1
    raw = O.quantize_rows(w, q, rounds=0)
    d16, codes = O.unpack_blocks(raw)
    amax_codes = O.unpack_blocks(O.quantize_rows(w, q, encoder="amax"))[1]
    assert np.array_equal(codes, amax_codes)              # same pattern as the amax encoder
    assert not np.array_equal(d16, O.unpack_blocks(O.quantize_rows(w, q, encoder="amax"))[0])


# ---------------------------------------------------------------------------
# P4 step optimality in exact rational arithmetic
# ---------------------------------------------------------------------------
def _one_zero_patterns():
    return [t for t in itertools.product((-1, 0, 1), repeat=4) if t.count(0) == 1]


def test_choose_zero_is_exact_best_pattern_for_fixed_d():
    rng = np.random.default_rng(21)
    pats = _one_zero_patterns()
    close = 0
    for _ in range(400):
        w = rng.normal(0, 1, size=4).astype(np.float32)
        q = (rng.chisquare(2, size=4) / 2 + 1e-3).astype(np.float32)
        d = float(rng.uniform(0.05, 2.0))
        absw = np.abs(w.astype(np.float64)).reshape(1, 1, 4)
        z = int(O.choose_zero(absw, q.astype(np.float64).reshape(1, 1, 4), np.array([d]))[0, 0])
        W = [Fraction(float(v)) for v in w]
        Q = [Fraction(float(v)) for v in q]
        D = Fraction(d)
        # exact best error for each zero lane, over every sign choice of the other lanes
        best_by_lane = {}
        for t in pats:
            e = sum(Q[j] * (W[j] - D * t[j]) ** 2 for j in range(4))
            j0 = t.index(0)
            best_by_lane[j0] = min(best_by_lane.get(j0, e), e)
        best = min(best_by_lane.values())
        lowest_best_lane = min(j for j, e in best_by_lane.items() if e == best)
        if z != lowest_best_lane:
            # allowed only inside fp64 rounding of the per-lane costs
            close += 1
            assert float(best_by_lane[z] - best) <= 1e-12 * float(best + 1), (w, q, d)
    assert close <= 2


def test_wls_scale_is_exact_minimiser():
    rng = np.random.default_rng(8)
    w = rng.normal(0, 0.02, size=(2, 512)).astype(np.float32)
    q = rng.uniform(0.0, 3.0, size=512).astype(np.float32)
    tr = O.encode_trace(w, q, rounds=1)
    absw, qq = tr["absw"], tr["q"]
    for r in range(2):
        z = tr["z"][r]
        d = tr["d"][r]
        for idx in [(0, 0), (0, 1), (1, 0), (1, 1)]:
            num = Fraction(0)
            den = Fraction(0)
            for g in range(64):
                for j in range(4):
                    if j != z[idx][g]:
                        num += Fraction(float(qq[idx][g, j])) * Fraction(float(absw[idx][g, j]))
                        den += Fraction(float(qq[idx][g, j]))
            exact = num / den
            assert abs(Fraction(float(d[idx])) - exact) <= exact * Fraction(1, 2 ** 50)
            # closed form: E(d) = E(d*) + den*(d-d*)^2, so any other d is worse
            for delta in (Fraction(1, 10 ** 6), -Fraction(1, 10 ** 6)):
                dd = exact + delta * exact
                e_star = O.pattern_error(absw[idx][None], qq[idx][None], z[idx][None], np.array([float(exact)]))[0]
                e_dd = O.pattern_error(absw[idx][None], qq[idx][None], z[idx][None], np.array([float(dd)]))[0]
                assert e_dd >= e_star


def test_zero_weight_columns_give_zero_scale():
    w = np.random.default_rng(1).normal(0, 1, size=(1, 256)).astype(np.float32)
    q = np.zeros(256, dtype=np.float32)
    d16, _ = O.unpack_blocks(O.quantize_rows(w, q))
    assert d16[0] == 0


# ---------------------------------------------------------------------------
# P5 brute force on tiny blocks: the encoder never beats the global optimum,
# and usually reaches it.  Groups beyond the first G get q = 0.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G,trials", [(1, 300), (2, 150), (3, 25)])
def test_brute_force_tiny_blocks(G, trials):
    rng = np.random.default_rng(100 + G)
    pats = np.array(_one_zero_patterns(), dtype=np.float64)          # [32, 4]
    hits = 0
    for _ in range(trials):
        w = np.zeros((1, 256), dtype=np.float32)
        w[0, :4 * G] = rng.normal(0, 1, size=4 * G)
        w[0, 4 * G:] = rng.normal(0, 1, size=256 - 4 * G)
        q = np.zeros(256, dtype=np.float32)
        q[:4 * G] = (rng.chisquare(2, size=4 * G) / 2 + 1e-3).astype(np.float32)
        tr = O.encode_trace(w, q, rounds=3)
        z, d = tr["z"][-1][0, 0, :G], float(tr["d"][-1][0, 0])
        wg = w[0, :4 * G].astype(np.float64).reshape(G, 4)
        qg = q[:4 * G].astype(np.float64).reshape(G, 4)
        t_enc = np.where(np.arange(4)[None] == z[:, None], 0.0, np.where(wg < 0, -1.0, 1.0))
        e_enc = np.sum(qg * (wg - d * t_enc) ** 2)
        # exhaustive: every combination of G patterns with its optimal real d
        best = np.inf
        for combo in itertools.product(range(32), repeat=G):
            t = pats[list(combo)]
            den = np.sum(qg * t * t)
            dd = np.sum(qg * wg * t) / den if den > 0 else 0.0
            best = min(best, np.sum(qg * (wg - dd * t) ** 2))
        assert e_enc >= best * (1 - 1e-12) - 1e-300
        hits += e_enc <= best * (1 + 1e-9)
    assert hits / trials >= 0.8                                      # not required to be 1


# ---------------------------------------------------------------------------
# P6 errors never increase along the rounds (exact in Fraction on a small case,
# fp64 with 1e-12 slack on a larger one)
# ---------------------------------------------------------------------------
def _exact_block_error(w, q, z, d):
    e = Fraction(0)
    D = Fraction(float(d))
    for g in range(64):
        for j in range(4):
            wv = Fraction(float(w[4 * g + j]))
            qv = Fraction(float(q[4 * g + j]))
            t = 0 if j == z[g] else (1 if w[4 * g + j] >= 0 else -1)
            e += qv * (wv - D * t) ** 2
    return e


def test_rounds_never_increase_error_exact():
    rng = np.random.default_rng(77)
    w = rng.standard_t(3, size=(1, 256)).astype(np.float32) * np.float32(0.02)
    q = (rng.chisquare(1, size=256) + 1e-4).astype(np.float32)
    tr = O.encode_trace(w, q, rounds=3)
    amax = float(np.max(np.abs(w)))
    seq = [_exact_block_error(w[0], q, tr["z"][0][0, 0], amax)]
    for r in range(4):
        if r >= 1:
            # choice step alone: new pattern with the previous d
            seq.append(_exact_block_error(w[0], q, tr["z"][r][0, 0], tr["d"][r - 1][0, 0]))
        seq.append(_exact_block_error(w[0], q, tr["z"][r][0, 0], tr["d"][r][0, 0]))
    for a, b in zip(seq, seq[1:]):
        assert b <= a * (1 + Fraction(1, 10 ** 12))


def test_rounds_never_increase_error_fp64():
    w, q, _ = S.single_gemv_case()
    tr = O.encode_trace(w, q, rounds=3)
    absw, qq = tr["absw"], tr["q"]
    amax = absw.reshape(absw.shape[0], absw.shape[1], -1).max(axis=-1)
    e = [O.pattern_error(absw, qq, tr["z"][0], amax)]
    for r in range(4):
        e.append(O.pattern_error(absw, qq, tr["z"][r], tr["d"][r]))
    for a, b in zip(e, e[1:]):
        assert np.all(b <= a * (1 + 1e-12))
    assert np.sum(e[-1]) < np.sum(e[1])                  # the rounds do move something


# ---------------------------------------------------------------------------
# P7 well below the amax encoder on the small GEMV case
# (the pages report roughly 90% / 89.7% on real rows)
# ---------------------------------------------------------------------------
def test_reduction_against_amax_on_small_case():
    w, q, _ = S.single_gemv_case()
    e = {}
    for enc in ("wls", "amax"):
        w_hat = O.dequantize_rows(O.quantize_rows(w, q, encoder=enc), 256, 1024)
        e[enc] = O.weighted_error(w, w_hat, q)
    red = 1.0 - e["wls"] / e["amax"]
    assert 0.85 <= red < 1.0, red


# ---------------------------------------------------------------------------
# P8 worked example (one group, its own d), checked with exact rationals
# ---------------------------------------------------------------------------
def test_worked_example_zero_is_not_the_smallest_weight():
    wv = [0.10, 0.12, 1.0, 1.0]
    qv = [0.1, 10.0, 1.0, 1.0]
    w = np.full((1, 256), 0.5, dtype=np.float32)
    q = np.zeros(256, dtype=np.float32)
    w[0, :4] = wv
    q[:4] = qv
    # hand computation with exact rationals (on the exact decimal inputs)
    Wx = [Fraction(1, 10), Fraction(12, 100), Fraction(1), Fraction(1)]
    Qx = [Fraction(1, 10), Fraction(10), Fraction(1), Fraction(1)]
    e_amax = Qx[0] * Wx[0] ** 2 + Qx[1] * (Wx[1] - 1) ** 2
    assert e_amax == Fraction(7745, 1000)
    d0 = (Qx[1] * Wx[1] + 2) / (Qx[1] + 2)
    assert d0 == Fraction(4, 15)
    costs = [Qx[j] * (2 * Wx[j] - d0) for j in range(4)]
    assert min(range(4), key=lambda j: costs[j]) == 1                 # not lane 0, the smallest |w|
    d1 = (Qx[0] * Wx[0] + 2) / (Qx[0] + 2)
    assert d1 == Fraction(67, 70)
    # the oracle on the fp32-rounded inputs
    tr = O.encode_trace(w, q, rounds=3)
    assert int(tr["z"][0][0, 0, 0]) == 0
    assert abs(tr["d"][0][0, 0] - float(d0)) < 1e-7
    assert int(tr["z"][1][0, 0, 0]) == 1
    assert abs(tr["d"][-1][0, 0] - float(d1)) < 1e-7
    raw = O.quantize_rows(w, q)
    d16, codes = O.unpack_blocks(raw)
    assert d16[0] == 0x3BA8                                           # fp16(67/70) = 0.95703125
    assert codes[0, 0] == 8                                           # zero in lane 1, all +
    e_final = O.pattern_error(tr["absw"], tr["q"], tr["z"][-1], tr["d"][-1])[0, 0]
    assert abs(e_final - 0.2211428571) < 1e-6


def test_amax_encoder_on_hand_block():
    w = np.zeros((1, 256), dtype=np.float32)
    w[0, :8] = [0.5, -0.25, 1.0, -2.0, -0.0, 0.75, -0.75, 0.125]
    raw = O.quantize_rows(w, None, encoder="amax")
    d16, codes = O.unpack_blocks(raw)
    assert O.fp16_bits_to_f32(d16)[0] == 2.0
    # group 0: smallest |w| is lane 1; lanes 0,2,3 signs (+,+,-) -> m = 0b100 -> c = 8+4
    assert codes[0, 0] == 12
    # group 1: smallest |w| is lane 0 (-0.0 counts as +); lanes 1..3 = (+,-,+) -> m = 0b010
    assert codes[0, 1] == 2
    assert np.all(codes[0, 2:] == 0)


# ---------------------------------------------------------------------------
# reduction order of the encoder (balanced tree of adjacent pairs)
# ---------------------------------------------------------------------------
def test_encoder_sum_order_is_the_documented_tree():
    # lane magnitudes chosen so sequential and tree sums differ in fp64
    rng = np.random.default_rng(9)
    w = np.zeros((1, 256), dtype=np.float32)
    w[0] = (rng.uniform(0.5, 1.0, size=256) * np.where(rng.random(256) < 0.5, 1e-7, 1.0)).astype(np.float32)
    q = rng.uniform(0.1, 10, size=256).astype(np.float32)
    tr = O.encode_trace(w, q, rounds=0)
    z = tr["z"][0][0, 0]
    vals = []
    for g in range(64):
        s = 0.0
        for j in range(4):
            s = s + (float(q[4 * g + j]) * abs(float(w[0, 4 * g + j])) if j != z[g] else 0.0)
        vals.append(s)

    def tree(v):
        if len(v) == 1:
            return v[0]
        h = len(v) // 2
        return tree(v[:h]) + tree(v[h:])

    def seq(v):
        s = 0.0
        for x in v:
            s += x
        return s

    den = []
    for g in range(64):
        s = 0.0
        for j in range(4):
            s = s + (float(q[4 * g + j]) if j != z[g] else 0.0)
        den.append(s)
    want = tree(vals) / tree(den)
    assert tr["d"][0][0, 0] == want
    assert seq(vals) != tree(vals) or seq(den) != tree(den)      # the order is actually exercised


def test_fp16_scale_rounding_reading():
    d = np.array([0.0, 1.0, 67 / 70, 65504.0, 65519.0, 1e9, 2.0 ** -24, 2.0 ** -26, 1 / 3])
    bits = O.fp16_scale_bits(d)
    assert bits[0] == 0 and bits[1] == 0x3C00 and bits[2] == 0x3BA8
    assert bits[3] == 0x7BFF and bits[4] == 0x7BFF and bits[5] == 0x7BFF   # clamped to 65504
    assert bits[6] == 0x0001 and bits[7] == 0x0000
    assert bits[8] == 0x3555                                                # 1/3 -> 0.333251953125


# ---------------------------------------------------------------------------
# O7 / O8 products
# ---------------------------------------------------------------------------
def _small_packed(seed, n, k):
    w = S.gaussian_weights(seed, n, k)
    return O.quantize_rows(w, None)


def test_gemv_unit_vectors_give_columns_exactly():
    n, k = 8, 512
    q = _small_packed(4, n, k)
    w_hat = O.dequantize_rows(q, n, k)
    for col in (0, 3, 255, 256, 511):
        x = np.zeros(k, dtype=np.float32)
        x[col] = 1.0
        assert np.array_equal(O.gemv(q, n, k, x), w_hat[:, col].astype(np.float64))


def test_gemv_block_indicator_counts_signs():
    n, k = 6, 768
    q = _small_packed(5, n, k)
    d16, codes = O.unpack_blocks(O.unpack_matrix(q, n, 3).reshape(-1, 42))
    d = O.fp16_bits_to_f32(d16).reshape(n, 3)
    codes = codes.reshape(n, 3, 64)
    for b in range(3):
        x = np.zeros(k, dtype=np.float32)
        x[256 * b: 256 * (b + 1)] = 1.0
        y = O.gemv(q, n, k, x)
        for r in range(n):
            # count signs straight from the enumeration of one-zero patterns
            pos = neg = 0
            for c in codes[r, b]:
                z, m = int(c) >> 3, int(c) & 7
                signs = [(m >> i) & 1 for i in range(3)]
                neg += sum(signs)
                pos += 3 - sum(signs)
            assert y[r] == float(d[r, b]) * (pos - neg)


def test_gemv_matches_exact_fsum():
    n, k = 5, 1024
    q = _small_packed(6, n, k)
    x = np.random.default_rng(7).normal(0, 1, size=k).astype(np.float32)
    w_hat = O.dequantize_rows(q, n, k)
    y = O.gemv(q, n, k, x)
    A = O.tolerance_scale(q, n, k, x)[0]
    for r in range(n):
        exact = math.fsum(float(w_hat[r, i]) * float(x[i]) for i in range(k))
        assert abs(y[r] - exact) <= 1e-13 * A[r]


def test_tolerance_scale_closed_form():
    n, k = 3, 512
    q = _small_packed(10, n, k)
    x = np.ones(k, dtype=np.float32)
    d16, _ = O.unpack_blocks(O.unpack_matrix(q, n, 2).reshape(-1, 42))
    d = O.fp16_bits_to_f32(d16).reshape(n, 2).astype(np.float64)
    A = O.tolerance_scale(q, n, k, x)[0]
    assert np.allclose(A, 256.0 * d.sum(axis=1), rtol=0, atol=0)


def test_tolerance_scale_signed_inputs_and_scales():
    """A = sum_b |d_b| sum_{k in b} |x_k| for signed x and scales of either sign.
    Pins: (1) A bounds |W_hat x| (triangle inequality) and does not depend on
    the signs of x; (2) for x = sign(w_hat_r) * m (m >= 0, so x vanishes on
    row r's zero lanes) every term of row r's dot product is |w_hat| m, and
    the exactly summed y_r equals A_r; (3) putting mass on a zero lane of row r
    raises A_r by |d| times that mass but leaves y_r unchanged."""
    n, k = 4, 512
    nb = k // 256
    blocks = O.unpack_matrix(_small_packed(10, n, k), n, nb).copy()
    d16, codes = O.unpack_blocks(blocks.reshape(-1, 42))
    d16 = d16.reshape(n, nb).copy()
    d16[1, 0] |= 0x8000                                    # negative scales
    d16[3, 1] |= 0x8000
    blocks = O.pack_blocks(d16.reshape(-1), codes).reshape(n, nb, 42)
    q = O.pack_matrix(blocks)
    w_hat = O.dequantize_rows(q, n, k).astype(np.float64)
    assert np.any(w_hat[1, :256] < 0) and np.any(w_hat[3, 256:] > 0)
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, k).astype(np.float32)
    A = O.tolerance_scale(q, n, k, x)[0]
    assert np.all(A >= np.abs(O.gemv(q, n, k, x)))
    flips = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
    np.testing.assert_array_equal(O.tolerance_scale(q, n, k, x * flips)[0], A)
    np.testing.assert_array_equal(O.tolerance_scale(q, n, k, -x)[0], A)
    m = np.abs(x).astype(np.float64)
    for r in range(n):
        xr = (np.sign(w_hat[r]) * m).astype(np.float32)   # exact: a sign times an fp32
        exact = math.fsum(float(w_hat[r, i]) * float(xr[i]) for i in range(k))
        assert O.tolerance_scale(q, n, k, xr)[0][r] == pytest.approx(exact, rel=1e-14)
        z = int(np.flatnonzero(w_hat[r] == 0)[0])          # a zero lane of row r
        xz = xr.copy()
        xz[z] = np.float32(-3.0)
        b = z // 256
        dz = abs(float(O.fp16_bits_to_f32(np.array([d16[r, b]], dtype=np.uint16))[0]))
        assert O.tolerance_scale(q, n, k, xz)[0][r] == pytest.approx(exact + 3.0 * dz, rel=1e-14)
        assert O.gemv(q, n, k, xz)[r] == pytest.approx(exact, rel=1e-14)


def test_grouped_gemm_matches_per_expert_gemv():
    n, k, E = 16, 512, 4
    rb = O.row_bytes(k)
    stride = n * rb + 64                                  # padded stride is allowed
    table = np.zeros(E * stride, dtype=np.uint8)
    for e in range(E):
        table[e * stride: e * stride + n * rb] = _small_packed(20 + e, n, k).reshape(-1)
    offsets = np.array([0, 3, 3, 4, 9], dtype=np.int32)   # expert 1 has no rows
    xb, x = S.bf16_normal(np.random.default_rng(1), (9, k))
    y = O.grouped_gemm(table, stride, n, k, x, offsets)
    for e in range(E):
        raw = table[e * stride: e * stride + n * rb]
        for r in range(offsets[e], offsets[e + 1]):
            assert np.allclose(y[r], O.gemv(raw, n, k, x[r]), rtol=1e-14, atol=1e-14)
