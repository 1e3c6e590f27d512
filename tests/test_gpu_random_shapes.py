"""Seeded random-shape parity of the GPU path against the oracle.

Each case draws its own shapes and inputs from a fixed seed: ragged row
counts and k, several experts with skewed token counts (so experts are
parted and passes split), invalid expert and token ids, fp32 or bf16
activations across a range of magnitudes, packed matrices with scales of
either sign (zero and subnormal ones included) and, for the GEMV, a forced
(k splits, part cap) plan or the planner's own.  The bounds are the ones the
hand-picked cases use: |y - y_ref| <= 1e-3 * A per element for the GEMV,
2e-3 * A plus 2e-3 normwise for the bf16-MFMA grouped GEMM, the derived
per-element bound for the FFN, and bit-exactness for the encoder."""
import numpy as np
import pytest
import torch

from oracle import stq_oracle as O
import synth_inputs as S

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-3
GEMM_TOL = 2e-3


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


def packed_rows(rng, n_rows, nb, exp_lo=8, exp_hi=22):
    """Valid packed rows: uniform codes; fp16 scales of random sign with
    exponent fields in [exp_lo, exp_hi), 2 % zero and 2 % subnormal."""
    m = n_rows * nb
    codes = rng.integers(0, 32, size=(m, 64)).astype(np.uint8)
    exp = rng.integers(exp_lo, exp_hi, size=m)
    man = rng.integers(0, 1024, size=m)
    sign = rng.integers(0, 2, size=m)
    d16 = ((sign << 15) | (exp << 10) | man).astype(np.uint16)
    d16[rng.random(m) < 0.02] = 0
    sub = rng.random(m) < 0.02
    d16[sub] &= 0x83FF
    return O.pack_matrix(O.pack_blocks(d16, codes).reshape(n_rows, nb, O.BLOCK_BYTES)).reshape(-1)


def activations(rng, shape):
    """bf16 activations N(0, 1) times a power of two in [2^-6, 2^6]: (bits, fp32 values)."""
    scale = 2.0 ** int(rng.integers(-6, 7))
    bits = S.f32_to_bf16_bits((rng.normal(0.0, 1.0, size=shape) * scale).astype(np.float32))
    return bits, S.bf16_bits_to_f32(bits)


def table_of(mats, n_bytes, pad):
    stride = (n_bytes + 15) // 16 * 16 + 16 * pad
    t = np.zeros(len(mats) * stride, dtype=np.uint8)
    for e, m in enumerate(mats):
        t[e * stride: e * stride + n_bytes] = m
    return t, stride


@pytest.mark.parametrize("case", range(40))
def test_gemv_random_shapes(stq, monkeypatch, case):
    rng = np.random.default_rng(7100 + case)
    nb = int(rng.integers(1, 13))
    k = 256 * nb
    n = int(rng.integers(1, 70)) if rng.random() < 0.3 else int(rng.integers(64, 1300))
    n_experts, n_tokens = int(rng.integers(1, 11)), int(rng.integers(1, 11))
    rb = O.row_bytes(k)
    mats = [packed_rows(rng, n, nb) for _ in range(n_experts)]
    table, stride = table_of(mats, n * rb, int(rng.integers(0, 4)))
    bits, xf = activations(rng, (n_tokens, k))
    use_f32 = rng.random() < 0.4
    if rng.random() < 0.15:
        pe = pt = None  # every pair on expert 0, pair i on token i
        n_pairs = n_tokens
        pe_h, pt_h = np.zeros(n_pairs, dtype=np.int32), np.arange(n_pairs, dtype=np.int32)
    else:
        n_pairs = int(rng.integers(1, 49))
        hot = rng.integers(0, n_experts, size=max(1, n_experts // 2))
        pe_h = np.where(rng.random(n_pairs) < 0.6, rng.choice(hot, n_pairs),
                        rng.integers(0, n_experts, n_pairs)).astype(np.int32)
        pt_h = rng.integers(0, n_tokens, n_pairs).astype(np.int32)
        bad_e = rng.random(n_pairs) < 0.08
        pe_h[bad_e] = rng.choice([-1, n_experts, n_experts + 5], int(bad_e.sum()))
        bad_t = rng.random(n_pairs) < 0.05
        pt_h[bad_t] = rng.choice([-1, n_tokens], int(bad_t.sum()))
        pe, pt = dev(pe_h), dev(pt_h)
    plan = None if rng.random() < 0.4 else f"{int(rng.integers(1, nb + 1))},{int(rng.integers(1, 9))}"
    if plan:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    else:
        monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    xt = dev(xf) if use_f32 else dev(bits.view(np.int16)).view(torch.bfloat16)
    what = f"case {case}: n={n} k={k} experts={n_experts} tokens={n_tokens} pairs={n_pairs} plan={plan} f32={use_f32}"

    y = host(stq.gemv(dev(table), stride, n_experts, n, k, xt, pe, pt, n_pairs=n_pairs))
    valid = (pe_h >= 0) & (pe_h < n_experts) & (pt_h >= 0) & (pt_h < n_tokens)
    assert np.all(np.isnan(y[~valid])), what
    for e in np.unique(pe_h[valid]):
        idx = np.nonzero(valid & (pe_h == e))[0]
        raw = table[e * stride: e * stride + n * rb]
        xs = xf[pt_h[idx]]
        y_ref = O.gemv_tokens(raw, n, k, xs)
        A = O.tolerance_scale(raw, n, k, xs)
        err = np.abs(y[idx].astype(np.float64) - y_ref)
        assert np.all(err <= GEMV_TOL * A), f"{what}: expert {e}, worst {np.max(err / np.maximum(A, 1e-300))}"
    y2 = host(stq.gemv(dev(table), stride, n_experts, n, k, xt, pe, pt, n_pairs=n_pairs))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), what


@pytest.mark.parametrize("case", range(16))
def test_grouped_gemm_random_shapes(stq, case):
    rng = np.random.default_rng(7300 + case)
    nb = int(rng.integers(1, 9))
    k = 256 * nb
    n = int(rng.integers(1, 700))
    n_experts = int(rng.integers(1, 7))
    counts = np.array([int(rng.choice([0, 1, int(rng.integers(2, 16)), int(rng.integers(16, 81)),
                                       int(rng.integers(81, 200))])) for _ in range(n_experts)])
    if counts.sum() == 0:
        counts[-1] = int(rng.integers(1, 40))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rb = O.row_bytes(k)
    mats = [packed_rows(rng, n, nb, 10, 20) for _ in range(n_experts)]
    table, stride = table_of(mats, n * rb, int(rng.integers(0, 3)))
    bits, xf = activations(rng, (int(offsets[-1]), k))
    what = f"case {case}: n={n} k={k} counts={counts.tolist()}"

    y = host(stq.grouped_gemm(dev(table), stride, n_experts, n, k,
                              dev(bits.view(np.int16)).view(torch.bfloat16), dev(offsets)))
    y_ref = O.grouped_gemm(table, stride, n, k, xf, offsets)
    for e in range(n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        raw = table[e * stride: e * stride + n * rb]
        A = O.tolerance_scale(raw, n, k, xf[lo:hi])
        err = np.abs(y[lo:hi].astype(np.float64) - y_ref[lo:hi])
        assert np.all(err <= GEMM_TOL * A), f"{what}: expert {e}"
        assert np.max(err) <= GEMM_TOL * max(np.max(np.abs(y_ref[lo:hi])), 1e-300), f"{what}: expert {e} normwise"


@pytest.mark.parametrize("case", range(12))
def test_moe_ffn_random_shapes(stq, monkeypatch, case):
    rng = np.random.default_rng(7500 + case)
    n_experts = int(rng.integers(1, 7))
    d_model, d_ff = 256 * int(rng.integers(1, 4)), 256 * int(rng.integers(1, 4))
    n_tokens = int(rng.integers(1, 7))
    top_k = int(rng.integers(1, min(n_experts, 4) + 1))
    gu = {e: packed_rows(rng, 2 * d_ff, d_model // 256, 10, 16) for e in range(n_experts)}
    dn = {e: packed_rows(rng, d_model, d_ff // 256, 10, 16) for e in range(n_experts)}
    tg, sg = table_of([gu[e] for e in range(n_experts)], 2 * d_ff * O.row_bytes(d_model), int(rng.integers(0, 3)))
    td, sd = table_of([dn[e] for e in range(n_experts)], d_model * O.row_bytes(d_ff), int(rng.integers(0, 3)))
    pe = np.concatenate([rng.choice(n_experts, top_k, replace=False) for _ in range(n_tokens)]).astype(np.int32)
    bad = rng.random(pe.size) < 0.1
    pe[bad] = rng.choice([-1, n_experts], int(bad.sum()))
    pw = S.routing_weights(7600 + case, n_tokens, top_k)
    bits, xf = activations(rng, (n_tokens, d_model))
    plan = None if rng.random() < 0.5 else f"{int(rng.integers(1, 4))},{int(rng.integers(1, 5))}"
    if plan:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    else:
        monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    what = f"case {case}: experts={n_experts} d_model={d_model} d_ff={d_ff} tokens={n_tokens} top_k={top_k} plan={plan}"

    y = stq.moe_ffn_decode(dev(tg), sg, dev(td), sd, n_experts, d_model, d_ff,
                           dev(bits.view(np.int16)).view(torch.bfloat16), dev(pe), dev(pw), top_k)
    y = host(y).astype(np.float64)
    ref = O.moe_ffn_decode(gu, dn, d_model, d_ff, xf, pe, pw, top_k)
    bound = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, xf, pe, pw, top_k)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan), what
    err = np.abs(y[~nan] - ref[~nan])
    assert np.all(err <= bound[~nan]), f"{what}: worst {np.max(err / np.maximum(bound[~nan], 1e-300))}"


@pytest.mark.parametrize("case", range(12))
def test_quantize_random_shapes_bit_exact(stq, case):
    rng = np.random.default_rng(7700 + case)
    n_rows, k = int(rng.integers(1, 40)), 256 * int(rng.integers(1, 9))
    w = (rng.normal(0.0, 1.0, size=(n_rows, k)) * 10.0 ** rng.uniform(-4, 2)).astype(np.float32)
    w[rng.random(w.shape) < 0.05] = 0.0
    if n_rows > 2:
        w[1] = 0.0
    im = None
    if rng.random() < 0.7:
        im = (rng.gamma(0.5, 1.0, size=k) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
        im[rng.random(k) < 0.05] = 0.0
        im[rng.random(k) < 0.02] *= 1000.0
    encoder = "amax" if rng.random() < 0.3 else "wls"
    rounds = int(rng.integers(0, 6))
    q = host(stq.quantize_rows(dev(w), None if im is None else dev(im),
                               stq.ENC_AMAX if encoder == "amax" else stq.ENC_WLS, rounds))
    ref = O.quantize_rows(w, im, encoder, rounds)
    assert np.array_equal(q.reshape(-1), ref.reshape(-1)), \
        f"case {case}: rows={n_rows} k={k} encoder={encoder} rounds={rounds} imatrix={im is not None}"
