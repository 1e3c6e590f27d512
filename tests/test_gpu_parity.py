"""GPU parity: every HIP entry point against the CPU oracle, through the C ABI.

Packing, decoding and pattern choice are compared bit for bit.  GEMV results
must satisfy |y - y_ref| <= 1e-3 * A and grouped-GEMM results
|y - y_ref| <= 2e-3 * A elementwise (A = sum over blocks of d * sum|x|) plus a
per-expert normwise 2e-3; inputs whose exact result is representable (unit
vectors, block indicators) must match exactly.  Full-size cases run the
shapes the benchmark times and check sampled outputs one by one.
"""
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


def random_blocks(rng, n_rows, nb):
    """Random valid packed rows: random codes, finite fp16 scales of any sign (incl. +-0, subnormal)."""
    codes = rng.integers(0, 32, size=(n_rows * nb, 64)).astype(np.uint8)
    exp = rng.integers(0, 31, size=n_rows * nb)
    man = rng.integers(0, 1024, size=n_rows * nb)
    sign = rng.integers(0, 2, size=n_rows * nb)
    d16 = ((sign << 15) | (exp << 10) | man).astype(np.uint16)
    return O.pack_matrix(O.pack_blocks(d16, codes).reshape(n_rows, nb, 42))


def check_close(y, y_ref, A, tol, what=""):
    err = np.abs(np.asarray(y, dtype=np.float64) - y_ref)
    bad = err > tol * A
    assert not bad.any(), f"{what}: {bad.sum()} outputs out of tolerance, worst ratio {np.max(err / np.maximum(A, 1e-300))}"
    return float(np.max(err / np.maximum(A, 1e-300))) if err.size else 0.0


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_rows,k", [(1, 256), (3, 768), (37, 1024), (5, 7168), (130, 512)])
def test_dequantize_bit_exact(stq, n_rows, k):
    rng = np.random.default_rng(n_rows * 1000 + k)
    raw = random_blocks(rng, n_rows, k // 256)
    got = host(stq.dequantize_rows(dev(raw), n_rows, k))
    want = O.dequantize_rows(raw, n_rows, k)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# encode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("encoder,rounds", [("wls", 3), ("wls", 0), ("wls", 1), ("wls", 5), ("amax", 3)])
def test_quantize_bit_exact_small_case(stq, encoder, rounds):
    w, q, _ = S.single_gemv_case()
    enc = stq.ENC_WLS if encoder == "wls" else stq.ENC_AMAX
    got = host(stq.quantize_rows(dev(w), dev(q), encoder=enc, rounds=rounds))
    want = O.quantize_rows(w, q, encoder=encoder, rounds=rounds)
    assert np.array_equal(got, want)


def _weight_cases():
    rng = np.random.default_rng(42)
    yield "t3 heavy tails", (rng.standard_t(3, size=(7, 512)) * 0.02).astype(np.float32), True
    yield "tiny (subnormal fp16 d)", (rng.normal(0, 1e-6, size=(3, 256))).astype(np.float32), True
    yield "huge (clamped d)", (rng.normal(0, 1e5, size=(2, 768))).astype(np.float32), True
    z = np.zeros((4, 512), dtype=np.float32)
    z[1] = -0.0
    z[2] = 0.375
    z[3, ::3] = -1.5
    yield "zeros, constants, sparse", z, False
    yield "ragged rows, no imatrix", rng.normal(0, 0.02, size=(129, 256)).astype(np.float32), False
    yield "k=1792", rng.normal(0, 0.02, size=(9, 1792)).astype(np.float32), True
    ties = np.repeat(rng.normal(0, 0.02, size=(2, 256 // 2)).astype(np.float32), 2, axis=1)
    yield "pairwise ties", ties, True


@pytest.mark.parametrize("case", list(range(7)))
@pytest.mark.parametrize("encoder", ["wls", "amax"])
def test_quantize_bit_exact_varied(stq, case, encoder):
    name, w, use_q = list(_weight_cases())[case]
    rng = np.random.default_rng(case)
    q = None
    if use_q:
        q = (rng.chisquare(1, size=w.shape[1]) + 1e-3).astype(np.float32)
        q[rng.integers(0, w.shape[1], size=5)] = 0.0
    enc = stq.ENC_WLS if encoder == "wls" else stq.ENC_AMAX
    got = host(stq.quantize_rows(dev(w), None if q is None else dev(q), encoder=enc, rounds=3))
    want = O.quantize_rows(w, q, encoder=encoder, rounds=3)
    assert np.array_equal(got, want), name


@pytest.mark.parametrize("rounds", [0, 1, 3, 5])
def test_quantize_bit_exact_heavy_tailed_imatrix(stq, rounds):
    """Outlier-channel importance, where the rounds move many zeros away from
    the smallest |w|: still byte-identical to the oracle."""
    w = S.gaussian_weights(0, 256, 1024)
    q = S.heavy_tailed_imatrix(1, 64, 1024)
    got = host(stq.quantize_rows(dev(w), dev(q), encoder=stq.ENC_WLS, rounds=rounds))
    assert np.array_equal(got, O.quantize_rows(w, q, rounds=rounds))


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------
def test_gemv_small_case_fp32(stq):
    w, q, x = S.single_gemv_case()
    packed = O.quantize_rows(w, q)
    y = host(stq.gemv(dev(packed), packed.nbytes, 1, 256, 1024, dev(x[None, :])))[0]
    y_ref = O.gemv(packed, 256, 1024, x)
    A = O.tolerance_scale(packed, 256, 1024, x)[0]
    check_close(y, y_ref, A, GEMV_TOL, "small case")
    # the GPU encoder's bytes give the same product
    packed_gpu = stq.quantize_rows(dev(w), dev(q))
    y2 = host(stq.gemv(packed_gpu, packed.nbytes, 1, 256, 1024, dev(x[None, :])))[0]
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("k", [768, 1024])
@pytest.mark.parametrize("xdtype", ["f32", "bf16"])
def test_gemv_exact_special_inputs(stq, k, xdtype):
    n = 96
    rng = np.random.default_rng(k)
    raw = random_blocks(rng, n, k // 256)
    raw16 = raw.reshape(-1, 42)
    raw16[:, 1] &= 0x7F                                   # keep d >= 0 finite (any sign works, this keeps it simple)
    w_hat = O.dequantize_rows(raw, n, k)
    cols = [0, 5, 255, 256, k - 1]
    xs = np.zeros((len(cols) + k // 256, k), dtype=np.float32)
    for i, c in enumerate(cols):
        xs[i, c] = 1.0
    for b in range(k // 256):
        xs[len(cols) + b, 256 * b: 256 * (b + 1)] = 1.0
    xt = dev(xs) if xdtype == "f32" else dev(xs).to(torch.bfloat16)
    y = host(stq.gemv(dev(raw), raw.nbytes, 1, n, k, xt, pair_expert=None,
                      pair_token=dev(np.arange(len(xs), dtype=np.int32))))
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], w_hat[:, c]), c          # exact (a signed zero may differ)
    y_ref = w_hat.astype(np.float64) @ xs.astype(np.float64).T
    assert np.array_equal(y[len(cols):], y_ref.T[len(cols):].astype(np.float32))


def _pair_case(rng, n_experts, n_tokens):
    pe = [2, 0, 2, 5, 2, 2, 1, 2, 2, -1, 6, 3, 0]
    pt = [0, 1, 2, 3, 4, 5, 6, 7, 8, 0, 1, n_tokens, 2]
    return np.array(pe, dtype=np.int32), np.array(pt, dtype=np.int32)


@pytest.mark.parametrize("k,n", [(256, 300), (768, 257), (1024, 300), (2048, 513)])
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_gemv_pairs_against_oracle(stq, k, n, xdtype):
    rng = np.random.default_rng(k + n)
    n_experts, n_tokens = 6, 9
    rb = O.row_bytes(k)
    stride = (n * rb + 15) // 16 * 16 + 32
    table = np.zeros(n_experts * stride, dtype=np.uint8)
    for e in range(n_experts):
        w = S.gaussian_weights(100 + e, n, k)
        table[e * stride: e * stride + n * rb] = O.quantize_rows(w, None).reshape(-1)
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    x = xf  # bf16-representable values either way; the dtype picks the kernel's load path
    xt = dev(x) if xdtype == "f32" else dev(xb.view(np.int16)).view(torch.bfloat16)
    pe, pt = _pair_case(rng, n_experts, n_tokens)
    y = host(stq.gemv(dev(table), stride, n_experts, n, k, xt, dev(pe), dev(pt)))
    for i, (e, t) in enumerate(zip(pe, pt)):
        if not (0 <= e < n_experts and 0 <= t < n_tokens):
            assert np.all(np.isnan(y[i])), i
            continue
        raw = table[e * stride: e * stride + n * rb]
        y_ref = O.gemv(raw, n, k, x[t])
        A = O.tolerance_scale(raw, n, k, x[t])[0]
        check_close(y[i], y_ref, A, GEMV_TOL, f"pair {i}")
    # repeat calls give identical bits (fixed summation order, including the k split)
    y2 = host(stq.gemv(dev(table), stride, n_experts, n, k, xt, dev(pe), dev(pt)))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_gemv_many_pairs_one_expert(stq):
    """More tokens on one expert than one pass holds; null expert list = expert 0."""
    rng = np.random.default_rng(9)
    n, k, n_tokens = 256, 1024, 11
    w = S.gaussian_weights(7, n, k)
    raw = O.quantize_rows(w, None)
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    xt = dev(xb.view(np.int16)).view(torch.bfloat16)
    y = host(stq.gemv(dev(raw), raw.nbytes, 1, n, k, xt))
    y_ref = O.gemv_tokens(raw, n, k, xf)
    for t in range(n_tokens):
        A = O.tolerance_scale(raw, n, k, xf[t])[0]
        check_close(y[t], y_ref[t], A, GEMV_TOL, f"token {t}")


@pytest.mark.parametrize("plan", [None, "1,1", "3,2"])
def test_gemv_matrix_core_passes_of_5_to_16_tokens(stq, monkeypatch, plan):
    """bf16 activations with at least as many pairs as experts take the
    matrix-core kernel: experts with 5-8 tokens run one pass of two token
    sets, 12 and 16 tokens two passes (8 + 4, 8 + 8), next to experts with
    1-3 tokens on the tables; ragged n (not a multiple of 64), several
    blocks, pairs interleaved across experts.  Every output element within
    1e-3 * A of the oracle."""
    if plan:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    else:
        monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    rng = np.random.default_rng(64)
    counts = [5, 6, 7, 8, 12, 16, 1, 2, 3]
    n_experts, n, k, n_tokens = len(counts), 200, 1536, 16
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(1100 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    pe = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    pt = np.concatenate([rng.choice(n_tokens, c, replace=False) for c in counts]).astype(np.int32)
    perm = rng.permutation(pe.size)
    pe, pt = pe[perm], pt[perm]
    assert pe.size >= n_experts
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                      dev(pe), dev(pt)))
    for i in range(pe.size):
        raw = table[int(pe[i]) * n * rb:(int(pe[i]) + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[pt[i]]), O.tolerance_scale(raw, n, k, xf[pt[i]])[0],
                    GEMV_TOL, f"plan {plan} pair {i} (expert {int(pe[i])}, {counts[int(pe[i])]} tokens)")


@pytest.mark.parametrize("plan", [None, "4,1", "3,3"])
def test_gemv_single_pair_valid_and_invalid(stq, monkeypatch, plan):
    """One (token, expert) pair takes the single-pair path (no unit search):
    a valid pair matches the oracle under planned, split and split-and-parted
    plans; an unknown expert or token gives a row of NaN."""
    if plan:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    else:
        monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    n_experts, n, k, n_tokens = 3, 136, 1280, 4
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(1300 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    xb, xf = S.bf16_normal(np.random.default_rng(65), (n_tokens, k))
    xt = dev(xb.view(np.int16)).view(torch.bfloat16)
    for e, t in [(2, 3), (0, 0), (3, 1), (-1, 1), (1, 4), (1, -1)]:
        pe = dev(np.array([e], dtype=np.int32))
        pt = dev(np.array([t], dtype=np.int32))
        y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, xt, pe, pt))
        if 0 <= e < n_experts and 0 <= t < n_tokens:
            raw = table[e * n * rb:(e + 1) * n * rb]
            check_close(y[0], O.gemv(raw, n, k, xf[t]), O.tolerance_scale(raw, n, k, xf[t])[0], GEMV_TOL,
                        f"plan {plan} expert {e} token {t}")
        else:
            assert np.all(np.isnan(y[0])), (plan, e, t)


@pytest.mark.parametrize("xdtype,plan", [("bf16", None), ("bf16", "1,3"), ("f32", None), ("f32", "2,2")])
def test_gemv_units_numbered_by_cost_class(stq, monkeypatch, xdtype, plan):
    """More workgroups than the CUs keep resident (300 pairs x 4 row tiles):
    the device numbers units by cost class (experts with 5+, 3-4, 2, 1
    tokens, then parted experts).  Experts with 1-9 tokens, invalid ids and
    pairs in random order; every pair within 1e-3 * A of the oracle, invalid
    pairs NaN, and a repeat call bit-equal."""
    if plan:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    else:
        monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    rng = np.random.default_rng(66)
    n_experts, n, k, n_tokens = 60, 2048, 512, 24
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(1400 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    counts = rng.integers(1, 10, size=n_experts)
    counts = counts * (rng.random(n_experts) < 0.8)           # some experts idle
    pe = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    pt = np.concatenate([rng.choice(n_tokens, c, replace=False) for c in counts]).astype(np.int32)
    pe = np.concatenate([pe, np.array([n_experts, -1, 3], np.int32)])
    pt = np.concatenate([pt, np.array([0, 1, n_tokens], np.int32)])
    perm = rng.permutation(pe.size)
    pe, pt = pe[perm], pt[perm]
    assert 200 <= pe.size <= 512
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    x = dev(xb.view(np.int16)).view(torch.bfloat16) if xdtype == "bf16" else dev(xf)
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, x, dev(pe), dev(pt)))
    for i in range(pe.size):
        e, t = int(pe[i]), int(pt[i])
        if not (0 <= e < n_experts and 0 <= t < n_tokens):
            assert np.all(np.isnan(y[i])), i
            continue
        raw = table[e * n * rb:(e + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[t]), O.tolerance_scale(raw, n, k, xf[t])[0], GEMV_TOL,
                    f"{xdtype} plan {plan} pair {i} (expert {e}, {counts[e]} tokens)")
    y2 = host(stq.gemv(dev(table), n * rb, n_experts, n, k, x, dev(pe), dev(pt)))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_gemv_wide_batch(stq):
    """512 pairs over 16 experts: shared and distinct experts mixed."""
    n_experts, n, k, n_tokens = 16, 256, 1024, 64
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(300 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    pe, pt = S.uniform_topk_pairs(5, n_tokens, n_experts, 8)
    xb, xf = S.bf16_normal(np.random.default_rng(1), (n_tokens, k))
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                      dev(pe), dev(pt)))
    for i in range(0, len(pe), 7):
        raw = table[pe[i] * n * rb:(pe[i] + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[pt[i]]), O.tolerance_scale(raw, n, k, xf[pt[i]])[0],
                    GEMV_TOL, f"pair {i}")


def test_gemv_plan_uses_the_device_cu_count(stq, monkeypatch):
    """stq_gemv_plan with n_cus = 0 plans for the current device's compute
    units, as stq_gemv does."""
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for n_pairs in (1, 8, 32, 128, 512):
        assert stq.gemv_plan(256, 4096, 7168, n_pairs) == stq.gemv_plan(256, 4096, 7168, n_pairs, n_cus=cus)


@pytest.mark.parametrize("plan", [None, "1,2", "1,8", "2,3", "3,4", "5,8", "10,1"])
def test_gemv_token_parts_match_oracle(stq, monkeypatch, plan):
    """Experts with 0-8 tokens under forced (k splits, part cap) plans: an
    expert with m tokens has each split's blocks parted min(m, cap) ways and
    the parts' partial sums added in k order.  k = 2560 (10 blocks), so
    "3,4" (splits of 4, 4, 2 blocks) and "5,8" (2 blocks a split) leave
    some parts empty; pairs shuffled, one invalid."""
    if plan is not None:
        monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    rng = np.random.default_rng(61)
    counts = [1, 2, 3, 4, 5, 8, 0]
    n_experts, n, k, n_tokens = len(counts), 192, 2560, 12
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(800 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    pe = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)] + [np.array([n_experts], np.int32)])
    pt = np.concatenate([rng.choice(n_tokens, c, replace=False) for c in counts] + [np.array([0])]).astype(np.int32)
    perm = rng.permutation(pe.size)
    pe, pt = pe[perm], pt[perm]
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                      dev(pe), dev(pt)))
    for i, (e, t) in enumerate(zip(pe, pt)):
        if e >= n_experts:
            assert np.all(np.isnan(y[i])), i
            continue
        raw = table[e * n * rb:(e + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[t]), O.tolerance_scale(raw, n, k, xf[t])[0], GEMV_TOL,
                    f"plan {plan} pair {i} (expert {e})")


def _pass_sizes(pe, per_pass):
    """Tokens in the pass that serves each pair: an expert's pairs are taken in
    pair order, per_pass to a pass."""
    size = np.zeros(pe.size, dtype=int)
    for e in np.unique(pe):
        idx = np.flatnonzero(pe == e)
        for c in range(0, idx.size, per_pass):
            size[idx[c:c + per_pass]] = min(per_pass, idx.size - c)
    return size


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("plan", ["1,1", "3,1"])
def test_gemv_pair_result_does_not_depend_on_its_companions(stq, monkeypatch, plan, xdt):
    """Under a plan that does not part experts by token count, a pair's output
    does not depend on the other pairs batched with it, as long as its pass
    runs on the same form.  Experts hold 1-8, 10 and 11 tokens.  Table
    passes take up to 4 tokens, matrix-core passes up to 8.  Passes of 1-2
    tokens run on the tables (two-token tables have the sums and per-token
    order of adds of one-token tables), so such a pair equals the pair
    computed alone (a one-token pass) bit for bit; fp32 activations always
    take the tables, in passes of up to 4.  In the bf16 call (as many pairs
    as experts or more, so the matrix-core kernel variant) passes of 3-8
    tokens run on the matrix cores, where a token's results use only its own
    activations and every set of four tokens runs the same instructions:
    such a pair equals the same pair in a second call with the pairs in
    another order (other companions), bit for bit, where it again sits in a
    pass of 3-8 tokens."""
    monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    rng = np.random.default_rng(63)
    counts = [1, 2, 3, 4, 5, 6, 7, 8, 10, 11]
    n_experts, n, k, n_tokens = len(counts), 320, 2560, 12
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(900 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    pe = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    pt = np.concatenate([rng.choice(n_tokens, c, replace=False) for c in counts]).astype(np.int32)
    perm = rng.permutation(pe.size)
    pe, pt = pe[perm], pt[perm]
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    x = dev(xb.view(np.int16)).view(torch.bfloat16) if xdt == "bf16" else dev(xf)
    wt = dev(table)
    y = host(stq.gemv(wt, n * rb, n_experts, n, k, x, dev(pe), dev(pt)))
    per_pass = 8 if xdt == "bf16" else 4
    size = _pass_sizes(pe, per_pass)
    matrix = (size >= 3) if xdt == "bf16" else np.zeros(pe.size, bool)
    for i in np.flatnonzero(~matrix):
        yi = host(stq.gemv(wt, n * rb, n_experts, n, k, x, dev(pe[i:i + 1]), dev(pt[i:i + 1])))
        assert np.array_equal(yi[0].view(np.uint32), y[i].view(np.uint32)), (i, int(pe[i]))
    if matrix.any():
        order = rng.permutation(pe.size)
        y2 = host(stq.gemv(wt, n * rb, n_experts, n, k, x, dev(pe[order]), dev(pt[order])))
        size2 = _pass_sizes(pe[order], per_pass)
        checked = 0
        for j, i in enumerate(order):
            if matrix[i] and size2[j] >= 3:
                assert np.array_equal(y2[j].view(np.uint32), y[i].view(np.uint32)), (i, int(pe[i]))
                checked += 1
        assert checked >= 8
    # every pair within the tolerance of the oracle
    for i in range(pe.size):
        raw = table[int(pe[i]) * n * rb:(int(pe[i]) + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[pt[i]]), O.tolerance_scale(raw, n, k, xf[pt[i]])[0], GEMV_TOL, str(i))


@pytest.mark.parametrize("per_expert", [2, 3, 4, 9])
def test_gemv_pairs_grouped_by_expert(stq, per_expert):
    """Pairs sorted by expert (every expert's pairs adjacent) with invalid
    pairs mixed in: each pair still gets its own expert's product, invalid
    ones NaN.  (Workgroups serve leading pairs by rank, whatever the pair
    order.)"""
    rng = np.random.default_rng(40 + per_expert)
    n_experts, n, k, n_tokens = 12, 256, 512, 16
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(500 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    pe = np.repeat(np.arange(n_experts, dtype=np.int32), per_expert)
    pt = rng.integers(0, n_tokens, pe.size).astype(np.int32)
    pe[5] = n_experts + 3          # invalid expert
    pt[-2] = -1                    # invalid token
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                      dev(pe), dev(pt)))
    for i, (e, t) in enumerate(zip(pe, pt)):
        if not (0 <= e < n_experts and 0 <= t < n_tokens):
            assert np.all(np.isnan(y[i])), i
            continue
        raw = table[e * n * rb:(e + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[t]), O.tolerance_scale(raw, n, k, xf[t])[0], GEMV_TOL, f"pair {i}")


@pytest.mark.parametrize("order", ["token_major", "sorted_by_expert"])
def test_gemv_pairs_beyond_one_scan_chunk(stq, order):
    """1500 pairs (three 512-pair chunks of the on-device leader ranking and
    pair gathering) over 40 experts, several passes per expert, in token
    order and sorted by expert; every pair against the oracle."""
    n_experts, n, k, n_tokens = 40, 128, 512, 300
    rb = O.row_bytes(k)
    table = np.concatenate([O.quantize_rows(S.gaussian_weights(700 + e, n, k), None).reshape(-1)
                            for e in range(n_experts)])
    rng = np.random.default_rng(77)
    pe = np.concatenate([rng.choice(n_experts, 5, replace=False) for _ in range(n_tokens)]).astype(np.int32)
    pt = np.repeat(np.arange(n_tokens, dtype=np.int32), 5)
    if order == "sorted_by_expert":
        perm = np.argsort(pe, kind="stable")
        pe, pt = pe[perm], pt[perm]
    xb, xf = S.bf16_normal(rng, (n_tokens, k))
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                      dev(pe), dev(pt)))
    for i in range(len(pe)):
        raw = table[pe[i] * n * rb:(pe[i] + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[pt[i]]), O.tolerance_scale(raw, n, k, xf[pt[i]])[0],
                    GEMV_TOL, f"pair {i}")


def test_gemv_more_experts_than_the_lds_leader_table(stq):
    """20000 experts (beyond what the in-LDS first-pair table holds): the
    per-pair leader scan serves them; shared, invalid and far experts."""
    n_experts, n, k, n_tokens = 20000, 64, 256, 5
    rb = O.row_bytes(k)
    used = {0: 1, 7: 2, 19999: 3, 12345: 4}
    table = np.zeros(n_experts * n * rb, dtype=np.uint8)
    for e, seed in used.items():
        table[e * n * rb:(e + 1) * n * rb] = O.quantize_rows(S.gaussian_weights(600 + seed, n, k), None).reshape(-1)
    pe = np.array([7, 19999, 7, 0, 12345, 20000, 19999, 7], dtype=np.int32)
    pt = np.array([0, 1, 2, 3, 4, 0, 0, 1], dtype=np.int32)
    xb, xf = S.bf16_normal(np.random.default_rng(8), (n_tokens, k))
    y = host(stq.gemv(dev(table), n * rb, n_experts, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                      dev(pe), dev(pt)))
    for i, (e, t) in enumerate(zip(pe, pt)):
        if e >= n_experts:
            assert np.all(np.isnan(y[i])), i
            continue
        raw = table[e * n * rb:(e + 1) * n * rb]
        check_close(y[i], O.gemv(raw, n, k, xf[t]), O.tolerance_scale(raw, n, k, xf[t])[0], GEMV_TOL, f"pair {i}")


# ---------------------------------------------------------------------------
# grouped GEMM
# ---------------------------------------------------------------------------
def _grouped_case(k, n, offsets, seed):
    n_experts = len(offsets) - 1
    rb = O.row_bytes(k)
    stride = (n * rb + 15) // 16 * 16
    table = np.zeros(n_experts * stride, dtype=np.uint8)
    for e in range(n_experts):
        table[e * stride: e * stride + n * rb] = O.quantize_rows(S.gaussian_weights(seed + e, n, k), None).reshape(-1)
    return table, stride


def _check_grouped(y, table, stride, n, k, xf, offsets, tol=GEMM_TOL):
    y_ref = O.grouped_gemm(table, stride, n, k, xf, offsets)
    rb = O.row_bytes(k)
    worst = 0.0
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        if hi <= lo:
            continue
        raw = table[e * stride: e * stride + n * rb]
        A = O.tolerance_scale(raw, n, k, xf[lo:hi])
        worst = max(worst, check_close(y[lo:hi], y_ref[lo:hi], A, tol, f"expert {e}"))
        nw = np.max(np.abs(y[lo:hi] - y_ref[lo:hi])) / max(np.max(np.abs(y_ref[lo:hi])), 1e-300)
        assert nw <= tol, (e, nw)
    return worst


@pytest.mark.parametrize("k,n", [(512, 200), (768, 128), (1024, 256)])
def test_grouped_gemm_against_oracle(stq, k, n):
    offsets = np.array([0, 3, 3, 140, 141, 150, 150], dtype=np.int32)   # M = 3, 0, 137 (two passes), 1, 9, 0
    table, stride = _grouped_case(k, n, offsets, 500)
    xb, xf = S.bf16_normal(np.random.default_rng(k), (int(offsets[-1]), k))
    y = host(stq.grouped_gemm(dev(table), stride, len(offsets) - 1, n, k,
                              dev(xb.view(np.int16)).view(torch.bfloat16), dev(offsets)))
    _check_grouped(y, table, stride, n, k, xf, offsets)


@pytest.mark.parametrize("k,n", [(256, 130), (16384, 72)])
def test_grouped_gemm_pass_boundaries(stq, k, n):
    """Token counts at and around the 16-token tile and the 80-token pass
    (16, 17, 80, 81, 200 = three passes), empty experts in between; n not a
    multiple of 4 or 64 (scalar stores, partial tiles); k of 1 and 64 blocks."""
    counts = [16, 0, 17, 80, 0, 81, 200, 1]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    table, stride = _grouped_case(k, n, offsets, 600)
    xb, xf = S.bf16_normal(np.random.default_rng(k + n), (int(offsets[-1]), k))
    y = host(stq.grouped_gemm(dev(table), stride, len(counts), n, k,
                              dev(xb.view(np.int16)).view(torch.bfloat16), dev(offsets)))
    _check_grouped(y, table, stride, n, k, xf, offsets)


def test_grouped_gemm_exact_special_inputs(stq):
    k, n = 768, 160
    rng = np.random.default_rng(3)
    raw = random_blocks(rng, n, k // 256)
    raw.reshape(-1, 42)[:, 1] &= 0x7F
    stride = (raw.nbytes + 15) // 16 * 16
    table = np.zeros(stride, dtype=np.uint8)
    table[:raw.nbytes] = raw.reshape(-1)
    cols = [0, 1, 300, 767]
    xs = np.zeros((len(cols) + 3, k), dtype=np.float32)
    for i, c in enumerate(cols):
        xs[i, c] = 1.0
    for b in range(3):
        xs[len(cols) + b, 256 * b: 256 * (b + 1)] = 1.0
    offsets = np.array([0, len(xs)], dtype=np.int32)
    y = host(stq.grouped_gemm(dev(table), stride, 1, n, k, dev(xs).to(torch.bfloat16), dev(offsets)))
    w_hat = O.dequantize_rows(raw, n, k)
    want = (w_hat.astype(np.float64) @ xs.astype(np.float64).T).T.astype(np.float32)
    assert np.array_equal(y, want)


def test_grouped_gemm_empty_and_single_rows(stq):
    k, n = 512, 64
    offsets = np.array([0, 0, 1, 1, 2, 2], dtype=np.int32)
    table, stride = _grouped_case(k, n, offsets, 900)
    xb, xf = S.bf16_normal(np.random.default_rng(0), (2, k))
    y = host(stq.grouped_gemm(dev(table), stride, 5, n, k, dev(xb.view(np.int16)).view(torch.bfloat16),
                              dev(offsets)))
    _check_grouped(y, table, stride, n, k, xf, offsets)
    # an M=1 expert equals the GEMV of that token
    raw = table[1 * stride: 1 * stride + n * O.row_bytes(k)]
    gv = host(stq.gemv(dev(raw), raw.nbytes, 1, n, k, dev(xf[:1])))[0]
    A = O.tolerance_scale(raw, n, k, xf[0])[0]
    assert np.all(np.abs(gv - y[0]) <= 2 * GEMM_TOL * A)


def test_grouped_gemm_offsets_outside_the_contract_stay_in_bounds(stq):
    """Offsets that are negative, decreasing or past total_m: each expert's
    rows are clamped to [0, total_m], so nothing is read past x_sorted and
    sentinel rows after y stay untouched; rows in one range match that
    expert, rows in two ranges match one of them."""
    k, n, total_m = 512, 96, 12
    offsets = np.array([-5, 4, 2, 50], dtype=np.int32)
    # clamped: expert 0 [0, 4); expert 1 lo = 4, hi = max(2, 4) = 4 (empty); expert 2 [2, 12)
    ranges = [(0, 4), (4, 4), (2, 12)]
    table, stride = _grouped_case(k, n, np.array([0, 1, 1, 1], dtype=np.int32), 950)
    xb, xf = S.bf16_normal(np.random.default_rng(11), (total_m, k))
    big = torch.full((total_m + 3, n), 7.0, dtype=torch.float32, device="cuda")
    out = big[:total_m]
    stq.grouped_gemm(dev(table), stride, 3, n, k, dev(xb.view(np.int16)).view(torch.bfloat16), dev(offsets),
                     out=out)
    yb = host(big)
    assert np.all(yb[total_m:] == 7.0)
    rb = O.row_bytes(k)
    refs = []
    for e in range(3):
        raw = table[e * stride: e * stride + n * rb]
        refs.append((O.gemv_tokens(raw, n, k, xf), O.tolerance_scale(raw, n, k, xf)))
    for r in range(total_m):
        owners = [e for e, (lo, hi) in enumerate(ranges) if lo <= r < hi]
        assert owners, r
        ok = [np.all(np.abs(yb[r] - refs[e][0][r]) <= GEMM_TOL * refs[e][1][r]) for e in owners]
        assert any(ok), (r, owners)


def test_binding_refuses_buffers_smaller_than_the_shapes(stq):
    """The binding checks every buffer the kernels index against the shapes
    before any launch: outputs, weight tables, activation rows, importance."""
    k, n, E = 256, 64, 3
    rb = O.row_bytes(k)
    table = torch.zeros(E * n * rb, dtype=torch.uint8, device="cuda")
    short = table[: (E - 1) * n * rb + n * rb - 1]
    x = torch.zeros((2, k), dtype=torch.bfloat16, device="cuda")
    pe = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="out"):
        stq.gemv(table, n * rb, E, n, k, x, pe, out=torch.empty((1, n), device="cuda"))
    with pytest.raises(ValueError, match="w_table"):
        stq.gemv(short, n * rb, E, n, k, x, pe)
    offs = torch.tensor([0, 1, 2, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="out"):
        stq.grouped_gemm(table, n * rb, E, n, k, x, offs, out=torch.empty((2, n - 1), device="cuda"))
    with pytest.raises(ValueError, match="w_table"):
        stq.grouped_gemm(short, n * rb, E, n, k, x, offs)
    with pytest.raises(ValueError, match="x_sorted"):
        stq.grouped_gemm(table, n * rb, E, n, k, torch.zeros((2, 2 * k), dtype=torch.bfloat16, device="cuda"), offs)
    with pytest.raises(ValueError, match="out"):
        stq.dequantize_rows(table, n, k, out=torch.empty((n, k - 1), device="cuda"))
    with pytest.raises(ValueError, match="imatrix"):
        stq.quantize_rows(torch.zeros((4, k), device="cuda"), torch.ones(k - 1, device="cuda"))
    d_model, d_ff = 256, 256
    tg = torch.zeros(E * 2 * d_ff * O.row_bytes(d_model), dtype=torch.uint8, device="cuda")
    td = torch.zeros(E * d_model * O.row_bytes(d_ff), dtype=torch.uint8, device="cuda")
    pw = torch.ones(2, dtype=torch.float32, device="cuda")
    sg, sd = 2 * d_ff * O.row_bytes(d_model), d_model * O.row_bytes(d_ff)
    with pytest.raises(ValueError, match="out"):
        stq.moe_ffn_decode(tg, sg, td, sd, E, d_model, d_ff, x, pe, pw, 1, out=torch.empty((1, d_model), device="cuda"))
    with pytest.raises(ValueError, match="w_down"):
        stq.moe_ffn_decode(tg, sg, td[:-1], sd, E, d_model, d_ff, x, pe, pw, 1)


def test_empty_calls_succeed_without_work(stq):
    """Zero pairs, zero decode tokens, zero prefill rows and zero rows to
    encode: every entry point returns an empty result without error."""
    k, n, E = 256, 64, 2
    rb = O.row_bytes(k)
    table = torch.zeros(E * n * rb, dtype=torch.uint8, device="cuda")
    x0 = torch.zeros((0, k), dtype=torch.bfloat16, device="cuda")
    pe0 = torch.zeros(0, dtype=torch.int32, device="cuda")
    assert tuple(stq.gemv(table, n * rb, E, n, k, x0, pe0).shape) == (0, n)
    offs = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    assert tuple(stq.grouped_gemm(table, n * rb, E, n, k, x0, offs).shape) == (0, n)
    assert stq.quantize_rows(torch.zeros((0, k), device="cuda")).numel() == 0
    assert tuple(stq.dequantize_rows(table, 0, k).shape) == (0, k)
    d_model = d_ff = 256
    tg = torch.zeros(E * 2 * d_ff * O.row_bytes(d_model), dtype=torch.uint8, device="cuda")
    td = torch.zeros(E * d_model * O.row_bytes(d_ff), dtype=torch.uint8, device="cuda")
    y = stq.moe_ffn_decode(tg, 2 * d_ff * O.row_bytes(d_model), td, d_model * O.row_bytes(d_ff), E, d_model, d_ff,
                           x0, pe0, torch.zeros(0, dtype=torch.float32, device="cuda"), 2)
    assert tuple(y.shape) == (0, d_model)
    torch.cuda.synchronize()


def test_stream_read_probe_runs(stq):
    """The read-rate reference kernel (measurement only) over a small and a
    ragged buffer: it completes and leaves the buffer untouched."""
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")
    before = buf.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stq.stream_read_probe(buf, sink)
    stq.stream_read_probe(buf[: 1000], sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_mfma_and_lds_probes_run(stq):
    """The matrix-core and LDS reference kernels (measurement only) complete
    on a few rounds and touch no memory but their sink: the MFMA sums are
    positive, so its float sink keeps its value; the LDS sink keeps its
    value or takes the fixed tag a fold may match."""
    fs = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    is_ = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    stq.mfma_loop_probe(3, fs)
    stq.mfma_loop_probe(0, fs)
    for mode in (0, 1):
        stq.lds_read_probe(mode, 5, is_)
        stq.lds_read_probe(mode, 0, is_)
    torch.cuda.synchronize()
    assert fs.item() == 7.0
    assert is_.item() in (7, 0x5EED5EED)
