"""GPU parity of the routed-expert FFN for decode (stq_moe_ffn_decode)
against the oracle, with the per-element bound the oracle derives from the
GEMV tolerance; plus, at the benchmark's shapes, linearity in the routing
weights (a property that holds at any size)."""
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


def _tables(seed, n_experts, d_model, d_ff):
    """Oracle-encoded gate/up and down matrices of n_experts experts, as dicts
    for the oracle and as padded device tables for the library."""
    rng = np.random.default_rng(seed)
    gu = {e: O.quantize_rows(rng.normal(0, 0.05, (2 * d_ff, d_model)).astype(np.float32)) for e in range(n_experts)}
    dn = {e: O.quantize_rows(rng.normal(0, 0.05, (d_model, d_ff)).astype(np.float32)) for e in range(n_experts)}

    def table(mats):
        size = mats[0].size
        stride = (size + 15) // 16 * 16
        t = np.zeros(n_experts * stride, dtype=np.uint8)
        for e, m in mats.items():
            t[e * stride: e * stride + size] = m
        return torch.from_numpy(t).cuda(), stride

    return gu, dn, table(gu), table(dn)


def _run(stq, tabs, n_experts, d_model, d_ff, xb, pe, pw, top_k):
    (tg, sg), (td, sd) = tabs
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    y = stq.moe_ffn_decode(tg, sg, td, sd, n_experts, d_model, d_ff, x,
                           torch.from_numpy(pe.astype(np.int32)).cuda(),
                           torch.from_numpy(pw.astype(np.float32)).cuda(), top_k)
    return y.cpu().numpy().astype(np.float64)


def _check(y, gu, dn, d_model, d_ff, xf, pe, pw, top_k):
    ref = O.moe_ffn_decode(gu, dn, d_model, d_ff, xf, pe, pw, top_k)
    bound = O.moe_ffn_tolerance(gu, dn, d_model, d_ff, xf, pe, pw, top_k)
    ok = np.isnan(ref)
    assert np.array_equal(np.isnan(y), ok)
    err = np.abs(y[~ok] - ref[~ok])
    assert np.all(err <= bound[~ok]), float(np.max(err / np.maximum(bound[~ok], 1e-300)))


@pytest.mark.parametrize("n_tokens,top_k,seed", [(4, 2, 11), (1, 1, 12), (3, 4, 13)])
def test_small_layers_match_oracle(stq, n_tokens, top_k, seed):
    E, d_model, d_ff = 5, 512, 256
    gu, dn, tg, td = _tables(seed, E, d_model, d_ff)
    rng = np.random.default_rng(seed + 100)
    pe = np.concatenate([rng.choice(E, top_k, replace=False) for _ in range(n_tokens)]).astype(np.int32)
    pw = S.routing_weights(seed + 200, n_tokens, top_k)
    xb, xf = S.bf16_normal(np.random.default_rng(seed + 300), (n_tokens, d_model))
    y = _run(stq, (tg, td), E, d_model, d_ff, xb, pe, pw, top_k)
    _check(y, gu, dn, d_model, d_ff, xf, pe, pw, top_k)


def test_shared_experts_and_invalid_pair(stq):
    E, d_model, d_ff = 3, 256, 512
    gu, dn, tg, td = _tables(21, E, d_model, d_ff)
    # every token routes to expert 1; token 2 also names expert 9 (invalid)
    pe = np.array([1, 0, 1, 2, 1, 9, 2, 1], dtype=np.int32)
    pw = S.routing_weights(22, 4, 2)
    xb, xf = S.bf16_normal(np.random.default_rng(23), (4, d_model))
    y = _run(stq, (tg, td), E, d_model, d_ff, xb, pe, pw, 2)
    assert np.all(np.isnan(y[2])) and np.all(np.isfinite(np.delete(y, 2, axis=0)))
    _check(y, gu, dn, d_model, d_ff, xf, pe, pw, 2)


@pytest.mark.parametrize("plan", ["2,2", "4,3", "1,4"])
def test_split_outputs_added_by_the_elementwise_passes(stq, monkeypatch, plan):
    """Both projections under forced (k splits, part cap) plans: the SwiGLU
    and combine passes add the split slots themselves ("4,3": up to 12
    slots, some parts empty), with shared experts (one routed to by every
    token) and an invalid pair."""
    monkeypatch.setenv("STQ_GEMV_PLAN", plan)
    E, d_model, d_ff = 4, 1024, 1024
    gu, dn, tg, td = _tables(31, E, d_model, d_ff)
    n_tokens, top_k = 6, 3
    pe = np.array([0, 1, 2, 0, 3, 1, 0, 2, 9, 0, 1, 3, 0, 2, 1, 0, 3, 2], dtype=np.int32)
    pw = S.routing_weights(32, n_tokens, top_k)
    xb, xf = S.bf16_normal(np.random.default_rng(33), (n_tokens, d_model))
    y = _run(stq, (tg, td), E, d_model, d_ff, xb, pe, pw, top_k)
    assert np.all(np.isnan(y[2])) and np.all(np.isfinite(np.delete(y, 2, axis=0)))
    _check(y, gu, dn, d_model, d_ff, xf, pe, pw, top_k)


def test_exact_hand_built_expert(stq):
    # gate rows (-1, 0, +1, +1 | others 0,+,+,+) d=1, up rows (+1, 0, +1, +1 | ...) d=2, down all (0,+,+,+) d=1:
    # with x = e_0, every output is 192 * 2 * silu(-1) up to fp32 rounding of the activation
    d_model = d_ff = 256
    gate = [9] + [0] * 63
    up = [8] + [0] * 63

    def mat(rows, dbits, nb):
        blocks = np.zeros((len(rows), nb, O.BLOCK_BYTES), dtype=np.uint8)
        for r, codes in enumerate(rows):
            blocks[r, :] = O.pack_blocks(np.array([dbits[r]], dtype=np.uint16), np.array(codes, dtype=np.uint8)[None])[0]
        return O.pack_matrix(blocks)

    gu = mat([gate] * d_ff + [up] * d_ff, [0x3C00] * d_ff + [0x4000] * d_ff, 1)
    dn = mat([[0] * 64] * d_model, [0x3C00] * d_model, 1)
    tg = torch.from_numpy(np.pad(gu, (0, (-gu.size) % 16))).cuda()
    td = torch.from_numpy(np.pad(dn, (0, (-dn.size) % 16))).cuda()
    xb = np.zeros((1, d_model), dtype=np.uint16)
    xb[0, 0] = 0x3F80
    y = _run(stq, ((tg, tg.numel()), (td, td.numel())), 1, d_model, d_ff, xb, np.array([0]), np.array([1.0]), 1)
    expect = 192 * 2 * -0.2689414213699951
    assert np.all(np.abs(y - expect) <= 1e-5 * abs(expect))


@pytest.fixture(scope="module")
def full_tables(stq):
    """The benchmark's layer: 256 experts, gate/up 4096 x 7168 and down
    7168 x 2048 in STQ1_0, encoded on the GPU from the seeded fp32 draws."""
    import stq_workloads as W
    q = W.table_imatrix()
    tg, sg = W.encode_table(imatrix=q)
    td, sd = W.encode_down_table()
    torch.cuda.synchronize()
    return (tg, sg), (td, sd), q.cpu().numpy()


def _oracle_layer(experts, qn, down_rows):
    """The oracle's own encodings of the listed experts' gate/up matrices (all
    rows) and of rows `down_rows` of their down matrices, from the raw fp32
    draws (the same draws the GPU tables were encoded from)."""
    import stq_workloads as W
    from _oracle_pool import encode_all
    experts = [int(e) for e in experts]
    gu_raw = [W.expert_weight_rows(W.TABLE_SEED, e, np.arange(W.N_ROWS)) for e in experts]
    gu = dict(zip(experts, encode_all(gu_raw, qn)))
    del gu_raw
    dn = {e: O.quantize_rows(W.expert_weight_rows(W.DOWN_SEED, e, down_rows, n=W.K, k=W.D_FF)) for e in experts}
    return gu, dn


def test_full_size_token_matches_oracle(stq, full_tables):
    """d_model 7168, d_ff 2048, 256-expert tables encoded on the GPU; one bf16
    token routed to 3 experts: the oracle encodes those experts' raw fp32
    draws itself and computes all 7168 outputs."""
    import stq_workloads as W
    tabs_g, tabs_d, qn = full_tables
    experts = [3, 77, 250]
    pe = np.array(experts, dtype=np.int32)
    pw = S.routing_weights(31, 1, 3)
    xb, xf = S.bf16_normal(np.random.default_rng(32), (1, W.K))
    y = _run(stq, (tabs_g, tabs_d), W.N_EXPERTS, W.K, W.D_FF, xb, pe, pw, 3)
    gu, dn = _oracle_layer(experts, qn, np.arange(W.K))
    _check(y, gu, dn, W.K, W.D_FF, xf, pe, pw, 3)


@pytest.mark.parametrize("n_tokens,seed", [(16, 51), (64, 52)])
def test_full_size_batch_matches_oracle(stq, full_tables, n_tokens, seed):
    """A decode batch of 16 or 64 tokens, top-8 of 256 experts, at the
    benchmark's shapes: four sampled tokens' outputs (all eight routed pairs
    each, 96 sampled output rows) against the oracle, which encodes those
    tokens' experts from the raw fp32 draws."""
    import stq_workloads as W
    (tg, sg), (td, sd), qn = full_tables
    pe_t, _, pe, _ = W.decode_pairs(seed, n_tokens)
    pw = S.routing_weights(seed + 1, n_tokens, 8)
    x = S.torch_bf16_normal(seed + 2, (n_tokens, W.K))
    y = stq.moe_ffn_decode(tg, sg, td, sd, W.N_EXPERTS, W.K, W.D_FF, x, pe_t,
                           torch.from_numpy(pw).cuda(), 8).cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    toks = np.unique(np.concatenate([[0, n_tokens - 1], rng.choice(n_tokens, 2, replace=False)]))
    rows = np.unique(np.concatenate([[0, W.K - 1], rng.integers(0, W.K, 94)]))
    sel = (toks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    gu, dn = _oracle_layer(np.unique(pe[sel]), qn, rows)
    xf = x.float().cpu().numpy()[toks]
    ref = O.moe_ffn_decode(gu, dn, W.K, W.D_FF, xf, pe[sel], pw[sel], 8, n_out=len(rows))
    bound = O.moe_ffn_tolerance(gu, dn, W.K, W.D_FF, xf, pe[sel], pw[sel], 8, n_out=len(rows))
    err = np.abs(y[toks][:, rows] - ref)
    assert np.all(np.isfinite(ref)) and np.all(err <= bound), float(np.max(err / bound))


def test_bench_shape_is_linear_in_routing_weights(stq, full_tables):
    """Batch 16, top-8 of 256 experts at full size: y(w) equals the sum over k
    of w_k times y(one-hot k), up to fp32 rounding of the 8-term combine."""
    import stq_workloads as W
    (tg, sg), (td, sd), _ = full_tables
    pe_t, _, pe, _ = W.decode_pairs(41, 16)
    pw = S.routing_weights(42, 16, 8)
    x = S.torch_bf16_normal(43, (16, W.K))
    run = lambda w: stq.moe_ffn_decode(tg, sg, td, sd, W.N_EXPERTS, W.K, W.D_FF, x, pe_t,
                                       torch.from_numpy(w).cuda(), 8).cpu().numpy().astype(np.float64)
    y = run(pw)
    parts = []
    for k in range(8):
        w = np.zeros_like(pw)
        w[k::8] = 1.0
        parts.append(run(w))
    z = np.stack(parts)                                   # [8, T, d_model]: expert outputs z_k
    w8 = pw.reshape(16, 8).T[:, :, None].astype(np.float64)
    lin = (w8 * z).sum(axis=0)
    mag = (np.abs(w8) * np.abs(z)).sum(axis=0)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y - lin) <= 8 * 2.0 ** -23 * mag + 1e-30)
